// MFMA issue-rate microbenchmark (libufp4_probe.so, a measurement aid for
// the bench; not part of the libufp4 C ABI).  Times a grid of waves that each
// issue `reps` x 4 independent MFMAs of one kind, so the returned rate is the
// instruction's sustained peak on this GPU: the denominator for the GEMM's
// "fraction of the peak of the MFMA instruction used", and the measurement
// behind the choice of instruction.
//   kind 0  v_mfma_f32_32x32x16_fp8_fp8          (the GEMM's instruction)
//   kind 1  v_mfma_i32_32x32x16_i8               (int8 alternative)
//   kind 2  v_mfma_scale_f32_32x32x64_f8f6f4 fp8 (scaled, K = 64)
//   kind 3  v_mfma_scale_f32_32x32x64_f8f6f4 fp6 E2M3
//   kind 4  v_mfma_scale_f32_32x32x64_f8f6f4 fp4 E2M1
//   kind 5  v_mfma_f32_32x32x16_bf16              (context)
//   kind 6  v_mfma_f32_32x32x1_2b_f32             (the GEMM's scale products)
//   kind 7  v_mfma_f32_32x32x8_bf16               (what a split-bf16 scale product would use)
// Operands are arbitrary register contents (results are discarded); no
// memory is touched except one guarded store per workgroup.
//
// A second loop times the GEMM's per-block instruction mix of one wave (two
// FP8 MFMAs, one FP32 outer-product MFMA, 32 independent v_fmac_f32) and its
// parts on their own, to show how far matrix-core and vector work overlap on
// one SIMD.
//
// A third loop puts the matrix-core and the vector work in different waves
// of one SIMD, to show which MFMA kinds the other waves' vector instructions
// can overlap.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x32 __attribute__((ext_vector_type(32)));

template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop(float *out, int reps) {
  f32x16 acc[4] = {};
  i32x16 iacc[4] = {};
  f32x32 wide[4] = {};
  const int t = threadIdx.x;
  const float fa = 1.0f + 0.001f * (float)t, fb = 1.0f - 0.001f * (float)t;
  const long a = 0x3C3C3C3C3C3C3C3Cll + t, b = 0x3838383838383838ll - t;
  i32x8 a8, b8;
  bf16x8 ab;
  s16x4 h4;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a8[i] = 0x22222222 + t + i;
    b8[i] = 0x11111111 - t + i;
    ab[i] = (__bf16)(1.0f + 0.001f * (float)(t + i));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) h4[i] = (short)(0x3F80 + t + i);
  for (int r = 0; r < reps; ++r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (KIND == 0) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, acc[j], 0, 0, 0);
      if (KIND == 1) iacc[j] = __builtin_amdgcn_mfma_i32_32x32x16_i8(a, b, iacc[j], 0, 0, 0);
      if (KIND == 2)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[j], 0, 0, 0, 127, 0,
                                                                 127);
      if (KIND == 3)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[j], 2, 2, 0, 127, 0,
                                                                 127);
      if (KIND == 4)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[j], 4, 4, 0, 127, 0,
                                                                 127);
      if (KIND == 5) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, ab, acc[j], 0, 0, 0);
      if (KIND == 7) acc[j] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(h4, h4, acc[j], 0, 0, 0);
      if (KIND == 6) {
        const f32x32 o = __builtin_amdgcn_mfma_f32_32x32x1f32(fa, fb, wide[j], 1, 0, 0);
        wide[j] = o;
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r] + (float)iacc[j][r] + wide[j][r] + wide[j][16 + r];
  if (s == 1234.5f) out[blockIdx.x] = s;   // keeps the loop; practically never taken
}

// One iteration = one K-block of a wave's 32 x 64 GEMM tile: MODE 0 the whole
// mix, 1 the 32 FMAs only, 2 the three MFMAs only.  The FMAs are independent
// of the MFMAs (and of each other in groups of 16), as in the GEMM where a
// block's FMAs consume the previous MFMAs' results.
#define UFP4_FMAC(i) "v_fmac_f32 %" #i ", %16, %17\n"
#define UFP4_FMAC16                                                                          \
  UFP4_FMAC(0) UFP4_FMAC(1) UFP4_FMAC(2) UFP4_FMAC(3) UFP4_FMAC(4) UFP4_FMAC(5) UFP4_FMAC(6) \
  UFP4_FMAC(7) UFP4_FMAC(8) UFP4_FMAC(9) UFP4_FMAC(10) UFP4_FMAC(11) UFP4_FMAC(12)           \
  UFP4_FMAC(13) UFP4_FMAC(14) UFP4_FMAC(15)
template <int MODE>
__global__ __launch_bounds__(256) void mix_loop(float *out, int reps) {
  const int t = threadIdx.x;
  const long a = 0x3C3C3C3C3C3C3C3Cll + t, b = 0x3838383838383838ll - t;
  const float fa = 1.0f + 0.001f * (float)t, fb = 1.0f - 0.001f * (float)t;
  const float m = 1.0001f + 1e-9f * (float)t, c = 0.5f;
  f32x16 p0 = {}, p1 = {};
  f32x32 sc = {};
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = (float)(t + i);
  for (int r = 0; r < reps; ++r) {
    if (MODE != 1) {
      sc = __builtin_amdgcn_mfma_f32_32x32x1f32(fa, fb, sc, 1, 0, 0);
      p0 = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, p0, 0, 0, 0);
      p1 = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, p1, 0, 0, 0);
    }
    if (MODE != 2) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
        asm volatile(UFP4_FMAC16
                     : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                       "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]),
                       "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])
                     : "v"(m), "v"(c));
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += v[i] + p0[i] + p1[i] + sc[i] + sc[16 + i];
  if (s == 1234.5f) out[blockIdx.x] = s;
}

// Cross-wave overlap: 512-thread workgroups, so SIMD s holds waves s and s+4
// of each workgroup.  Waves 0-3 issue matrix-core work (ROLES bit 0), waves
// 4-7 issue 32 independent v_fmac_f32 per iteration (bit 1); with one bit
// set the other half of the waves exits at once.  KIND 0: two FP8 MFMAs
// (v_mfma_f32_32x32x16_fp8_fp8), 1: one FP32 outer-product MFMA
// (v_mfma_f32_32x32x1_2b_f32), 2: two v_mfma_f32_32x32x8_bf16 -- each about
// 64 matrix-core cycles per iteration.
template <int KIND, int ROLES>
__global__ __launch_bounds__(512) void overlap_loop(float *out, int reps) {
  const int t = threadIdx.x;
  const int w = t >> 6;
  const long a = 0x3C3C3C3C3C3C3C3Cll + t, b = 0x3838383838383838ll - t;
  const float fa = 1.0f + 0.001f * (float)t, fb = 1.0f - 0.001f * (float)t;
  const float m = 1.0001f + 1e-9f * (float)t, c = 0.5f;
  s16x4 h4;
#pragma unroll
  for (int i = 0; i < 4; ++i) h4[i] = (short)(0x3F80 + t + i);
  f32x16 p0 = {}, p1 = {};
  f32x32 sc = {};
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = (float)(t + i);
  if (w < 4 && (ROLES & 1)) {
    for (int r = 0; r < reps; ++r) {
      if (KIND == 0) {
        p0 = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, p0, 0, 0, 0);
        p1 = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, p1, 0, 0, 0);
      } else if (KIND == 1) {
        sc = __builtin_amdgcn_mfma_f32_32x32x1f32(fa, fb, sc, 1, 0, 0);
      } else {
        p0 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(h4, h4, p0, 0, 0, 0);
        p1 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(h4, h4, p1, 0, 0, 0);
      }
    }
  }
  if (w >= 4 && (ROLES & 2)) {
    for (int r = 0; r < reps; ++r) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
        asm volatile(UFP4_FMAC16
                     : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                       "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]),
                       "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])
                     : "v"(m), "v"(c));
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += v[i] + p0[i] + p1[i] + sc[i] + sc[16 + i];
  if (s == 1234.5f) out[blockIdx.x] = s;
}

template <int KIND, int ROLES>
hipError_t launch_overlap(float *out, int wgs, int reps) {
  hipLaunchKernelGGL((overlap_loop<KIND, ROLES>), dim3(wgs), dim3(512), 0, 0, out, reps);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch(float *out, int wgs, int reps) {
  hipLaunchKernelGGL(mfma_loop<KIND>, dim3(wgs), dim3(256), 0, 0, out, reps);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mix(float *out, int wgs, int reps) {
  hipLaunchKernelGGL(mix_loop<MODE>, dim3(wgs), dim3(256), 0, 0, out, reps);
  return hipGetLastError();
}

// Times launcher(out) twice (the first pass warms up) and returns the second
// pass in milliseconds, or a negative value on a HIP error.
template <typename F>
double time_ms(F &&launcher, int wgs) {
  float *out = nullptr;
  if (hipMalloc(&out, sizeof(float) * (size_t)wgs) != hipSuccess) return -2.0;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    (void)hipFree(out);
    return -2.0;
  }
  hipError_t err = hipSuccess;
  float ms = 0.0f;
  for (int pass = 0; pass < 2 && err == hipSuccess; ++pass) {
    (void)hipEventRecord(e0, 0);
    err = launcher(out);
    (void)hipEventRecord(e1, 0);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipFree(out);
  if (err != hipSuccess || ms <= 0.0f) return -3.0;
  return (double)ms;
}

}  // namespace

extern "C" {

// FLOP of one instruction of `kind` (2 * M * N * K), 0 for an unknown kind.
double ufp4_probe_mfma_flops(int kind) {
  switch (kind) {
    case 0: case 1: case 5: return 2.0 * 32 * 32 * 16;
    case 2: case 3: case 4: return 2.0 * 32 * 32 * 64;
    case 6: return 2.0 * 32 * 32 * 1 * 2;
    case 7: return 2.0 * 32 * 32 * 8;
  }
  return 0.0;
}

// Runs the loop of `kind` on `wgs` workgroups of 256 threads (4 waves) with
// `reps` iterations, on the null stream, and returns the sustained rate in
// TFLOP/s (TOP/s for int8), or a negative value on a bad argument or a HIP
// error.  Synchronises the device.
double ufp4_probe_mfma_tflops(int kind, int wgs, int reps) {
  if (kind < 0 || kind > 7 || wgs < 1 || wgs > (1 << 20) || reps < 1) return -1.0;
  const double ms = time_ms(
      [&](float *out) {
        switch (kind) {
          case 0: return launch<0>(out, wgs, reps);
          case 1: return launch<1>(out, wgs, reps);
          case 2: return launch<2>(out, wgs, reps);
          case 3: return launch<3>(out, wgs, reps);
          case 4: return launch<4>(out, wgs, reps);
          case 5: return launch<5>(out, wgs, reps);
          case 6: return launch<6>(out, wgs, reps);
          default: return launch<7>(out, wgs, reps);
        }
      },
      wgs);
  if (ms <= 0.0) return ms;
  const double instrs = (double)wgs * 4.0 /* waves */ * 4.0 /* per iteration */ * (double)reps;
  return instrs * ufp4_probe_mfma_flops(kind) / (ms * 1e-3) / 1e12;
}

// Runs the GEMM-mix loop (mode 0: 3 MFMAs + 32 FMAs per iteration, 1: the
// FMAs only, 2: the MFMAs only) on `wgs` workgroups of 4 waves and returns the
// elapsed milliseconds, or a negative value on a bad argument or a HIP error.
// Synchronises the device.
double ufp4_probe_mix_ms(int mode, int wgs, int reps) {
  if (mode < 0 || mode > 2 || wgs < 1 || wgs > (1 << 20) || reps < 1) return -1.0;
  return time_ms(
      [&](float *out) {
        switch (mode) {
          case 0: return launch_mix<0>(out, wgs, reps);
          case 1: return launch_mix<1>(out, wgs, reps);
          default: return launch_mix<2>(out, wgs, reps);
        }
      },
      wgs);
}

// Runs the cross-wave overlap loop (kind 0 FP8, 1 FP32 outer product, 2 bf16
// K = 8; roles 1 = matrix-core waves only, 2 = FMA waves only, 3 = both) on
// `wgs` workgroups of 8 waves and returns the elapsed milliseconds, or a
// negative value on a bad argument or a HIP error.  Synchronises the device.
double ufp4_probe_overlap_ms(int kind, int roles, int wgs, int reps) {
  if (kind < 0 || kind > 2 || roles < 1 || roles > 3 || wgs < 1 || wgs > (1 << 20) || reps < 1)
    return -1.0;
  return time_ms(
      [&](float *out) {
#define UFP4_OV(K)                                              \
  if (kind == K) {                                              \
    if (roles == 1) return launch_overlap<K, 1>(out, wgs, reps); \
    if (roles == 2) return launch_overlap<K, 2>(out, wgs, reps); \
    return launch_overlap<K, 3>(out, wgs, reps);                 \
  }
        UFP4_OV(0)
        UFP4_OV(1)
        UFP4_OV(2)
#undef UFP4_OV
        return hipErrorInvalidValue;
      },
      wgs);
}

}  // extern "C"
