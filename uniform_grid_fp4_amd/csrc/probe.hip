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
// Operands are arbitrary register contents (results are discarded); no
// memory is touched except one guarded store per workgroup.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop(float *out, int reps) {
  f32x16 acc[4] = {};
  i32x16 iacc[4] = {};
  const int t = threadIdx.x;
  const long a = 0x3C3C3C3C3C3C3C3Cll + t, b = 0x3838383838383838ll - t;
  i32x8 a8, b8;
  bf16x8 ab;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a8[i] = 0x22222222 + t + i;
    b8[i] = 0x11111111 - t + i;
    ab[i] = (__bf16)(1.0f + 0.001f * (float)(t + i));
  }
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
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r] + (float)iacc[j][r];
  if (s == 1234.5f) out[blockIdx.x] = s;   // keeps the loop; practically never taken
}

template <int KIND>
hipError_t launch(float *out, int wgs, int reps) {
  hipLaunchKernelGGL(mfma_loop<KIND>, dim3(wgs), dim3(256), 0, 0, out, reps);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// FLOP of one instruction of `kind` (2 * M * N * K), 0 for an unknown kind.
double ufp4_probe_mfma_flops(int kind) {
  switch (kind) {
    case 0: case 1: case 5: return 2.0 * 32 * 32 * 16;
    case 2: case 3: case 4: return 2.0 * 32 * 32 * 64;
  }
  return 0.0;
}

// Runs the loop of `kind` on `wgs` workgroups of 256 threads (4 waves) with
// `reps` iterations, on the null stream, and returns the sustained rate in
// TFLOP/s (TOP/s for int8), or a negative value on a bad argument or a HIP
// error.  Synchronises the device.
double ufp4_probe_mfma_tflops(int kind, int wgs, int reps) {
  if (kind < 0 || kind > 5 || wgs < 1 || wgs > (1 << 20) || reps < 1) return -1.0;
  float *out = nullptr;
  if (hipMalloc(&out, sizeof(float) * (size_t)wgs) != hipSuccess) return -2.0;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    (void)hipFree(out);
    return -2.0;
  }
  hipError_t err = hipSuccess;
  float ms = 0.0f;
  for (int pass = 0; pass < 2 && err == hipSuccess; ++pass) {   // pass 0 warms up
    (void)hipEventRecord(e0, 0);
    switch (kind) {
      case 0: err = launch<0>(out, wgs, reps); break;
      case 1: err = launch<1>(out, wgs, reps); break;
      case 2: err = launch<2>(out, wgs, reps); break;
      case 3: err = launch<3>(out, wgs, reps); break;
      case 4: err = launch<4>(out, wgs, reps); break;
      default: err = launch<5>(out, wgs, reps); break;
    }
    (void)hipEventRecord(e1, 0);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipFree(out);
  if (err != hipSuccess || ms <= 0.0f) return -3.0;
  const double instrs = (double)wgs * 4.0 /* waves */ * 4.0 /* per iteration */ * (double)reps;
  return instrs * ufp4_probe_mfma_flops(kind) / (ms * 1e-3) / 1e12;
}

}  // extern "C"
