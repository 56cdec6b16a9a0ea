// Block-scaled 4-bit GEMM, C = A_hat * B_hat^T, on CDNA4 MFMA (gfx950).
//
// Method: the low-precision training GEMMs consume the rotated quantized
// operands and contract along the dimension they were quantized and rotated
// along ("Rethinking Shrinkage Bias in LLM FP4 Pretraining", arXiv
// 2606.20381, paperlayer.ai summary, section 2 "Random Hadamard transforms").
// With codes q and FP32 block scales s per 16 elements:
//   C[m,n] = (1/g^2) * sum_kb sa[m,kb] * sb[n,kb] * P_kb[m,n],
//   P_kb[m,n] = sum_{k in kb} qa[m,k] * qb[n,k]   (an exact small integer).
//
// Design for gfx950: every grid level is an exact FP8 E4M3 value (uniform:
// 0..7; E2M1 doubled: 0,1,2,3,4,6,8,12), so one v_mfma_f32_32x32x16_fp8_fp8
// per 16-element block yields P_kb exactly in FP32 (|P| <= 16*144).  The
// per-block rescale is an FP32 multiply and fused multiply-add per output on
// the vector ALU, which is the bound of this kernel (two VALU operations per
// 16 MACs); the MFMA of the next tile overlaps it.  Nibbles are expanded to
// FP8 once per workgroup while staging into LDS (v_perm_b32 look-up), so the
// waves only read ready operands.
//
// Tiling: 256 threads = 4 waves, 128 x 128 output tile, each wave 32 rows x
// 128 columns = four 32x32 MFMA tiles sharing one A fragment and one set of
// 16 row scales per block.  K advances 64 (4 blocks) per LDS stage.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ufp4_device.h"
#include "ufp4_kernels.h"

namespace ufp4 {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kStageBlocks = 4;                 // 16-element blocks per stage
constexpr int kRowBytes = kStageBlocks * 16 + 8; // fp8 bytes per LDS row (+8 pad)
constexpr int kMaxGemmGroups = 1024;

// 8 nibbles -> 8 FP8 E4M3 bytes.  Output byte order [n0 n2 n4 n6 | n1 n3 n5
// n7]; A and B use the same order so products still pair up.
template <int GRID>
__device__ __forceinline__ uint2 nib8_to_fp8(uint32_t w) {
  constexpr uint32_t lut_lo = 0x44403800u;  // 0, 1, 2, 3
  constexpr uint32_t lut_hi = (GRID == kGridUniform) ? 0x4E4C4A48u   // 4, 5, 6, 7
                                                     : 0x54504C48u;  // 4, 6, 8, 12
  const uint32_t me = w & 0x07070707u;
  const uint32_t mo = (w >> 4) & 0x07070707u;
  const uint32_t fe = __builtin_amdgcn_perm(lut_hi, lut_lo, me) | ((w << 4) & 0x80808080u);
  const uint32_t fo = __builtin_amdgcn_perm(lut_hi, lut_lo, mo) | (w & 0x80808080u);
  return make_uint2(fe, fo);
}

struct TileJob {
  int64_t a_row0, a_row_end;   // A rows of this tile [a_row0, a_row_end)
  int64_t b_row0, b_row_end;   // B rows
  int64_t kb0, kb1;            // block range [kb0, kb1)
  float *c;                    // C element (0,0) of the tile
  int64_t ldc;
};

// Stage one K slice of the A or B tile: 128 rows x 4 blocks.  Thread t takes
// (row, block) items t and t + 256.
template <int GRID>
__device__ __forceinline__ void stage_operand(const uint8_t *__restrict__ codes,
                                              const float *__restrict__ scales, int64_t kpad,
                                              int64_t row0, int64_t row_end, int64_t kb,
                                              int64_t kb_end, uint8_t *s_q, float *s_s) {
  const int64_t kblocks = kpad / 16;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int i = threadIdx.x + 256 * it;
    const int r = i >> 2;
    const int b = i & 3;
    const int64_t row = row0 + r;
    const int64_t blk = kb + b;
    uint2 w = make_uint2(0u, 0u);
    float s = 0.0f;
    if (row < row_end && blk < kb_end) {
      w = *reinterpret_cast<const uint2 *>(codes + row * (kpad / 2) + blk * 8);
      s = scales[row * kblocks + blk];
    }
    const uint2 lo = nib8_to_fp8<GRID>(w.x);
    const uint2 hi = nib8_to_fp8<GRID>(w.y);
    uint2 *dst = reinterpret_cast<uint2 *>(s_q + r * kRowBytes + b * 16);
    dst[0] = lo;
    dst[1] = hi;
    s_s[b * kBM + r] = s;
  }
}

template <int GRID>
__device__ __forceinline__ void gemm_tile(const GemmArgs &g, const TileJob &job, uint8_t *s_a,
                                          uint8_t *s_b, float *s_sa, float *s_sb) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  floatx16 acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[nt][r] = 0.0f;
  const floatx16 zero = acc[0];

  for (int64_t kb = job.kb0; kb < job.kb1; kb += kStageBlocks) {
    stage_operand<GRID>(g.a_codes, g.a_scales, g.kpad, job.a_row0, job.a_row_end, kb, job.kb1,
                        s_a, s_sa);
    stage_operand<GRID>(g.b_codes, g.b_scales, g.kpad, job.b_row0, job.b_row_end, kb, job.kb1,
                        s_b, s_sb);
    __syncthreads();
#pragma unroll 1
    for (int b = 0; b < kStageBlocks; ++b) {
      const long af = *reinterpret_cast<const long *>(s_a + (wave * 32 + l32) * kRowBytes +
                                                      b * 16 + 8 * half);
      floatx16 p[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const long bf = *reinterpret_cast<const long *>(s_b + (nt * 32 + l32) * kRowBytes +
                                                        b * 16 + 8 * half);
        p[nt] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(af, bf, zero, 0, 0, 0);
      }
      float sa[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 v =
            *reinterpret_cast<const float4 *>(s_sa + b * kBM + wave * 32 + 8 * j + 4 * half);
        sa[4 * j + 0] = v.x;
        sa[4 * j + 1] = v.y;
        sa[4 * j + 2] = v.z;
        sa[4 * j + 3] = v.w;
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float sb = s_sb[b * kBN + nt * 32 + l32];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nt][r] = fmaf(sa[r] * sb, p[nt][r], acc[nt][r]);
      }
    }
    __syncthreads();
  }
  constexpr float inv_g2 = (GRID == kGridUniform) ? (1.0f / 49.0f) : (1.0f / 144.0f);
  const int64_t m_rows = job.a_row_end - job.a_row0;
  const int64_t n_cols = job.b_row_end - job.b_row0;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int n = nt * 32 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = wave * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (m < m_rows && n < n_cols) job.c[(int64_t)m * job.ldc + n] = acc[nt][r] * inv_g2;
    }
  }
}

__device__ __forceinline__ int64_t clampv(int64_t v, int64_t n) {
  return v < 0 ? 0 : (v > n ? n : v);
}

// Group tables for the grouped modes: s_off = row offsets, s_pre = prefix of
// per-group tile counts (mode 1) or padded K offsets (mode 2).
__device__ void load_gemm_groups(const GemmArgs &g, int64_t *s_off, int64_t *s_pre,
                                 int64_t *s_scan) {
  const int tid = threadIdx.x;
  const int ng = g.n_groups;
  const int per = (ng + 255) / 256;
  const int g0 = tid * per;
  const int64_t tiles_n = (g.N + kBN - 1) / kBN;
  // Offsets are clamped to [0, limit] (A rows in mode 1, padded K in mode 2
  // is bounded separately) so no access leaves the operands whatever the
  // device array holds; a decreasing pair is an empty group.
  const int64_t limit = (g.mode == 1) ? g.M : INT64_MAX / 4;
  int64_t local = 0;
  for (int e = g0; e < g0 + per && e < ng; ++e) {
    const int64_t a = clampv(g.goff[e], limit), b = clampv(g.goff[e + 1], limit);
    s_off[e] = a;
    const int64_t cnt = b > a ? b - a : 0;
    local += (g.mode == 1) ? ((cnt + kBM - 1) / kBM) * tiles_n : (cnt + 15) / 16 * 16;
  }
  if (tid == 0) s_off[ng] = clampv(g.goff[ng], limit);
  s_scan[tid] = local;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const int64_t add = tid >= d ? s_scan[tid - d] : 0;
    __syncthreads();
    s_scan[tid] += add;
    __syncthreads();
  }
  int64_t run = tid ? s_scan[tid - 1] : 0;
  for (int e = g0; e < g0 + per && e < ng; ++e) {
    s_pre[e] = run;
    int64_t cnt = s_off[e + 1] - s_off[e];
    cnt = cnt > 0 ? cnt : 0;
    run += (g.mode == 1) ? ((cnt + kBM - 1) / kBM) * tiles_n : (cnt + 15) / 16 * 16;
  }
  if (tid == 255) s_pre[ng] = s_scan[255];
  __syncthreads();
}

template <int GRID>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t s_a[kBM * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[kBN * kRowBytes];
  __shared__ __attribute__((aligned(16))) float s_sa[kStageBlocks * kBM];
  __shared__ __attribute__((aligned(16))) float s_sb[kStageBlocks * kBN];
  __shared__ int64_t s_off[kMaxGemmGroups + 1];
  __shared__ int64_t s_pre[kMaxGemmGroups + 1];
  __shared__ int64_t s_scan[256];

  const int64_t tiles_m = (g.M + kBM - 1) / kBM;
  const int64_t tiles_n = (g.N + kBN - 1) / kBN;
  const int64_t kblocks = g.kpad / 16;
  if (g.mode != 0) load_gemm_groups(g, s_off, s_pre, s_scan);

  int64_t total;
  if (g.mode == 0) total = tiles_m * tiles_n;
  else if (g.mode == 1) total = s_pre[g.n_groups];
  else total = (int64_t)g.n_groups * tiles_m * tiles_n;

  for (int64_t t = blockIdx.x; t < total; t += gridDim.x) {
    TileJob job;
    if (g.mode == 0) {
      const int64_t tm = t / tiles_n, tn = t - tm * tiles_n;
      job.a_row0 = tm * kBM;
      job.a_row_end = min(job.a_row0 + kBM, g.M);
      job.b_row0 = tn * kBN;
      job.b_row_end = min(job.b_row0 + kBN, g.N);
      job.kb0 = 0;
      job.kb1 = kblocks;
      job.c = g.c + job.a_row0 * g.ldc + job.b_row0;
      job.ldc = g.ldc;
    } else if (g.mode == 1) {
      int lo = 0, hi = g.n_groups;   // largest e with s_pre[e] <= t
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pre[mid] <= t) lo = mid; else hi = mid;
      }
      const int e = lo;
      const int64_t local = t - s_pre[e];
      const int64_t tm = local / tiles_n, tn = local - tm * tiles_n;
      job.a_row0 = s_off[e] + tm * kBM;
      job.a_row_end = min(job.a_row0 + kBM, s_off[e + 1]);
      job.b_row0 = (int64_t)e * g.N + tn * kBN;
      job.b_row_end = min(job.b_row0 + kBN, (int64_t)(e + 1) * g.N);
      job.kb0 = 0;
      job.kb1 = kblocks;
      job.c = g.c + job.a_row0 * g.ldc + tn * kBN;
      job.ldc = g.ldc;
    } else {
      const int64_t per_group = tiles_m * tiles_n;
      const int64_t e = t / per_group;
      const int64_t local = t - e * per_group;
      const int64_t tm = local / tiles_n, tn = local - tm * tiles_n;
      job.a_row0 = tm * kBM;
      job.a_row_end = min(job.a_row0 + kBM, g.M);
      job.b_row0 = tn * kBN;
      job.b_row_end = min(job.b_row0 + kBN, g.N);
      job.kb0 = min(s_pre[e] / 16, kblocks);
      job.kb1 = min(s_pre[e + 1] / 16, kblocks);
      job.c = g.c + e * g.M * g.ldc + job.a_row0 * g.ldc + job.b_row0;
      job.ldc = g.ldc;
    }
    gemm_tile<GRID>(g, job, s_a, s_b, s_sa, s_sb);
  }
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t st) {
  const int64_t tiles_m = (g.M + kBM - 1) / kBM;
  const int64_t tiles_n = (g.N + kBN - 1) / kBN;
  int64_t total;
  if (g.mode == 0) total = tiles_m * tiles_n;
  else if (g.mode == 1) total = (tiles_m + g.n_groups) * tiles_n;   // upper bound
  else total = (int64_t)g.n_groups * tiles_m * tiles_n;
  int64_t blocks = total < 1 ? 1 : total;
  if (blocks > 65536) blocks = 65536;
  if (g.grid == kGridUniform)
    hipLaunchKernelGGL((gemm_kernel<kGridUniform>), dim3((unsigned)blocks), dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_kernel<kGridE2M1>), dim3((unsigned)blocks), dim3(256), 0, st, g);
  return hipGetLastError();
}

}  // namespace ufp4
