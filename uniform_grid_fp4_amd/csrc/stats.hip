// Quantization diagnostics on the GPU: the tensor and GEMM-output
// measurements of "Rethinking Shrinkage Bias in LLM FP4 Pretraining"
// (paperlayer.ai summary, section 3.2, section 5 Q1 and appendix A: SQNR and
// its change under RHT, bucket utilization; gist.science technical summary:
// the attenuation factor alpha of a GEMM; dreamwings.cn post, "RHT turning
// point": the quantization underflow ratio).  The kernels return raw FP64
// sums and integer counts; SQNR, alpha, delta_mag, the underflow ratio and
// the bucket utilization are formed from them on the host.
//
// Pairing: every logical element x (padding excluded) with its dequantized
// value xhat in x's own domain -- the dequantized block goes back through
// (1/4) D H16 in FP64 when the quantization used the RHT.  Underflow counts
// elements whose pre-rounding value y (FP32, the quantizer's own butterfly)
// is nonzero while their magnitude index is 0.
//
// Determinism: a fixed-size grid (a function of the shape only) writes one
// partial per workgroup to the caller's workspace; one workgroup then sums
// the partials in a fixed order.  No atomics.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "ufp4_device.h"
#include "ufp4_kernels.h"

namespace ufp4 {

constexpr int kStatsThreads = 256;

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Per-thread accumulators -> one StatsPartial per workgroup (fixed order:
// butterfly within each wave, then waves 0..3 in order).
struct Acc {
  double s[5];
  uint32_t n[3];
  uint32_t h[16];
};

__device__ void block_reduce_store(Acc &a, StatsPartial *dst) {
  __shared__ double s_s[4][5];
  __shared__ uint32_t s_n[4][19];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 5; ++i) a.s[i] = wave_sum(a.s[i]);
#pragma unroll
  for (int i = 0; i < 3; ++i) a.n[i] = wave_sum(a.n[i]);
#pragma unroll
  for (int i = 0; i < 16; ++i) a.h[i] = wave_sum(a.h[i]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < 5; ++i) s_s[wave][i] = a.s[i];
#pragma unroll
    for (int i = 0; i < 3; ++i) s_n[wave][i] = a.n[i];
#pragma unroll
    for (int i = 0; i < 16; ++i) s_n[wave][3 + i] = a.h[i];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    StatsPartial p;
    for (int i = 0; i < 5; ++i) p.sum[i] = ((s_s[0][i] + s_s[1][i]) + s_s[2][i]) + s_s[3][i];
    uint64_t c[19];
    for (int i = 0; i < 19; ++i)
      c[i] = (uint64_t)s_n[0][i] + s_n[1][i] + s_n[2][i] + s_n[3][i];
    p.n_elems = c[0];
    p.n_nonzero = c[1];
    p.n_underflow = c[2];
    for (int i = 0; i < 16; ++i) p.hist[i] = c[3 + i];
    *dst = p;
  }
}

template <int GRID>
__global__ __launch_bounds__(kStatsThreads) void quant_stats_kernel(const StatsArgs a,
                                                                    StatsPartial *partials) {
  Acc acc;
#pragma unroll
  for (int i = 0; i < 5; ++i) acc.s[i] = 0.0;
#pragma unroll
  for (int i = 0; i < 3; ++i) acc.n[i] = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc.h[i] = 0;
  constexpr double g = (double)grid_g<GRID>();
  const int64_t kblocks = a.kpad / 16;
  const int64_t nblk = a.rows * kblocks;
  const int64_t stride = (int64_t)gridDim.x * kStatsThreads;
  for (int64_t b = (int64_t)blockIdx.x * kStatsThreads + threadIdx.x; b < nblk; b += stride) {
    // lanes walk the input's contiguous dimension: blocks of a row for the
    // row-wise layout, output rows (= input columns) for the transposed one
    int64_t r, kb;
    if (a.axis == 0) {
      r = b / kblocks;
      kb = b - r * kblocks;
    } else {
      kb = b / a.rows;
      r = b - kb * a.rows;
    }
    const uint2 c = *reinterpret_cast<const uint2 *>(a.codes + (r * kblocks + kb) * 8);
    const double sc = (double)a.scales[r * kblocks + kb];
    float xf[16], y[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t k = kb * 16 + j;
      uint32_t h = 0;
      if (k < a.kvalid) h = a.x[a.axis == 0 ? r * a.ld + k : k * a.ld + r];
      xf[j] = __uint_as_float(h << 16);
      y[j] = a.rht ? __uint_as_float((h << 16) ^ sign_bit(a.sign_mask, j)) : xf[j];
    }
    if (a.rht) fwht16(y);
    double d[16];
    uint32_t nib[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t w = j < 8 ? c.x : c.y;
      nib[j] = (w >> (4 * (j & 7))) & 0xFu;
      const uint32_t mi = nib[j] & 7u;
      double lv;
      if (GRID == kGridUniform) {
        lv = (double)mi;
      } else {
        lv = mi < 4 ? 0.5 * (double)mi : (mi == 4 ? 2.0 : (mi == 5 ? 3.0 : (mi == 6 ? 4.0 : 6.0)));
      }
      if (nib[j] & 8u) lv = -lv;
      d[j] = lv * sc / g;
    }
    if (a.rht) {
#pragma unroll
      for (int hs = 1; hs < 16; hs <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if ((i & hs) == 0) {
            const double u = d[i], v = d[i + hs];
            d[i] = u + v;
            d[i + hs] = u - v;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        d[j] *= 0.25;
        if ((a.sign_mask >> j) & 1u) d[j] = -d[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (kb * 16 + j < a.kvalid) {
        const double xv = (double)xf[j];
        const double e = d[j] - xv;
        acc.s[0] += xv * xv;
        acc.s[1] += e * e;
        acc.s[2] += xv * d[j];
        acc.s[3] += fabs(xv);
        acc.s[4] += fabs(d[j]);
        acc.n[0] += 1;
        if (y[j] != 0.0f) {
          acc.n[1] += 1;
          acc.n[2] += (nib[j] & 7u) == 0;
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) acc.h[v] += nib[j] == (uint32_t)v;
      }
    }
  }
  block_reduce_store(acc, partials + blockIdx.x);
}

__global__ __launch_bounds__(kStatsThreads) void output_stats_kernel(
    const float *__restrict__ ref, int64_t ld_ref, const float *__restrict__ test,
    int64_t ld_test, int64_t rows, int64_t cols, StatsPartial *partials) {
  Acc acc;
#pragma unroll
  for (int i = 0; i < 5; ++i) acc.s[i] = 0.0;
#pragma unroll
  for (int i = 0; i < 3; ++i) acc.n[i] = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc.h[i] = 0;
  const int64_t n = rows * cols;
  const int64_t stride = (int64_t)gridDim.x * kStatsThreads;
  for (int64_t e = (int64_t)blockIdx.x * kStatsThreads + threadIdx.x; e < n; e += stride) {
    const int64_t r = e / cols, c = e - r * cols;
    const double rv = (double)ref[r * ld_ref + c];
    const double tv = (double)test[r * ld_test + c];
    const double d = tv - rv;
    acc.s[0] += rv * rv;
    acc.s[1] += d * d;
    acc.s[2] += rv * tv;
    acc.s[3] += fabs(rv);
    acc.s[4] += fabs(tv);
    acc.n[0] += 1;
  }
  block_reduce_store(acc, partials + blockIdx.x);
}

// One workgroup: thread t sums partials t, t + 256, ... in order, then
// thread 0 sums the 256 per-thread results in order.
__global__ __launch_bounds__(kStatsThreads) void stats_final_kernel(const StatsPartial *partials,
                                                                    int n_partials,
                                                                    StatsPartial *out) {
  __shared__ StatsPartial s_p[kStatsThreads];
  StatsPartial p{};
  for (int i = threadIdx.x; i < n_partials; i += kStatsThreads) {
    const StatsPartial &q = partials[i];
    for (int f = 0; f < 5; ++f) p.sum[f] += q.sum[f];
    p.n_elems += q.n_elems;
    p.n_nonzero += q.n_nonzero;
    p.n_underflow += q.n_underflow;
    for (int f = 0; f < 16; ++f) p.hist[f] += q.hist[f];
  }
  s_p[threadIdx.x] = p;
  __syncthreads();
  if (threadIdx.x == 0) {
    StatsPartial t{};
    for (int i = 0; i < kStatsThreads; ++i) {
      const StatsPartial &q = s_p[i];
      for (int f = 0; f < 5; ++f) t.sum[f] += q.sum[f];
      t.n_elems += q.n_elems;
      t.n_nonzero += q.n_nonzero;
      t.n_underflow += q.n_underflow;
      for (int f = 0; f < 16; ++f) t.hist[f] += q.hist[f];
    }
    *out = t;
  }
}

static int stats_grid(int64_t work) {
  int64_t b = (work + kStatsThreads - 1) / kStatsThreads;
  if (b > kStatsMaxBlocks) b = kStatsMaxBlocks;
  return b < 1 ? 1 : (int)b;
}

hipError_t launch_quant_stats(const StatsArgs &a, StatsPartial *workspace, StatsPartial *out,
                              hipStream_t st) {
  const int blocks = stats_grid(a.rows * (a.kpad / 16));
  if (a.grid == kGridUniform)
    hipLaunchKernelGGL((quant_stats_kernel<kGridUniform>), dim3(blocks), dim3(kStatsThreads), 0,
                       st, a, workspace);
  else if (a.grid == kGridE2M1)
    hipLaunchKernelGGL((quant_stats_kernel<kGridE2M1>), dim3(blocks), dim3(kStatsThreads), 0, st,
                       a, workspace);
  else
    hipLaunchKernelGGL((quant_stats_kernel<kGridE2M1Max2>), dim3(blocks), dim3(kStatsThreads), 0,
                       st, a, workspace);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(kStatsThreads), 0, st, workspace, blocks,
                     out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of the no-allocation diagnostics call: the kStatsMaxBlocks partial
// records (192 KiB) in device memory the library itself owns.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` only stands in for the symbol; its device address comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept below, and only that address reaches kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) StatsPartial scratch[kStatsMaxBlocks];

constexpr int kMaxDevices = 64;
static std::atomic<StatsPartial *> g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (looked up on the first call on
// that device; concurrent first calls store the same address).
static hipError_t scratch_address(StatsPartial **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  StatsPartial *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void *addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (addr == nullptr) return hipErrorInvalidSymbol;
    p = static_cast<StatsPartial *>(addr);
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_quant_stats_scratch(const StatsArgs &a, StatsPartial *out, hipStream_t st) {
  // the grid (one partial per workgroup) never exceeds the array
  if (stats_grid(a.rows * (a.kpad / 16)) > kStatsMaxBlocks) return hipErrorInvalidValue;
  StatsPartial *ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_quant_stats(a, ws, out, st);
}

hipError_t launch_output_stats(const float *ref, int64_t ld_ref, const float *test,
                               int64_t ld_test, int64_t rows, int64_t cols,
                               StatsPartial *workspace, StatsPartial *out, hipStream_t st) {
  const int blocks = stats_grid(rows * cols);
  hipLaunchKernelGGL(output_stats_kernel, dim3(blocks), dim3(kStatsThreads), 0, st, ref, ld_ref,
                     test, ld_test, rows, cols, workspace);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(kStatsThreads), 0, st, workspace, blocks,
                     out);
  return hipGetLastError();
}

}  // namespace ufp4
