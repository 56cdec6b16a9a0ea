// Host-side launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ufp4 {

struct QuantArgs {
  const uint16_t *x;
  int64_t n_rows, n_cols, ld;
  int axis;                 // 0 along columns, 1 along rows (transposed), 2 stacked
  const int64_t *goff;      // device group offsets or nullptr
  int n_groups;
  int rht;
  uint32_t sign_mask;
  int grid, rnd;
  uint32_t seed_lo, seed_hi, stream_id;
  int64_t kpad;             // padded contraction length of the output
  uint8_t *codes;
  float *scales;
};

constexpr int kMaxGroupsApi = 1024;

hipError_t launch_quantize(const QuantArgs &a, hipStream_t st);
// Dual-axis quantization: the row-wise operand (blocks along columns) and
// the column-wise one (axis 1 or 2, with groups / stacking as QuantArgs) from
// one read of x.  Signs are 0 for a side without RHT.
struct DualArgs {
  const uint16_t *x;
  int64_t n_rows, n_cols, ld;
  int col_axis;             // 1 along rows (transposed), 2 stacked
  const int64_t *goff;      // device group offsets or nullptr (axis 1 only)
  int n_groups;
  int grid, rnd;
  uint32_t seed_lo, seed_hi;
  int rht_r;                // row-wise output
  uint32_t mask_r, sid_r;
  int64_t kpad_r;
  uint8_t *codes_r;
  float *scales_r;
  int rht_c;                // column-wise output
  uint32_t mask_c, sid_c;
  int64_t kpad_c;
  uint8_t *codes_c;
  float *scales_c;
};

hipError_t launch_quantize_dual(const DualArgs &a, hipStream_t st);
hipError_t launch_dequantize(const uint8_t *codes, const float *scales, int64_t rows,
                             int64_t kpad, int grid, bool inverse, uint32_t sign_mask, float *out,
                             int64_t ld_out, hipStream_t st);

// Diagnostics: sums and counts comparing an input with its quantization
// (axis 0 row-wise, 1 transposed, one group), or a GEMM output with its
// reference.  Same layout as the public ufp4_stats.
struct StatsPartial {
  double sum[5];            // x^2, (xhat - x)^2, x * xhat, |x|, |xhat|
  uint64_t n_elems, n_nonzero, n_underflow;
  uint64_t hist[16];
};
constexpr int kStatsMaxBlocks = 1024;   // partials in the workspace

struct StatsArgs {
  const uint16_t *x;
  int64_t ld;
  int axis;
  int64_t rows, kpad, kvalid;   // quantized rows, padded K, logical K
  const uint8_t *codes;
  const float *scales;
  int grid, rht;
  uint32_t sign_mask;
};

hipError_t launch_quant_stats(const StatsArgs &a, StatsPartial *workspace, StatsPartial *out,
                              hipStream_t st);
// The same with the partials in the library's own per-device scratch array
// (no workspace argument, no allocation).
hipError_t launch_quant_stats_scratch(const StatsArgs &a, StatsPartial *out, hipStream_t st);
hipError_t launch_output_stats(const float *ref, int64_t ld_ref, const float *test,
                               int64_t ld_test, int64_t rows, int64_t cols,
                               StatsPartial *workspace, StatsPartial *out, hipStream_t st);

// GEMM C = A * B^T on quantized K-contiguous operands.
//   mode 0: dense, A [M, kpad], B [N, kpad], C [M, N].
//   mode 1: grouped along M: A rows split by goff, B [n_groups*N, kpad].
//   mode 2: grouped along K: per-group padded K segments, C [n_groups, M, N].
struct GemmArgs {
  const uint8_t *a_codes;
  const float *a_scales;
  const uint8_t *b_codes;
  const float *b_scales;
  int64_t M, N, kpad;
  void *c;                  // FP32, or bf16 bit patterns when out_bf16
  int64_t ldc;
  int out_bf16;             // 1: round the FP32 result to bf16 (nearest even)
  int mode;
  const int64_t *goff;
  int n_groups;
  int grid;
  // mode 0 split-K: n_split > 1 splits the blocks into runs of split_kb, and
  // split s writes its partial output at c + s * split_stride
  int n_split;
  int64_t split_kb;
  int64_t split_stride;
};

hipError_t launch_gemm(const GemmArgs &g, hipStream_t st);

// Split-K of a dense GEMM whose output tiles do not fill the GPU: partial
// outputs of the K splits in the FP32 workspace ws [n_split, M, N], then a
// fixed-order sum into g.c (FP32, row stride g.ldc).
constexpr int kSplitSlots = 512;      // workgroups the GPU runs at once (2 per CU, 256 CUs)
constexpr int kMaxSplits = 16;
constexpr int kMinSplitBlocks = 64;   // at least 1024 of K per split
int gemm_splits(int64_t M, int64_t N, int64_t kpad);
hipError_t launch_gemm_split(const GemmArgs &g, float *ws, hipStream_t st);

}  // namespace ufp4
