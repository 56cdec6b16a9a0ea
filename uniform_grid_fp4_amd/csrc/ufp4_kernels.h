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
hipError_t launch_dequantize(const uint8_t *codes, const float *scales, int64_t rows,
                             int64_t kpad, int grid, bool inverse, uint32_t sign_mask, float *out,
                             int64_t ld_out, hipStream_t st);

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
  float *c;
  int64_t ldc;
  int mode;
  const int64_t *goff;
  int n_groups;
  int grid;
};

hipError_t launch_gemm(const GemmArgs &g, hipStream_t st);

}  // namespace ufp4
