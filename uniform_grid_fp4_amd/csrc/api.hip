// C ABI of libufp4.so: host-side validation, then one launch on the caller's
// stream.  No allocation, no synchronisation, no global mutable state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ufp4.h"
#include "ufp4_kernels.h"

using namespace ufp4;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
int64_t round_up16(int64_t n) { return (n + 15) / 16 * 16; }

ufp4_status check_qtensor(const ufp4_qtensor *q) {
  if (q == nullptr || q->codes == nullptr || q->scales == nullptr) return UFP4_ERR_INVALID_ARG;
  if (!aligned16(q->codes) || !aligned16(q->scales) || q->reserved != 0)
    return UFP4_ERR_INVALID_ARG;
  if (q->grid != UFP4_GRID_UNIFORM && q->grid != UFP4_GRID_E2M1 && q->grid != UFP4_GRID_E2M1_MAX2)
    return UFP4_ERR_INVALID_ARG;
  if (q->rht != 0 && q->rht != 1) return UFP4_ERR_INVALID_ARG;
  if (q->rows <= 0 || q->kpad <= 0 || q->kpad % 16 != 0 || q->k <= 0 || q->k > q->kpad)
    return UFP4_ERR_SHAPE;
  return UFP4_OK;
}

// Size limits of the kernels' 32-bit buffer offsets: a GEMM tile's operand
// panel (128 rows x kpad/2 bytes) and a column-wise quantizer block (16 rows
// of ld elements) must stay below 2^31 bytes.
constexpr int64_t kMaxKpad = int64_t(1) << 24;
constexpr int64_t kMaxColumnLd = int64_t(1) << 26;

ufp4_status check_pair(const ufp4_qtensor *a, const ufp4_qtensor *b) {
  ufp4_status s = check_qtensor(a);
  if (s != UFP4_OK) return s;
  s = check_qtensor(b);
  if (s != UFP4_OK) return s;
  if (a->kpad > kMaxKpad) return UFP4_ERR_UNSUPPORTED;
  if (a->k != b->k || a->kpad != b->kpad || a->grid != b->grid || a->rht != b->rht ||
      (a->rht && ((a->sign_mask ^ b->sign_mask) & 0xFFFFu) != 0))
    return UFP4_ERR_MISMATCH;
  return UFP4_OK;
}

// Workspace bytes of a dense GEMM's split-K (0: it does not split).
size_t split_workspace_bytes(int64_t m, int64_t n, int64_t kpad) {
  if (m <= 0 || n <= 0 || kpad <= 0 || kpad % 16 != 0) return 0;
  const int splits = gemm_splits(m, n, kpad);
  return splits > 1 ? (size_t)splits * (size_t)m * (size_t)n * sizeof(float) : 0;
}

// Dense GEMM; with `ws` (FP32, at least split_workspace_bytes) K is split.
ufp4_status dense_gemm(const ufp4_qtensor *a, const ufp4_qtensor *b, void *c, int out_bf16,
                       int64_t ldc, hipStream_t stream, float *ws = nullptr) {
  ufp4_status s = check_pair(a, b);
  if (s != UFP4_OK) return s;
  if (c == nullptr) return UFP4_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(c) & (out_bf16 ? 1u : 3u)) != 0) return UFP4_ERR_INVALID_ARG;
  if (ldc < b->rows) return UFP4_ERR_SHAPE;
  GemmArgs g{};
  g.a_codes = a->codes;
  g.a_scales = a->scales;
  g.b_codes = b->codes;
  g.b_scales = b->scales;
  g.M = a->rows;
  g.N = b->rows;
  g.kpad = a->kpad;
  g.c = c;
  g.ldc = ldc;
  g.out_bf16 = out_bf16;
  g.mode = 0;
  g.goff = nullptr;
  g.n_groups = 1;
  g.grid = a->grid;
  g.n_split = 1;
  g.split_kb = a->kpad / 16;
  g.split_stride = 0;
  if (ws != nullptr && !out_bf16) {
    g.n_split = gemm_splits(g.M, g.N, g.kpad);
    if (g.n_split > 1) return launch_gemm_split(g, ws, stream) == hipSuccess ? UFP4_OK : UFP4_ERR_HIP;
    g.n_split = 1;
  }
  return launch_gemm(g, stream) == hipSuccess ? UFP4_OK : UFP4_ERR_HIP;
}

// Every check of one quantization call (shared by the single and the
// dual-axis entry points); nothing is launched unless it passes.
ufp4_status check_quant(const uint16_t *x_bf16, int64_t n_rows, int64_t n_cols, int64_t ld,
                        int32_t axis, const int64_t *d_group_offsets, int32_t n_groups,
                        int32_t rht, uint32_t sign_mask, int32_t grid, int32_t rnd,
                        const ufp4_qtensor *out) {
  if (x_bf16 == nullptr || out == nullptr || out->codes == nullptr || out->scales == nullptr)
    return UFP4_ERR_INVALID_ARG;
  if (!aligned16(out->codes) || !aligned16(out->scales) || out->reserved != 0)
    return UFP4_ERR_INVALID_ARG;
  if (axis != UFP4_BLOCKS_ALONG_COLS && axis != UFP4_BLOCKS_ALONG_ROWS &&
      axis != UFP4_BLOCKS_ALONG_ROWS_STACKED)
    return UFP4_ERR_INVALID_ARG;
  if (grid != UFP4_GRID_UNIFORM && grid != UFP4_GRID_E2M1 && grid != UFP4_GRID_E2M1_MAX2)
    return UFP4_ERR_INVALID_ARG;
  if (rnd != UFP4_ROUND_RTNE && rnd != UFP4_ROUND_SR) return UFP4_ERR_INVALID_ARG;
  if (rht != 0 && rht != 1) return UFP4_ERR_INVALID_ARG;
  if (sign_mask > 0xFFFFu) return UFP4_ERR_INVALID_ARG;
  if (n_rows <= 0 || n_cols <= 0 || ld < n_cols) return UFP4_ERR_SHAPE;
  if (axis != UFP4_BLOCKS_ALONG_COLS && ld > kMaxColumnLd) return UFP4_ERR_UNSUPPORTED;
  if (axis == UFP4_BLOCKS_ALONG_COLS && (d_group_offsets != nullptr || n_groups != 0))
    return UFP4_ERR_INVALID_ARG;
  if (axis == UFP4_BLOCKS_ALONG_ROWS) {
    if ((d_group_offsets == nullptr) != (n_groups == 0)) return UFP4_ERR_INVALID_ARG;
    if (d_group_offsets != nullptr && (n_groups < 1 || n_groups > kMaxGroupsApi))
      return UFP4_ERR_SHAPE;
  }
  if (axis == UFP4_BLOCKS_ALONG_ROWS_STACKED) {
    if (d_group_offsets != nullptr) return UFP4_ERR_INVALID_ARG;
    if (n_groups < 1 || n_rows % n_groups != 0) return UFP4_ERR_SHAPE;
  }
  int64_t rows, kmin;
  if (axis == UFP4_BLOCKS_ALONG_COLS) {
    rows = n_rows;
    kmin = round_up16(n_cols);
    if (out->kpad != kmin) return UFP4_ERR_SHAPE;
  } else if (axis == UFP4_BLOCKS_ALONG_ROWS_STACKED) {
    rows = n_cols * (int64_t)n_groups;
    kmin = round_up16(n_rows / n_groups);
    if (out->kpad != kmin) return UFP4_ERR_SHAPE;
  } else {
    rows = n_cols;
    kmin = d_group_offsets ? round_up16(n_rows + 15 * (int64_t)n_groups) : round_up16(n_rows);
    if (d_group_offsets ? (out->kpad < kmin || out->kpad % 16 != 0) : (out->kpad != kmin))
      return UFP4_ERR_SHAPE;
  }
  if (out->rows != rows) return UFP4_ERR_SHAPE;
  return UFP4_OK;
}

void fill_quant_desc(ufp4_qtensor *out, int64_t n_rows, int64_t n_cols, int32_t axis,
                     int32_t n_groups, int32_t rht, uint32_t sign_mask, int32_t grid) {
  out->k = (axis == UFP4_BLOCKS_ALONG_COLS) ? n_cols
           : (axis == UFP4_BLOCKS_ALONG_ROWS_STACKED) ? n_rows / n_groups : n_rows;
  out->grid = grid;
  out->rht = rht;
  out->sign_mask = rht ? sign_mask : 0u;
}

// Checks of a quantization-diagnostics call (workspace aside) and its
// kernel arguments.
ufp4_status quant_stats_args(const uint16_t *x_bf16, int64_t n_rows, int64_t n_cols, int64_t ld,
                             int32_t axis, const ufp4_qtensor *q, const ufp4_stats *d_out,
                             StatsArgs &a) {
  ufp4_status s = check_qtensor(q);
  if (s != UFP4_OK) return s;
  if (x_bf16 == nullptr || d_out == nullptr) return UFP4_ERR_INVALID_ARG;
  if (!aligned8(d_out)) return UFP4_ERR_INVALID_ARG;
  if (axis != UFP4_BLOCKS_ALONG_COLS && axis != UFP4_BLOCKS_ALONG_ROWS)
    return UFP4_ERR_INVALID_ARG;
  if (n_rows <= 0 || n_cols <= 0 || ld < n_cols) return UFP4_ERR_SHAPE;
  const int64_t rows = axis == UFP4_BLOCKS_ALONG_COLS ? n_rows : n_cols;
  const int64_t k = axis == UFP4_BLOCKS_ALONG_COLS ? n_cols : n_rows;
  if (q->rows != rows || q->k != k || q->kpad != round_up16(k)) return UFP4_ERR_SHAPE;
  a = StatsArgs{};
  a.x = x_bf16;
  a.ld = ld;
  a.axis = axis;
  a.rows = rows;
  a.kpad = q->kpad;
  a.kvalid = k;
  a.codes = q->codes;
  a.scales = q->scales;
  a.grid = q->grid;
  a.rht = q->rht;
  a.sign_mask = q->rht ? q->sign_mask : 0u;
  return UFP4_OK;
}

}  // namespace

extern "C" {

ufp4_status ufp4_rht_quantize(const uint16_t *x_bf16, int64_t n_rows, int64_t n_cols, int64_t ld,
                              int32_t axis, const int64_t *d_group_offsets, int32_t n_groups,
                              int32_t rht, uint32_t sign_mask, int32_t grid, int32_t rnd,
                              uint64_t seed, uint32_t stream_id, ufp4_qtensor *out,
                              hipStream_t stream) {
  ufp4_status st = check_quant(x_bf16, n_rows, n_cols, ld, axis, d_group_offsets, n_groups, rht,
                               sign_mask, grid, rnd, out);
  if (st != UFP4_OK) return st;
  QuantArgs a{};
  a.x = x_bf16;
  a.n_rows = n_rows;
  a.n_cols = n_cols;
  a.ld = ld;
  a.axis = axis;
  a.goff = d_group_offsets;
  a.n_groups = n_groups;
  a.rht = rht;
  a.sign_mask = sign_mask;
  a.grid = grid;
  a.rnd = rnd;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.stream_id = stream_id;
  a.kpad = out->kpad;
  a.codes = out->codes;
  a.scales = out->scales;
  if (launch_quantize(a, stream) != hipSuccess) return UFP4_ERR_HIP;
  fill_quant_desc(out, n_rows, n_cols, axis, n_groups, rht, sign_mask, grid);
  return UFP4_OK;
}

ufp4_status ufp4_rht_quantize_dual(const uint16_t *x_bf16, int64_t n_rows, int64_t n_cols,
                                   int64_t ld, int32_t col_axis, const int64_t *d_group_offsets,
                                   int32_t n_groups, int32_t grid, int32_t rnd, uint64_t seed,
                                   const ufp4_quant_side *rowwise, const ufp4_quant_side *colwise,
                                   ufp4_qtensor *out_rows, ufp4_qtensor *out_cols,
                                   hipStream_t stream) {
  if (rowwise == nullptr || colwise == nullptr || out_rows == nullptr || out_cols == nullptr)
    return UFP4_ERR_INVALID_ARG;
  if (rowwise->reserved != 0 || colwise->reserved != 0) return UFP4_ERR_INVALID_ARG;
  if (col_axis != UFP4_BLOCKS_ALONG_ROWS && col_axis != UFP4_BLOCKS_ALONG_ROWS_STACKED)
    return UFP4_ERR_INVALID_ARG;
  if (out_rows->codes == out_cols->codes || out_rows->scales == out_cols->scales)
    return UFP4_ERR_INVALID_ARG;
  ufp4_status st = check_quant(x_bf16, n_rows, n_cols, ld, UFP4_BLOCKS_ALONG_COLS, nullptr, 0,
                               rowwise->rht, rowwise->sign_mask, grid, rnd, out_rows);
  if (st != UFP4_OK) return st;
  st = check_quant(x_bf16, n_rows, n_cols, ld, col_axis, d_group_offsets, n_groups, colwise->rht,
                   colwise->sign_mask, grid, rnd, out_cols);
  if (st != UFP4_OK) return st;
  DualArgs a{};
  a.x = x_bf16;
  a.n_rows = n_rows;
  a.n_cols = n_cols;
  a.ld = ld;
  a.col_axis = col_axis;
  a.goff = d_group_offsets;
  a.n_groups = n_groups;
  a.grid = grid;
  a.rnd = rnd;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.rht_r = rowwise->rht;
  a.mask_r = rowwise->rht ? rowwise->sign_mask : 0u;
  a.sid_r = rowwise->stream_id;
  a.kpad_r = out_rows->kpad;
  a.codes_r = out_rows->codes;
  a.scales_r = out_rows->scales;
  a.rht_c = colwise->rht;
  a.mask_c = colwise->rht ? colwise->sign_mask : 0u;
  a.sid_c = colwise->stream_id;
  a.kpad_c = out_cols->kpad;
  a.codes_c = out_cols->codes;
  a.scales_c = out_cols->scales;
  if (launch_quantize_dual(a, stream) != hipSuccess) return UFP4_ERR_HIP;
  fill_quant_desc(out_rows, n_rows, n_cols, UFP4_BLOCKS_ALONG_COLS, 0, rowwise->rht,
                  rowwise->sign_mask, grid);
  fill_quant_desc(out_cols, n_rows, n_cols, col_axis, n_groups, colwise->rht, colwise->sign_mask,
                  grid);
  return UFP4_OK;
}

ufp4_status ufp4_dequantize(const ufp4_qtensor *q, int32_t inverse_rht, float *out,
                            int64_t ld_out, hipStream_t stream) {
  ufp4_status s = check_qtensor(q);
  if (s != UFP4_OK) return s;
  if (out == nullptr || (inverse_rht != 0 && inverse_rht != 1)) return UFP4_ERR_INVALID_ARG;
  if (inverse_rht && !q->rht) return UFP4_ERR_INVALID_ARG;
  if (ld_out < q->kpad) return UFP4_ERR_SHAPE;
  return launch_dequantize(q->codes, q->scales, q->rows, q->kpad, q->grid, inverse_rht != 0,
                           q->sign_mask, out, ld_out, stream) == hipSuccess
             ? UFP4_OK
             : UFP4_ERR_HIP;
}

ufp4_status ufp4_gemm_fprop(const ufp4_qtensor *xq, const ufp4_qtensor *wq, float *y, int64_t ldy,
                            hipStream_t stream) {
  return dense_gemm(xq, wq, y, 0, ldy, stream);
}

ufp4_status ufp4_gemm_dgrad(const ufp4_qtensor *dyq, const ufp4_qtensor *wtq, float *dx,
                            int64_t ldx, hipStream_t stream) {
  return dense_gemm(dyq, wtq, dx, 0, ldx, stream);
}

ufp4_status ufp4_gemm_wgrad(const ufp4_qtensor *dytq, const ufp4_qtensor *xtq, float *dw,
                            int64_t lddw, void *workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  if ((workspace == nullptr) != (workspace_bytes == 0)) return UFP4_ERR_INVALID_ARG;
  if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 3u) != 0)
    return UFP4_ERR_INVALID_ARG;
  float *ws = nullptr;
  if (workspace != nullptr && dytq != nullptr && xtq != nullptr) {
    const size_t need = split_workspace_bytes(dytq->rows, xtq->rows, dytq->kpad);
    if (need > 0 && workspace_bytes >= need) ws = static_cast<float *>(workspace);
  }
  return dense_gemm(dytq, xtq, dw, 0, lddw, stream, ws);
}

ufp4_status ufp4_gemm_out(int32_t kind, const ufp4_qtensor *a, const ufp4_qtensor *b, void *c,
                          int32_t out_dtype, int64_t ldc, hipStream_t stream) {
  if (kind < 0 || kind > 2) return UFP4_ERR_INVALID_ARG;
  if (out_dtype != UFP4_OUT_F32 && out_dtype != UFP4_OUT_BF16) return UFP4_ERR_INVALID_ARG;
  return dense_gemm(a, b, c, out_dtype == UFP4_OUT_BF16, ldc, stream);
}

ufp4_status ufp4_grouped_gemm(int32_t kind, int32_t n_groups, const int64_t *d_group_offsets,
                              const ufp4_qtensor *a, const ufp4_qtensor *b, float *c, int64_t ldc,
                              void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if ((workspace == nullptr) != (workspace_bytes == 0)) return UFP4_ERR_INVALID_ARG;
  return ufp4_grouped_gemm_out(kind, n_groups, d_group_offsets, a, b, c, UFP4_OUT_F32, ldc,
                               stream);
}

ufp4_status ufp4_grouped_gemm_out(int32_t kind, int32_t n_groups, const int64_t *d_group_offsets,
                                  const ufp4_qtensor *a, const ufp4_qtensor *b, void *c,
                                  int32_t out_dtype, int64_t ldc, hipStream_t stream) {
  if (kind < 0 || kind > 2) return UFP4_ERR_INVALID_ARG;
  if (d_group_offsets == nullptr || c == nullptr) return UFP4_ERR_INVALID_ARG;
  if (out_dtype != UFP4_OUT_F32 && out_dtype != UFP4_OUT_BF16) return UFP4_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(c) & (out_dtype == UFP4_OUT_BF16 ? 1u : 3u)) != 0)
    return UFP4_ERR_INVALID_ARG;
  if (n_groups < 1 || n_groups > kMaxGroupsApi) return UFP4_ERR_SHAPE;
  ufp4_status s = check_pair(a, b);
  if (s != UFP4_OK) return s;
  GemmArgs g{};
  g.a_codes = a->codes;
  g.a_scales = a->scales;
  g.b_codes = b->codes;
  g.b_scales = b->scales;
  g.kpad = a->kpad;
  g.c = c;
  g.ldc = ldc;
  g.out_bf16 = out_dtype == UFP4_OUT_BF16;
  g.goff = d_group_offsets;
  g.n_groups = n_groups;
  g.grid = a->grid;
  g.n_split = 1;
  g.split_kb = a->kpad / 16;
  g.split_stride = 0;
  g.M = a->rows;
  if (kind == 2) {
    g.mode = 2;
    g.N = b->rows;
  } else {
    g.mode = 1;
    if (b->rows % n_groups != 0) return UFP4_ERR_SHAPE;
    g.N = b->rows / n_groups;
  }
  if (ldc < g.N) return UFP4_ERR_SHAPE;
  return launch_gemm(g, stream) == hipSuccess ? UFP4_OK : UFP4_ERR_HIP;
}

static_assert(sizeof(ufp4_stats) == sizeof(StatsPartial), "ufp4_stats layout");

size_t ufp4_stats_workspace_size(void) { return (size_t)kStatsMaxBlocks * sizeof(StatsPartial); }

ufp4_status ufp4_quant_stats(const uint16_t *x_bf16, int64_t n_rows, int64_t n_cols, int64_t ld,
                             int32_t axis, const ufp4_qtensor *q, void *workspace,
                             size_t workspace_bytes, ufp4_stats *d_out, hipStream_t stream) {
  StatsArgs a;
  const ufp4_status s = quant_stats_args(x_bf16, n_rows, n_cols, ld, axis, q, d_out, a);
  if (s != UFP4_OK) return s;
  if (workspace == nullptr || !aligned8(workspace)) return UFP4_ERR_INVALID_ARG;
  if (workspace_bytes < ufp4_stats_workspace_size()) return UFP4_ERR_INVALID_ARG;
  return launch_quant_stats(a, static_cast<StatsPartial *>(workspace),
                            reinterpret_cast<StatsPartial *>(d_out), stream) == hipSuccess
             ? UFP4_OK
             : UFP4_ERR_HIP;
}

ufp4_status ufp4_quant_stats_noalloc(const uint16_t *x_bf16, int64_t n_rows, int64_t n_cols,
                                     int64_t ld, int32_t axis, const ufp4_qtensor *q,
                                     ufp4_stats *d_out, hipStream_t stream) {
  StatsArgs a;
  const ufp4_status s = quant_stats_args(x_bf16, n_rows, n_cols, ld, axis, q, d_out, a);
  if (s != UFP4_OK) return s;
  return launch_quant_stats_scratch(a, reinterpret_cast<StatsPartial *>(d_out), stream) ==
                 hipSuccess
             ? UFP4_OK
             : UFP4_ERR_HIP;
}

ufp4_status ufp4_output_stats(const float *ref, int64_t ld_ref, const float *test,
                              int64_t ld_test, int64_t rows, int64_t cols, void *workspace,
                              size_t workspace_bytes, ufp4_stats *d_out, hipStream_t stream) {
  if (ref == nullptr || test == nullptr || workspace == nullptr || d_out == nullptr)
    return UFP4_ERR_INVALID_ARG;
  if (!aligned8(workspace) || !aligned8(d_out)) return UFP4_ERR_INVALID_ARG;
  if (workspace_bytes < ufp4_stats_workspace_size()) return UFP4_ERR_INVALID_ARG;
  if (rows <= 0 || cols <= 0 || ld_ref < cols || ld_test < cols) return UFP4_ERR_SHAPE;
  return launch_output_stats(ref, ld_ref, test, ld_test, rows, cols,
                             static_cast<StatsPartial *>(workspace),
                             reinterpret_cast<StatsPartial *>(d_out), stream) == hipSuccess
             ? UFP4_OK
             : UFP4_ERR_HIP;
}

size_t ufp4_workspace_size(int32_t kind, int64_t m, int64_t n, int64_t kpad, int32_t n_groups) {
  if (kind != 2 || n_groups != 1) return 0;
  return split_workspace_bytes(m, n, kpad);
}

const char *ufp4_status_string(ufp4_status status) {
  switch (status) {
    case UFP4_OK: return "UFP4_OK";
    case UFP4_ERR_INVALID_ARG: return "UFP4_ERR_INVALID_ARG";
    case UFP4_ERR_SHAPE: return "UFP4_ERR_SHAPE";
    case UFP4_ERR_MISMATCH: return "UFP4_ERR_MISMATCH";
    case UFP4_ERR_UNSUPPORTED: return "UFP4_ERR_UNSUPPORTED";
    case UFP4_ERR_HIP: return "UFP4_ERR_HIP";
  }
  return "UFP4_ERR_UNKNOWN";
}

}  // extern "C"
