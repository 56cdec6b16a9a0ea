/*
 * ufp4.h -- C ABI of libufp4.so, the MI355X (gfx950) hot path of the UFP4
 * 4-bit training recipe: a fused random-Hadamard-transform + blockwise absmax
 * 4-bit quantizer and the block-scaled 4-bit GEMMs it feeds.
 *
 * What is computed comes from "Rethinking Shrinkage Bias in LLM FP4
 * Pretraining: Geometric Origin, Systemic Impact, and UFP4 Recipe"
 * (arXiv 2606.20381), as summarised on paperlayer.ai:
 *   - section 2 "Blockwise quantization": contiguous blocks, one shared scale
 *     per block, a normalised codebook with largest magnitude gmax and a
 *     rounding rule;
 *   - section 2 "Rounding rules": RTNE (nearest level, deterministic ties) or
 *     stochastic rounding between the adjacent levels (unbiased);
 *   - section 2 "Random Hadamard transforms": random sign diagonal, then a
 *     Sylvester Hadamard transform, applied along each training GEMM's
 *     reduction dimension (input channels for FPROP, output channels for
 *     DGRAD, tokens for WGRAD), the GEMM consuming the rotated quantized
 *     operands;
 *   - section 4 "UFP4 Recipe": uniform E1M2/INT4 grid, RHT on all three GEMMs,
 *     stochastic rounding on dY only.
 *
 * Fixed choices where the pages are silent: block = RHT size = 16, FP32
 * absmax block scale, one 16-bit sign mask per GEMM, Philox4x32-10 for the
 * stochastic rounding, nibble layout sign<<3 | magnitude index, low nibble
 * first.  Every quantized code and scale is bit-exact and deterministic;
 * GEMM outputs are FP32 and deterministic run to run.
 *
 * Conventions for every entry point:
 *   - All buffer pointers are DEVICE pointers owned by the caller (the
 *     library never allocates, frees or synchronises).  Descriptor structs
 *     are HOST memory read during the call.  The only state the library
 *     keeps is two host-side, write-once caches per device: the compute-unit
 *     count the quantizers size their grids by, and a bit recording that the
 *     GEMM kernels' dynamic-LDS attribute has been set; neither changes any
 *     result.
 *   - Work is enqueued on `stream` and runs asynchronously; results are valid
 *     once the stream has reached that point.  A call enqueues kernel
 *     launches only (no copy, memset or allocation), so a sequence of calls
 *     can be stream-captured into a HIP graph and replayed.  The first GEMM
 *     call of each kind on a device also sets a one-time kernel attribute;
 *     make it before capturing.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failed check returns a negative status and enqueues nothing.  A HIP
 *     launch failure returns UFP4_ERR_HIP.
 *   - Inputs must be finite with |x| < 2^123 (larger values may overflow the
 *     FP32 butterfly); NaN/Inf inputs give unspecified codes.
 */
#ifndef UFP4_H
#define UFP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  UFP4_OK = 0,
  UFP4_ERR_INVALID_ARG = -1, /* null pointer, unknown enum, misalignment  */
  UFP4_ERR_SHAPE = -2,       /* sizes inconsistent or out of range        */
  UFP4_ERR_MISMATCH = -3,    /* GEMM operands quantized incompatibly      */
  UFP4_ERR_UNSUPPORTED = -4, /* valid request this build does not serve   */
  UFP4_ERR_HIP = -5          /* the HIP runtime rejected a launch         */
} ufp4_status;

/* Grids (paperlayer.ai summary, section 2 "FP4 formats").
 *  UNIFORM: E1M2/INT4 grid {-7..7}/7 times the scale; the nibble's 3-bit
 *           magnitude field is the integer level k (the E1M2 bit layout).
 *  E2M1:    the OCP E2M1 grid {0,.5,1,1.5,2,3,4,6}/6 times the scale; the
 *           nibble is the E2M1 bit pattern.
 *  E2M1_MAX2: range-restricted E2M1 with max_fpx = 2.0 (paperlayer.ai
 *           section 5 "Q4: Recipe ablations"): only {0,.5,1,1.5,2}, i.e.
 *           {0,.5,1,1.5,2}/2 times the scale; E2M1 bit patterns with a
 *           magnitude index of at most 4. */
typedef enum { UFP4_GRID_UNIFORM = 0, UFP4_GRID_E2M1 = 1, UFP4_GRID_E2M1_MAX2 = 2 } ufp4_grid;

/* Rounding (paperlayer.ai summary, section 2 "Rounding rules").
 *  RTNE: nearest level, ties to the even level index.
 *  SR:   up with probability floor(f*2^32)/2^32, f the position between the
 *        two adjacent levels; the 32 random bits of output element idx
 *        (= row*kpad + k of the quantized layout) are word (idx & 3) of
 *        Philox4x32-10 with key (seed lo, seed hi) and counter
 *        (lo32(idx>>2), hi32(idx>>2), stream_id, 0). */
typedef enum { UFP4_ROUND_RTNE = 0, UFP4_ROUND_SR = 1 } ufp4_round;

/* Which input dimension the 16-element blocks run along.
 *  ALONG_COLS: the contiguous dimension; output row i = input row i.
 *  ALONG_ROWS: the strided dimension; the output is transposed (output row j
 *              = input column j) and contiguous along the blocked dimension,
 *              the K-contiguous layout every GEMM below consumes. */
/*  ALONG_ROWS_STACKED: the rows form n_groups equal groups (expert weights
 *              W_e stacked along rows); each group is quantized as ALONG_ROWS
 *              on its own and the transposed outputs are stacked: group e
 *              fills output rows [e * n_cols, (e + 1) * n_cols).  This builds
 *              the per-expert W_e^T operands of the grouped DGRAD. */
typedef enum {
  UFP4_BLOCKS_ALONG_COLS = 0,
  UFP4_BLOCKS_ALONG_ROWS = 1,
  UFP4_BLOCKS_ALONG_ROWS_STACKED = 2
} ufp4_axis;

/* A quantized operand.  Caller-owned device buffers:
 *   codes  [rows, kpad/2] bytes, byte j of a row = nib[2j] | nib[2j+1] << 4,
 *          nibble = sign << 3 | magnitude index (a zero magnitude is always
 *          nibble 0); 16-byte aligned.
 *   scales [rows, kpad/16] FP32, the block absmax after the RHT (0 for an
 *          all-zero block); 16-byte aligned.
 * Layout is dense: row r's codes start at codes + r*kpad/2.
 * `rows` and `kpad` describe the buffers and are set by the caller; the
 * quantizer validates them and fills in k, grid, rht and sign_mask. */
typedef struct {
  uint8_t *codes;
  float *scales;
  int64_t rows;      /* output rows                                        */
  int64_t k;         /* logical contraction length before padding          */
  int64_t kpad;      /* padded contraction length, a multiple of 16        */
  int32_t grid;      /* ufp4_grid                                          */
  int32_t rht;       /* 1 if the 16-point RHT was applied                  */
  uint32_t sign_mask;/* RHT signs: bit j set => d_j = -1 (bits 0..15 used) */
  int32_t reserved;  /* must be 0                                          */
} ufp4_qtensor;

/* ufp4_rht_quantize -- fused RHT + blockwise absmax 4-bit quantization.
 *
 * x_bf16: device bf16 bit patterns [n_rows, n_cols] with row stride `ld`
 *   elements (ld >= n_cols).  Any alignment works; 16-byte aligned x with ld
 *   a multiple of 8 takes the vector-load path.
 * axis: ufp4_axis.  ALONG_COLS: out->rows = n_rows, out->kpad =
 *   roundup16(n_cols), zero-padded.  ALONG_ROWS: out->rows = n_cols, the
 *   contraction runs over input rows.
 * ALONG_ROWS_STACKED: d_group_offsets must be NULL, n_groups >= 1 divides
 *   n_rows; out->rows = n_groups * n_cols, out->kpad = roundup16(n_rows /
 *   n_groups); the SR index is that of the stacked output layout.
 * d_group_offsets / n_groups (ALONG_ROWS only; NULL and 0 for ALONG_COLS): device
 *   int64 [n_groups+1] non-decreasing row offsets, first 0, last n_rows, that
 *   split the rows into groups (e.g. tokens per expert); every group is padded
 *   to a multiple of 16 on its own, so no block straddles two groups, and
 *   group e occupies columns [P_e, P_{e+1}) of the output with
 *   P_e = sum_{e'<e} roundup16(count_e').  out->kpad must be at least
 *   roundup16(n_rows + 15*n_groups) and a multiple of 16 (a multiple of 512
 *   keeps every output row 128-byte aligned, which the column-wise kernel
 *   writes fastest); columns from P_{n_groups} to kpad are written as zeros.
 *   NULL (n_groups 0) means one group with out->kpad = roundup16(n_rows)
 *   exactly.  1 <= n_groups <= 1024.
 * rht, sign_mask: apply y = (1/4) H16 D x per block (butterfly stages
 *   h = 1,2,4,8 in FP32, then the exact 1/4) with D from the mask.
 * grid, rnd, seed, stream_id: see the enums above (seed/stream_id ignored
 *   for RTNE).
 * Per block: s = max|y| (stored), r = RN(g/s) with g = 7 (uniform), 6
 *   (E2M1) or 2 (E2M1_MAX2), t = RN(y*r) -- two roundings, no FMA; blocks with
 *   0 < s < 2^-64 use y*2^64 and s*2^64 in that step (the stored scale is s).
 * Returns UFP4_OK, INVALID_ARG (null pointer, bad enum, codes/scales not
 *   16-byte aligned, reserved != 0), SHAPE (non-positive size, ld < n_cols,
 *   rows/kpad not what the call produces), UNSUPPORTED (ALONG_ROWS or
 *   ALONG_ROWS_STACKED with ld > 2^26 elements), HIP. */
ufp4_status ufp4_rht_quantize(const uint16_t *x_bf16, int64_t n_rows, int64_t n_cols,
                              int64_t ld, int32_t axis, const int64_t *d_group_offsets,
                              int32_t n_groups, int32_t rht, uint32_t sign_mask,
                              int32_t grid, int32_t rnd, uint64_t seed, uint32_t stream_id,
                              ufp4_qtensor *out, hipStream_t stream);

/* The options that differ between the two outputs of a dual-axis
 * quantization (host struct read during the call). */
typedef struct {
  int32_t rht;        /* 1: apply the 16-point RHT with sign_mask            */
  uint32_t sign_mask; /* bits 0..15, as in ufp4_rht_quantize                 */
  uint32_t stream_id; /* SR stream of this output (ignored for RTNE)         */
  int32_t reserved;   /* must be 0                                           */
} ufp4_quant_side;

/* ufp4_rht_quantize_dual -- both operands of one tensor from a single read of
 * it.  Each training tensor feeds two GEMMs that contract it along different
 * dimensions (X: FPROP along H, WGRAD along T; W: FPROP along H, DGRAD along
 * F; dY: DGRAD along F, WGRAD along T -- paperlayer.ai section 2 "Random
 * Hadamard transforms"), so it is quantized once per axis; the pages' fusion
 * argument for the RHT (the transform rides along with the quantizer's memory
 * traffic) applies to the second axis too.
 *   out_rows: bit-identical to ufp4_rht_quantize(x, ALONG_COLS, NULL, 0,
 *             rowwise->rht, rowwise->sign_mask, grid, rnd, seed,
 *             rowwise->stream_id, out_rows).
 *   out_cols: bit-identical to ufp4_rht_quantize(x, col_axis,
 *             d_group_offsets, n_groups, colwise->rht, colwise->sign_mask,
 *             grid, rnd, seed, colwise->stream_id, out_cols).
 * col_axis: UFP4_BLOCKS_ALONG_ROWS (optionally grouped by d_group_offsets /
 *   n_groups, as in ufp4_rht_quantize) or UFP4_BLOCKS_ALONG_ROWS_STACKED
 *   (d_group_offsets NULL, n_groups stacks).
 * grid, rnd and seed are shared by both outputs.  The two outputs must not
 * share buffers.  Traffic: 2 B read + 2 x 0.75 B written per element, against
 * 2 x 2.75 B for the two single-axis calls.
 * Returns UFP4_OK, INVALID_ARG (null pointer, bad enum or axis, reserved != 0,
 *   shared output buffers, misalignment), SHAPE (either output's rows/kpad
 *   not what its single-axis call would require), HIP. */
ufp4_status ufp4_rht_quantize_dual(const uint16_t *x_bf16, int64_t n_rows, int64_t n_cols,
                                   int64_t ld, int32_t col_axis, const int64_t *d_group_offsets,
                                   int32_t n_groups, int32_t grid, int32_t rnd, uint64_t seed,
                                   const ufp4_quant_side *rowwise, const ufp4_quant_side *colwise,
                                   ufp4_qtensor *out_rows, ufp4_qtensor *out_cols,
                                   hipStream_t stream);

/* ufp4_dequantize -- out[r, k] for k < kpad, FP32 row-major with stride
 * ld_out >= kpad:  (float)((double)(sign*L[idx]) * (double)s / g)  (the
 * dequantized value of paperlayer.ai section 2 "Blockwise quantization").
 * inverse_rht != 0 (requires q->rht): each block is mapped back through
 * (1/4) D H16 in FP64 before the cast.  Returns OK, INVALID_ARG, SHAPE, HIP. */
ufp4_status ufp4_dequantize(const ufp4_qtensor *q, int32_t inverse_rht, float *out,
                            int64_t ld_out, hipStream_t stream);

/* The three training GEMMs (paperlayer.ai section 2 "Random Hadamard
 * transforms" and section 3.2).  All are C = A_hat * B_hat^T with both
 * operands K-contiguous ("TN"), FP32 out, row-major with stride ldc >= N:
 *   C[m, n] = sum_kb sa[m,kb] * sb[n,kb] * (sum_{k in kb} qa*qb) / g^2
 * over the operands' common kpad.  Each block product is exact; the scale
 * products and the sum over blocks are FP32, block by block, in chunks of
 * 65536 K-elements whose partial results are added to C in chunk order (so
 * the FP32 rounding error of the sum does not grow with kpad beyond one
 * chunk's); results are deterministic.  Operands must agree on k, kpad, grid, rht
 * and sign_mask (else UFP4_ERR_MISMATCH), which is what makes the rotation
 * cancel.  All three grids are accepted; kpad > 2^24 returns
 * UFP4_ERR_UNSUPPORTED.
 *   FPROP: A = X  [T, H] (blocks along H), B = W   [F, H]  -> Y  [T, F]
 *   DGRAD: A = dY [T, F] (blocks along F), B = W^T [H, F] (W quantized with
 *          ALONG_ROWS) -> dX [T, H]
 *   WGRAD: A = dY^T [F, T], B = X^T [H, T] (both ALONG_ROWS over tokens)
 *          -> dW [F, H].  workspace may be NULL (workspace_bytes 0).  When
 *          ufp4_workspace_size(2, F, H, kpad, 1) is non-zero and the
 *          workspace (device, 4-byte aligned, contents ignored and
 *          overwritten) holds at least that many bytes, the call splits K:
 *          each split writes FP32 partial outputs into the workspace and a
 *          second kernel sums them in split order into dW (deterministic;
 *          equal to the unsplit result within the same tolerance, not bit
 *          for bit).  A smaller workspace runs unsplit.  Returns OK,
 *          INVALID_ARG (also: NULL workspace with a size, a size with no
 *          workspace, a misaligned workspace), SHAPE, MISMATCH, UNSUPPORTED,
 *          HIP. */
ufp4_status ufp4_gemm_fprop(const ufp4_qtensor *xq, const ufp4_qtensor *wq, float *y,
                            int64_t ldy, hipStream_t stream);
ufp4_status ufp4_gemm_dgrad(const ufp4_qtensor *dyq, const ufp4_qtensor *wtq, float *dx,
                            int64_t ldx, hipStream_t stream);
ufp4_status ufp4_gemm_wgrad(const ufp4_qtensor *dytq, const ufp4_qtensor *xtq, float *dw,
                            int64_t lddw, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Output element type of the GEMM calls with an out_dtype argument.
 *  F32:  the FP32 result, as the calls above write it.
 *  BF16: that FP32 result rounded to bf16, nearest even (bf16 bit patterns;
 *        the epilogue of a bf16 training step, half the output traffic).
 *        Past a chunk of 65536 K-elements the output holds the bf16 part of
 *        the running result and the kernel keeps the rounding residual, so
 *        the final value is the FP32 result rounded once more to bf16. */
typedef enum { UFP4_OUT_F32 = 0, UFP4_OUT_BF16 = 1 } ufp4_out_dtype;

/* ufp4_gemm_out -- FPROP (kind 0), DGRAD (1) or WGRAD (2) as above, with the
 * output element type chosen by out_dtype (ldc in elements).  c must be
 * aligned to its element size.  Returns OK, INVALID_ARG, SHAPE, MISMATCH,
 * UNSUPPORTED, HIP. */
ufp4_status ufp4_gemm_out(int32_t kind, const ufp4_qtensor *a, const ufp4_qtensor *b, void *c,
                          int32_t out_dtype, int64_t ldc, hipStream_t stream);

/* ufp4_grouped_gemm -- the expert-grouped (MoE) form of the three training
 * GEMMs, for the expert layers of the pages' MoE models (paperlayer.ai
 * summary, section 5 "Q2-Q3: Long-run training and scaling": MoE 7.9B and
 * 124B), with the RHT along each GEMM's contraction as in section 2 "Random
 * Hadamard transforms" -- for WGRAD that is the tokens, so each expert's
 * token run is padded and rotated on its own.
 * kind 0 (FPROP) / 1 (DGRAD): rows of A are split into n_groups groups by the
 *   device int64 offsets d_group_offsets[n_groups+1] (first 0, last a->rows);
 *   B stacks the groups' operands, b->rows = n_groups * N; group e computes
 *   C[off_e:off_{e+1}, :N] = A_e * B_e^T.  C is [a->rows, N], stride ldc.
 * kind 2 (WGRAD): the contraction is split: A [M, kpad] and B [N, kpad] were
 *   quantized ALONG_ROWS with the same offsets (per-group padding, see
 *   ufp4_rht_quantize); C is [n_groups, M, N] with group stride M*ldc, and an
 *   empty group writes zeros.
 * 1 <= n_groups <= 1024 (else SHAPE); kpad > 2^24 returns UNSUPPORTED, and
 * the sums are accumulated as for the dense calls.
 * The grouped forms never split K (their per-group tiles fill the GPU), so
 * the workspace is unused: pass NULL and 0 (a non-NULL workspace with a size
 * is accepted and ignored).  Returns OK, INVALID_ARG, SHAPE, MISMATCH,
 * UNSUPPORTED, HIP. */
ufp4_status ufp4_grouped_gemm(int32_t kind, int32_t n_groups, const int64_t *d_group_offsets,
                              const ufp4_qtensor *a, const ufp4_qtensor *b, float *c,
                              int64_t ldc, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* Diagnostics of the pages' quantization-quality measurements
 * (paperlayer.ai section 3.2, section 5 Q1 and appendix A: tensor and
 * GEMM-output SQNR and its change under RHT, bucket utilization;
 * gist.science technical summary: a GEMM's attenuation factor alpha;
 * dreamwings.cn post: the quantization underflow ratio).  Raw sums and
 * counts, written to DEVICE memory; from them, on the host:
 *   SQNR [dB]          = 10 log10(sum_x2 / sum_err2)
 *   alpha              = sum_x_xhat / sum_x2          (1 - alpha: shrinkage)
 *   delta_mag          = (sum_abs_xhat - sum_abs_x) / sum_abs_x
 *   underflow ratio    = n_underflow / n_nonzero
 *   bucket utilization = exp(H) / 15, H the entropy of hist with bins 0 and 8
 *                        merged (the 15 signed codes).
 * Sums are FP64 and bitwise reproducible (fixed reduction order). */
typedef struct {
  double sum_x2;       /* sum x^2 (reference values)                          */
  double sum_err2;     /* sum (xhat - x)^2                                    */
  double sum_x_xhat;   /* sum x * xhat                                        */
  double sum_abs_x;    /* sum |x|                                             */
  double sum_abs_xhat; /* sum |xhat|                                          */
  uint64_t n_elems;    /* logical elements compared (padding excluded)        */
  uint64_t n_nonzero;  /* elements whose rotated pre-rounding value is != 0   */
  uint64_t n_underflow;/* ... of which the magnitude index is 0               */
  uint64_t hist[16];   /* nibble histogram of the logical elements            */
} ufp4_stats;

/* Workspace bytes every diagnostics call needs (a constant). */
size_t ufp4_stats_workspace_size(void);

/* ufp4_quant_stats -- compare the bf16 input x [n_rows, n_cols] (stride ld)
 * with its quantization q, made by ufp4_rht_quantize along `axis`
 * (ALONG_COLS, or ALONG_ROWS with one group).  Each logical element x is
 * paired with xhat = its dequantized value taken back to x's domain (the
 * block's inverse RHT (1/4) D H16 in FP64 when q->rht).  An element
 * underflows when y, its value after the RHT exactly as the quantizer
 * computes it in FP32 (y = x without RHT), is nonzero and its magnitude index
 * is 0.  workspace: device, >= ufp4_stats_workspace_size() bytes, 8-byte
 * aligned, overwritten.  d_out: device ufp4_stats, 8-byte aligned.
 * Returns OK, INVALID_ARG (null, misaligned, bad axis, workspace too small),
 * SHAPE (q does not match x and axis), HIP. */
ufp4_status ufp4_quant_stats(const uint16_t *x_bf16, int64_t n_rows, int64_t n_cols, int64_t ld,
                             int32_t axis, const ufp4_qtensor *q, void *workspace,
                             size_t workspace_bytes, ufp4_stats *d_out, hipStream_t stream);

/* ufp4_quant_stats_noalloc -- ufp4_quant_stats without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments
 * (minus workspace and workspace_bytes), checks and results, bit for bit:
 * the partial sums go to a scratch array the library holds in device memory,
 * 1024 records of 192 bytes (192 KiB) per GPU, taken on the first call on
 * each device and kept until the process ends.  The diagnostics kernels use
 * at most 1024 partial records for any input size, so no input exceeds it;
 * nothing is allocated, freed or cleared by the call.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and may return wrong
 * sums -- order them on one stream.  Returns OK, INVALID_ARG, SHAPE, HIP (also
 * when the scratch array's address cannot be obtained). */
ufp4_status ufp4_quant_stats_noalloc(const uint16_t *x_bf16, int64_t n_rows, int64_t n_cols,
                                     int64_t ld, int32_t axis, const ufp4_qtensor *q,
                                     ufp4_stats *d_out, hipStream_t stream);

/* ufp4_output_stats -- the same sums for a GEMM output `test` [rows, cols]
 * (stride ld_test) against a reference output `ref` (stride ld_ref), FP32
 * device arrays: x = ref, xhat = test; n_nonzero, n_underflow and hist are 0.
 * Workspace and d_out as for ufp4_quant_stats.  Returns OK, INVALID_ARG,
 * SHAPE, HIP. */
ufp4_status ufp4_output_stats(const float *ref, int64_t ld_ref, const float *test,
                              int64_t ld_test, int64_t rows, int64_t cols, void *workspace,
                              size_t workspace_bytes, ufp4_stats *d_out, hipStream_t stream);

/* Bytes of workspace a GEMM call can use to split K: non-zero only for the
 * dense WGRAD (kind 2, n_groups 1) of an M x N output whose 128 x 128 tiles
 * number fewer than the 512 workgroups MI355X runs at once, with
 * s = min(16, 512 / tiles, kpad / 1024) >= 2 splits: s * M * N * 4 bytes.
 * 0 for every other kind, group count or invalid shape. */
size_t ufp4_workspace_size(int32_t kind, int64_t m, int64_t n, int64_t kpad, int32_t n_groups);

/* ufp4_grouped_gemm_out -- ufp4_grouped_gemm (the MoE expert layers of
 * paperlayer.ai section 5 "Q2-Q3") with the output element type chosen by
 * out_dtype (ufp4_out_dtype; ldc in elements) and no workspace. */
ufp4_status ufp4_grouped_gemm_out(int32_t kind, int32_t n_groups, const int64_t *d_group_offsets,
                                  const ufp4_qtensor *a, const ufp4_qtensor *b, void *c,
                                  int32_t out_dtype, int64_t ldc, hipStream_t stream);

/* Static, human-readable name of a status code. */
const char *ufp4_status_string(ufp4_status status);

#ifdef __cplusplus
}
#endif
#endif /* UFP4_H */
