"""Plain CPU oracle for the UFP4 quantize -> block-scaled GEMM hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test-suite, the smoke check and the bench's
CPU-baseline leg use it.  It shares no code with the HIP library and imports
nothing from the package.

What it follows (the pages are four web renderings of arXiv 2606.20381,
"Rethinking Shrinkage Bias in LLM FP4 Pretraining: Geometric Origin, Systemic
Impact, and UFP4 Recipe"):

* paperlayer.ai summary, section 2 "Preliminaries":
    - FP4 formats: sign bit plus ExMy fields; the study uses E2M1, E1M2, INT4.
    - Blockwise quantization: contiguous blocks, one shared scale per block,
      a normalized codebook G with largest magnitude gmax, rounding rule rho_G.
    - Rounding rules: RTNE (nearest level, deterministic tie-break) and SR
      (samples adjacent levels, unbiased in expectation).
    - Random Hadamard transforms: random diagonal sign matrix followed by a
      Sylvester Hadamard transform, norm preserving; applied along each
      training GEMM's reduction dimension.
* paperlayer.ai summary, section 3.1 "Geometric Origin": conditional RTNE
  error of a bin [q - l, q + r] under locally uniform density is (l - r)/2.
* gist.science (nl) technical summary, "Methodologie" (E2M1 = 2 exponent
  bits, 1 mantissa bit; uniform E1M2/INT4 grid has equal spacing).
* paperlayer.ai summary, section 4 and 7: UFP4 = uniform grid, RHT on all
  three GEMMs, stochastic rounding on dY only.
* Diagnostics (``quant_stats``, ``output_stats``, ``stats_summary``):
  paperlayer.ai section 3.2, section 5 Q1 and appendix A (tensor and
  GEMM-output SQNR, their change under RHT, effective bucket utilization);
  gist.science technical summary (attenuation factor alpha < 1 of a GEMM);
  the dreamwings.cn post, section on the RHT turning point (quantization
  underflow ratio, bucket utilization of E2M1's 15 codes).

Where the pages leave a step open the reading taken here is stated next to
the step.  All "FP32" steps are separate numpy float32 operations (numpy
never contracts a multiply and an add into an FMA); GEMMs run in float64.

Parity status: every function below is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` against closed forms, brute force, an independent
Philox implementation or the pages' worked value.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Grids (paperlayer summary section 2 "FP4 formats"; gist.science technical
# summary: E2M1 has 2 exponent and 1 mantissa bit; the uniform E1M2/INT4 grid
# has equal level spacing).
# ---------------------------------------------------------------------------
GRID_UNIFORM = 0
GRID_E2M1 = 1
GRID_E2M1_MAX2 = 2

# Magnitude levels indexed by the 3-bit magnitude field of the nibble.
#  uniform: the E1M2 magnitude field read as an integer, {0..7}; normalized
#           codebook {-7..7}/7, gmax = 1 (levels scaled by g = 7 below).
#  E2M1:    OCP E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; g = 6.
#  E2M1 range-restricted to max_fpx = 2.0 (paperlayer summary section 5 Q4:
#           the variant keeps only {0, 0.5, 1.0, 1.5, 2.0}): the block absmax
#           maps to 2.0, g = 2; the nibbles are E2M1 bit patterns with a
#           magnitude index of at most 4.
LEVELS = {
    GRID_UNIFORM: np.arange(8, dtype=np.float64),
    GRID_E2M1: np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]),
    GRID_E2M1_MAX2: np.array([0.0, 0.5, 1.0, 1.5, 2.0]),
}
GMAX = {GRID_UNIFORM: 7.0, GRID_E2M1: 6.0, GRID_E2M1_MAX2: 2.0}

ROUND_RTNE = 0
ROUND_SR = 1

AXIS_COLS = 0  # blocks along the contiguous (column) dimension, no transpose
AXIS_ROWS = 1  # blocks along the strided (row) dimension, output transposed
AXIS_ROWS_STACKED = 2  # equal row groups, each transposed on its own, stacked

BLOCK = 16

# ---------------------------------------------------------------------------
# Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
# as 1, 2, 3", SC'11).  Counter-based: output = bijection(counter) keyed by a
# 64-bit key.  Round: two 32x32->64 multiplies of counter words 0 and 2 by the
# published multipliers, cross-xor of the high halves with the other counter
# words and the key; the key is bumped by the published Weyl constants between
# rounds.
# ---------------------------------------------------------------------------
_PHILOX_M0 = np.uint64(0xD2511F53)
_PHILOX_M1 = np.uint64(0xCD9E8D57)
_PHILOX_W0 = 0x9E3779B9
_PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Four output words of Philox4x32 with 10 rounds.

    c0..c3 are uint32 arrays (broadcastable); k0, k1 the two key words.
    Returns a tuple of four uint32 arrays.
    """
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.asarray(c1, dtype=np.uint64)
    c2 = np.asarray(c2, dtype=np.uint64)
    c3 = np.asarray(c3, dtype=np.uint64)
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    for _ in range(10):
        p0 = _PHILOX_M0 * c0          # < 2^64, exact in uint64
        p1 = _PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
        k0 = (k0 + _PHILOX_W0) & 0xFFFFFFFF
        k1 = (k1 + _PHILOX_W1) & 0xFFFFFFFF
    return tuple(w.astype(np.uint32) for w in (c0, c1, c2, c3))


def sr_random_u32(idx, seed: int, stream_id: int):
    """32 random bits for element ``idx`` of a quantized output.

    Reading (the pages do not say how SR draws its randomness): element idx
    takes word (idx & 3) of Philox4x32-10 with key (seed_lo, seed_hi) and
    counter (lo32(idx >> 2), hi32(idx >> 2), stream_id, 0).
    """
    idx = np.asarray(idx, dtype=np.uint64)
    q = idx >> np.uint64(2)
    lo = (q & _MASK32).astype(np.uint32)
    hi = (q >> np.uint64(32)).astype(np.uint32)
    words = philox4x32_10(lo, hi, np.uint32(stream_id), np.uint32(0),
                          seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    sel = (idx & np.uint64(3)).astype(np.int64)
    out = np.choose(sel, words)
    return out.astype(np.uint32)


# ---------------------------------------------------------------------------
# bf16 input
# ---------------------------------------------------------------------------
def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact (the bf16 is the top half)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


# ---------------------------------------------------------------------------
# Random Hadamard transform, size 16
# (paperlayer summary section 2 "Random Hadamard transforms").
# ---------------------------------------------------------------------------
def signs_from_mask(sign_mask: int) -> np.ndarray:
    """Diagonal of the random sign matrix: d_j = -1 iff bit j of the mask is set.

    Reading: one 16-entry sign vector per GEMM, shared by both operands of that
    GEMM and by every block, so that the rotation cancels along the reduction
    dimension.
    """
    return np.array([-1.0 if (sign_mask >> j) & 1 else 1.0 for j in range(16)],
                    dtype=np.float32)


def fwht16(y: np.ndarray) -> np.ndarray:
    """Unnormalized Sylvester-order fast Walsh-Hadamard transform over the last
    axis (length 16), in float32, with a fixed operation order.

    Reading (the pages give no butterfly order): stages h = 1, 2, 4, 8; in each
    stage every pair (i, i + h) with (i & h) == 0 becomes
    (RN(y_i + y_{i+h}), RN(y_i - y_{i+h})).
    """
    y = np.array(y, dtype=np.float32, copy=True)
    assert y.shape[-1] == BLOCK
    for h in (1, 2, 4, 8):
        for i in range(BLOCK):
            if i & h:
                continue
            a = y[..., i].copy()
            b = y[..., i + h].copy()
            y[..., i] = a + b
            y[..., i + h] = a - b
    return y


def rht16(x_blocks: np.ndarray, sign_mask: int) -> np.ndarray:
    """y = (1/4) * H16 * D * x per block of 16 (float32).

    Reading: the 1/4 factor makes the transform orthonormal (the pages call
    RHT norm preserving); it is applied after the butterfly.  The sign flip
    and the 1/4 are exact for inputs that came from bf16.
    """
    d = signs_from_mask(sign_mask)
    y = x_blocks.astype(np.float32) * d
    y = fwht16(y)
    return y * np.float32(0.25)


# ---------------------------------------------------------------------------
# Blocking and padding
# ---------------------------------------------------------------------------
def round_up16(n: int) -> int:
    return (int(n) + 15) // 16 * 16


def padded_offsets(group_offsets) -> np.ndarray:
    """Per-group padded offsets: every group's length rounded up to 16 so that
    no block straddles two groups (reading: the pages are silent on padding)."""
    off = np.asarray(group_offsets, dtype=np.int64)
    counts = np.diff(off)
    return np.concatenate([[0], np.cumsum([round_up16(c) for c in counts])]).astype(np.int64)


def to_blocked_rows(x_f32: np.ndarray, axis: int, group_offsets=None,
                    n_stack: int = 1) -> np.ndarray:
    """Arrange the input so that rows are output rows and the last axis is the
    padded contraction axis K_p; pads with +0.0.

    axis == AXIS_COLS: blocks along the contiguous dim (row-wise quantization);
                       output row i is input row i.
    axis == AXIS_ROWS: blocks along the strided dim; output row j is input
                       column j, and the contraction runs over input rows,
                       padded per group.
    axis == AXIS_ROWS_STACKED: the rows are n_stack equal groups (e.g. expert
                       weights stacked along rows); each is arranged as with
                       AXIS_ROWS and the results are stacked along rows.
    """
    if axis == AXIS_ROWS_STACKED:
        n = x_f32.shape[0] // n_stack
        assert n * n_stack == x_f32.shape[0]
        return np.concatenate([to_blocked_rows(x_f32[e * n:(e + 1) * n], AXIS_ROWS)
                               for e in range(n_stack)], axis=0)
    if axis == AXIS_COLS:
        rows, k = x_f32.shape
        kp = round_up16(k)
        out = np.zeros((rows, kp), dtype=np.float32)
        out[:, :k] = x_f32
        return out
    xt = np.ascontiguousarray(x_f32.T)          # [n_cols, n_rows]
    n_out, n_in = xt.shape
    if group_offsets is None:
        group_offsets = [0, n_in]
    off = np.asarray(group_offsets, dtype=np.int64)
    poff = padded_offsets(off)
    out = np.zeros((n_out, int(poff[-1])), dtype=np.float32)
    for g in range(len(off) - 1):
        c = int(off[g + 1] - off[g])
        out[:, poff[g]:poff[g] + c] = xt[:, off[g]:off[g + 1]]
    return out


# ---------------------------------------------------------------------------
# Rounding onto the grid
# ---------------------------------------------------------------------------
def rtne_index(m: np.ndarray, grid: int) -> np.ndarray:
    """Nearest level index for magnitudes 0 <= m <= g; a tie picks the even
    index (paperlayer summary section 2 "Rounding rules": RTNE is nearest with
    deterministic tie-breaking; reading: ties to the even level index, which
    is IEEE round-half-even for both grids)."""
    L = LEVELS[grid]
    top = len(L) - 1
    m = np.asarray(m, dtype=np.float64)   # float32 values, exact in float64
    lo = np.clip(np.searchsorted(L, m, side="right") - 1, 0, top)
    hi = np.minimum(lo + 1, top)
    dlo = m - L[lo]                      # exact: float32 minus a short level
    dhi = L[hi] - m
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0) & (hi != lo))
    return np.where(pick_hi, hi, lo).astype(np.int64)


def sr_index(m: np.ndarray, grid: int, u32: np.ndarray) -> np.ndarray:
    """Stochastic rounding between the two adjacent levels
    (paperlayer summary section 2 "Rounding rules": unbiased in expectation).

    Reading: lo = largest level <= m, hi = next level; f = (m - lo)/(hi - lo)
    (exact); F = floor(f * 2^32); round up iff u32 < F.  At m = g there is no
    level above and f = 0.
    """
    L = LEVELS[grid]
    top = len(L) - 1
    m = np.asarray(m, dtype=np.float64)
    lo = np.clip(np.searchsorted(L, m, side="right") - 1, 0, top)
    hi = np.minimum(lo + 1, top)
    span = L[hi] - L[lo]
    f = np.where(hi == lo, 0.0, (m - L[lo]) / np.where(span == 0, 1.0, span))
    F = np.floor(f * 4294967296.0).astype(np.uint64)
    up = np.asarray(u32, dtype=np.uint64) < F
    return np.where(up, hi, lo).astype(np.int64)


# ---------------------------------------------------------------------------
# Quantizer
# (paperlayer summary section 2 "Blockwise quantization" + "Random Hadamard
# transforms"; section 4 "UFP4 Recipe")
# ---------------------------------------------------------------------------
_TWO64 = np.float32(2.0 ** 64)
_TINY = np.float32(2.0 ** -64)


def quantize_blocked(xb: np.ndarray, rht: bool, sign_mask: int, grid: int,
                     rnd: int, seed: int = 0, stream_id: int = 0, row_ids=None):
    """Quantize a [rows, K_p] float32 matrix along its last axis.

    row_ids (optional) gives each row's index in the full quantized output,
    so that a subset of rows draws the same SR random bits as in the full
    tensor (SR index = row_id * K_p + k); default 0..rows-1.

    Returns (nibbles int64 [rows, K_p], scales float32 [rows, K_p/16]).

    Steps (per block of 16):
      1. RHT if enabled: y = (1/4) H16 D x.
      2. s = max_j |y_j|, the stored FP32 block scale (absmax).
         s == 0: all codes 0.  0 < s < 2^-64: y and s are multiplied by 2^64
         (exact) for steps 3-4 only, so that g/s cannot overflow (reading).
      3. r = RN32(g / s);  t_j = RN32(y_j * r)  (two roundings, no FMA;
         reading: the pages do not fix the normalization arithmetic).
      4. m = min(|t_j|, g); index by RTNE or SR; nibble = sign<<3 | index with
         sign = (t_j < 0); a zero index always encodes as nibble 0.
    """
    rows, kp = xb.shape
    assert kp % BLOCK == 0
    g = np.float32(GMAX[grid])
    blocks = xb.reshape(rows, kp // BLOCK, BLOCK).astype(np.float32)
    y = rht16(blocks, sign_mask) if rht else blocks.copy()
    s = np.max(np.abs(y), axis=-1)                        # float32, exact
    tiny = (s < _TINY) & (s > 0)
    with np.errstate(over="ignore"):
        y_n = np.where(tiny[..., None], y * _TWO64, y)
        s_n = np.where(tiny, s * _TWO64, s)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s_n > 0, g / np.where(s_n > 0, s_n, np.float32(1)), np.float32(0))
    r = r.astype(np.float32)
    t = (y_n * r[..., None]).astype(np.float32)
    m = np.minimum(np.abs(t), g)
    if rnd == ROUND_RTNE:
        idx = rtne_index(m, grid)
    else:
        rid = (np.arange(rows, dtype=np.uint64) if row_ids is None
               else np.asarray(row_ids, dtype=np.uint64))
        flat = (rid[:, None] * np.uint64(kp) +
                np.arange(kp, dtype=np.uint64)[None, :]).reshape(rows, kp // BLOCK, BLOCK)
        u = sr_random_u32(flat, seed, stream_id)
        idx = sr_index(m, grid, u)
    neg = (t < 0)
    nib = np.where(idx == 0, 0, (neg.astype(np.int64) << 3) | idx)
    return nib.reshape(rows, kp), s.astype(np.float32)


def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """byte j = nib[2j] | nib[2j+1] << 4 (reading: low nibble first)."""
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out


def quantize(x_bits: np.ndarray, axis: int, rht: bool, sign_mask: int,
             grid: int, rnd: int, seed: int = 0, stream_id: int = 0,
             group_offsets=None, kpad=None, out_rows=None, n_stack: int = 1):
    """Full quantizer on bf16 bit patterns [n_rows, n_cols].

    Returns (codes uint8 [rows, K_p/2], scales float32 [rows, K_p/16], K_p).
    SR element index = row * K_p + k in the quantized output's layout
    (reading).

    kpad: a larger padded length than the minimum (columns beyond the data
      are zero blocks), as a caller-sized buffer may have.
    out_rows: evaluate only these output rows (indices into the full output);
      with AXIS_COLS they are input rows, with AXIS_ROWS input columns.  The
      codes equal those rows of the full result.
    """
    x = bf16_bits_to_f32(x_bits)
    if out_rows is not None:
        assert axis != AXIS_ROWS_STACKED
        out_rows = np.asarray(out_rows, dtype=np.int64)
        x = x[out_rows] if axis == AXIS_COLS else x[:, out_rows]
    xb = to_blocked_rows(x, axis, group_offsets, n_stack)
    if kpad is not None and kpad > xb.shape[1]:
        xb = np.concatenate([xb, np.zeros((xb.shape[0], kpad - xb.shape[1]), np.float32)], 1)
    nib, s = quantize_blocked(xb, rht, sign_mask, grid, rnd, seed, stream_id, out_rows)
    return pack_nibbles(nib), s, xb.shape[1]


# ---------------------------------------------------------------------------
# Dequantization (paperlayer summary section 2 "Blockwise quantization": a
# value is its level times the block scale over gmax)
# ---------------------------------------------------------------------------
def dequantize64(codes: np.ndarray, scales: np.ndarray, grid: int) -> np.ndarray:
    """Dequantized values in float64: sign * L[idx] * s / g, shape [rows, K_p]."""
    nib = unpack_nibbles(codes).astype(np.int64)
    L = np.concatenate([LEVELS[grid], np.full(8 - len(LEVELS[grid]), np.nan)])
    mag = L[nib & 7]          # an index past the grid's top level is no code: NaN
    sgn = np.where(nib & 8, -1.0, 1.0)
    rows, kp = nib.shape
    s = np.repeat(np.asarray(scales, dtype=np.float64), BLOCK, axis=-1).reshape(rows, kp)
    return (sgn * mag) * s / GMAX[grid]


def dequantize(codes, scales, grid: int, inverse_rht: bool = False,
               sign_mask: int = 0) -> np.ndarray:
    """FP32 output.  Without inverse RHT each value is
    (float)((double)(sign*L[idx]) * (double)s / g) (reading, fixes the
    rounding).  With inverse RHT the block is mapped back by (1/4) D H16 in
    float64 before the cast (compared within tolerance)."""
    v = dequantize64(codes, scales, grid)
    if inverse_rht:
        rows, kp = v.shape
        H = sylvester_hadamard(4)
        d = signs_from_mask(sign_mask).astype(np.float64)
        vb = v.reshape(rows, kp // BLOCK, BLOCK)
        v = (0.25 * (vb @ H.T) * d).reshape(rows, kp)
    return v.astype(np.float32)


def sylvester_hadamard(log2n: int) -> np.ndarray:
    """H_{2^n} by the Sylvester doubling H_{2n} = [[H, H], [H, -H]] (float64)."""
    H = np.array([[1.0]])
    for _ in range(log2n):
        H = np.block([[H, H], [H, -H]])
    return H


# ---------------------------------------------------------------------------
# GEMMs on dequantized operands (paperlayer summary section 2: the low
# precision GEMM consumes the rotated quantized operands; RHT along the shared
# reduction dimension cancels because (1/4 H D)^T (1/4 H D) = I).
# ---------------------------------------------------------------------------
def gemm_tn(a_codes, a_scales, b_codes, b_scales, grid: int = GRID_UNIFORM):
    """C = A_hat @ B_hat^T in float64, both operands [*, K_p] K-contiguous.
    Returns (C, bound) where bound = |A_hat| @ |B_hat|^T (for the tolerance
    max|err| <= 1e-5 * bound)."""
    A = dequantize64(a_codes, a_scales, grid)
    B = dequantize64(b_codes, b_scales, grid)
    return A @ B.T, np.abs(A) @ np.abs(B).T


def gemm_tn_rows(a_codes, a_scales, b_codes, b_scales, rows, grid: int = GRID_UNIFORM):
    """Same as gemm_tn for a subset of output rows (sampled parity at large
    sizes)."""
    rows = np.asarray(rows, dtype=np.int64)
    A = dequantize64(a_codes[rows], a_scales[rows], grid)
    B = dequantize64(b_codes, b_scales, grid)
    return A @ B.T, np.abs(A) @ np.abs(B).T


def grouped_gemm(kind: int, group_offsets, a_codes, a_scales, b_codes, b_scales,
                 n_out: int, grid: int = GRID_UNIFORM):
    """Expert-grouped GEMM in float64.

    kind 0 (FPROP) / 1 (DGRAD): rows of A are grouped by group_offsets (tokens
      per expert); B stacks the experts' [n_out, K_p] operands; group e writes
      C[off_e:off_{e+1}] = A_e @ B_e^T.
    kind 2 (WGRAD): the contraction is grouped; A [M, K_p] and B [N, K_p] hold
      all groups along K_p with per-group padding to 16; C[e] = A[:, seg_e] @
      B[:, seg_e]^T, zero for an empty group.  Returns (C, bound).
    """
    off = np.asarray(group_offsets, dtype=np.int64)
    E = len(off) - 1
    if kind in (0, 1):
        A = dequantize64(a_codes, a_scales, grid)
        B = dequantize64(b_codes, b_scales, grid)
        C = np.zeros((A.shape[0], n_out))
        bound = np.zeros_like(C)
        for e in range(E):
            Ae = A[off[e]:off[e + 1]]
            Be = B[e * n_out:(e + 1) * n_out]
            C[off[e]:off[e + 1]] = Ae @ Be.T
            bound[off[e]:off[e + 1]] = np.abs(Ae) @ np.abs(Be).T
        return C, bound
    poff = padded_offsets(off)
    A = dequantize64(a_codes, a_scales, grid)
    B = dequantize64(b_codes, b_scales, grid)
    C = np.zeros((E, A.shape[0], B.shape[0]))
    bound = np.zeros_like(C)
    for e in range(E):
        sl = slice(int(poff[e]), int(poff[e + 1]))
        C[e] = A[:, sl] @ B[:, sl].T
        bound[e] = np.abs(A[:, sl]) @ np.abs(B[:, sl]).T
    return C, bound


# ---------------------------------------------------------------------------
# Shrinkage diagnostics
# (gist.science technical summary, "Theoretische Analyse": per-GEMM
# attenuation alpha < 1 that compounds over layers; paperlayer summary
# section 3.1: conditional error of an asymmetric RTNE bin is (l - r)/2 in
# normalized magnitude space.)
# ---------------------------------------------------------------------------
def shrinkage_metrics(x: np.ndarray, xhat: np.ndarray) -> dict:
    """delta_mag = sum(|xhat| - |x|)/sum|x|; one_minus_alpha with
    alpha = <xhat, x>/<x, x> (the attenuation factor a GEMM sees);
    sqnr_db = 10 log10(sum x^2 / sum (xhat - x)^2)."""
    x = np.asarray(x, dtype=np.float64).ravel()
    xh = np.asarray(xhat, dtype=np.float64).ravel()
    ax = np.abs(x).sum()
    ex = (x * x).sum()
    err = ((xh - x) ** 2).sum()
    return {
        "delta_mag": float((np.abs(xh).sum() - ax) / ax),
        "one_minus_alpha": float(1.0 - (xh * x).sum() / ex),
        "sqnr_db": float(10.0 * np.log10(ex / err)) if err > 0 else float("inf"),
    }


def conditional_level_bias(m: np.ndarray, idx: np.ndarray, grid: int) -> dict:
    """Mean of (L[idx] - m) conditioned on the chosen level, in normalized
    magnitude units (the quantity of paperlayer summary section 3.1)."""
    L = LEVELS[grid]
    m = np.asarray(m, dtype=np.float64).ravel()
    idx = np.asarray(idx).ravel()
    out = {}
    for i in range(8):
        sel = idx == i
        if sel.any():
            out[float(L[i])] = (float(np.mean(L[i] - m[sel])), int(sel.sum()),
                                float(np.std(L[i] - m[sel])))
    return out


# ---------------------------------------------------------------------------
# Diagnostics (paperlayer summary section 3.2, section 5 Q1 and appendix A:
# tensor and GEMM-output SQNR and its change under RHT, bucket utilization;
# gist.science technical summary: the attenuation factor alpha of a GEMM;
# dreamwings.cn post, "RHT turning point": the quantization underflow ratio
# and the use of E2M1's 15 buckets).  Readings (the pages give no formulas):
#   * every sum runs over the tensor's logical elements (padding excluded),
#     pairing each input x with its dequantized value xhat in the input's own
#     domain: the dequantized block goes back through (1/4) D H16 in float64
#     when the quantization used the RHT;
#   * SQNR = 10 log10(sum x^2 / sum (xhat - x)^2), alpha = <xhat, x>/<x, x>,
#     delta_mag = (sum |xhat| - sum |x|) / sum |x|;
#   * underflow: an element whose pre-rounding value y (after the RHT, as the
#     quantizer computes it in FP32) is nonzero but whose magnitude index is
#     0; the ratio is over the elements with y != 0;
#   * bucket utilization: exp(H)/15 with H the entropy (natural log) of the
#     empirical distribution of the 15 signed codes -- 1 when all codes are
#     equally used, 1/15 when one is; the raw 16-bin nibble histogram is kept.
# ---------------------------------------------------------------------------
STAT_KEYS = ("sum_x2", "sum_err2", "sum_x_xhat", "sum_abs_x", "sum_abs_xhat")


def quant_stats(x_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, axis: int,
                rht: bool, sign_mask: int, grid: int) -> dict:
    """Sums and counts comparing bf16 input x [n_rows, n_cols] with its
    quantization (codes, scales) along `axis` (AXIS_COLS or AXIS_ROWS, one
    group)."""
    assert axis in (AXIS_COLS, AXIS_ROWS)
    x = bf16_bits_to_f32(x_bits)
    kvalid = x.shape[1] if axis == AXIS_COLS else x.shape[0]
    xb = to_blocked_rows(x, axis)                       # [rows, K_p] FP32, zero padded
    rows, kp = xb.shape
    blocks = xb.reshape(rows, kp // BLOCK, BLOCK)
    y = (rht16(blocks, sign_mask) if rht else blocks).reshape(rows, kp)
    v = dequantize64(codes, scales, grid)
    if rht:
        H = sylvester_hadamard(4)
        d = signs_from_mask(sign_mask).astype(np.float64)
        v = (0.25 * (v.reshape(rows, kp // BLOCK, BLOCK) @ H.T) * d).reshape(rows, kp)
    keep = np.arange(kp) < kvalid
    x64 = xb.astype(np.float64)[:, keep]
    xh = v[:, keep]
    nib = unpack_nibbles(codes)[:, keep]
    yk = y[:, keep]
    nz = yk != 0
    return {
        "sum_x2": float((x64 * x64).sum()),
        "sum_err2": float(((xh - x64) ** 2).sum()),
        "sum_x_xhat": float((x64 * xh).sum()),
        "sum_abs_x": float(np.abs(x64).sum()),
        "sum_abs_xhat": float(np.abs(xh).sum()),
        "n_elems": int(x64.size),
        "n_nonzero": int(nz.sum()),
        "n_underflow": int((nz & ((nib & 7) == 0)).sum()),
        "hist": np.bincount(nib.ravel(), minlength=16).astype(np.int64),
    }


def output_stats(ref: np.ndarray, test: np.ndarray) -> dict:
    """The same sums for a GEMM output `test` against its reference `ref`
    (x -> ref, xhat -> test); counts other than n_elems are zero."""
    r = np.asarray(ref, dtype=np.float64)
    t = np.asarray(test, dtype=np.float64)
    return {
        "sum_x2": float((r * r).sum()),
        "sum_err2": float(((t - r) ** 2).sum()),
        "sum_x_xhat": float((r * t).sum()),
        "sum_abs_x": float(np.abs(r).sum()),
        "sum_abs_xhat": float(np.abs(t).sum()),
        "n_elems": int(r.size),
        "n_nonzero": 0,
        "n_underflow": 0,
        "hist": np.zeros(16, dtype=np.int64),
    }


def stats_summary(st: dict) -> dict:
    """Derived metrics of a quant_stats / output_stats result."""
    out = {
        "sqnr_db": (float(10.0 * np.log10(st["sum_x2"] / st["sum_err2"]))
                    if st["sum_err2"] > 0 else float("inf")),
        "one_minus_alpha": float(1.0 - st["sum_x_xhat"] / st["sum_x2"]),
        "delta_mag": float((st["sum_abs_xhat"] - st["sum_abs_x"]) / st["sum_abs_x"]),
        "underflow_ratio": (st["n_underflow"] / st["n_nonzero"]) if st["n_nonzero"] else 0.0,
    }
    h = np.asarray(st["hist"], dtype=np.float64).copy()
    h[0] += h[8]          # +0 and -0 are one bucket (the quantizer never emits -0)
    h[8] = 0.0
    tot = h.sum()
    if tot > 0:
        p = h[h > 0] / tot
        out["bucket_utilization"] = float(np.exp(-(p * np.log(p)).sum()) / 15.0)
    else:
        out["bucket_utilization"] = 0.0
    return out
