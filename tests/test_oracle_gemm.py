"""Pins for the oracle's GEMMs on dequantized operands.

The three training GEMMs (paperlayer.ai summary of arXiv 2606.20381,
section 2 "Random Hadamard transforms" and section 3.2) contract along the
dimension the operands were quantized and rotated along; the oracle is a
float64 matrix product of the dequantized operands.  Pins: a brute-force
scalar sum over codes on tiny shapes, the grouped form against per-group
dense products, and the rotation cancelling up to quantization noise.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import ufp4_oracle as O


def rand_bits(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("grid", [O.GRID_UNIFORM, O.GRID_E2M1, O.GRID_E2M1_MAX2])
def test_gemm_equals_brute_force_sum_over_codes(grid):
    rng = np.random.default_rng(200)
    a = rand_bits(rng, (3, 40))
    b = rand_bits(rng, (4, 40))
    ca, sa, kp = O.quantize(a, O.AXIS_COLS, True, 0x1357, grid, O.ROUND_RTNE)
    cb, sb, _ = O.quantize(b, O.AXIS_COLS, True, 0x1357, grid, O.ROUND_RTNE)
    C, bound = O.gemm_tn(ca, sa, cb, sb, grid)
    assert kp == 48 and C.shape == (3, 4)
    L = [Fraction(v).limit_denominator(4) for v in O.LEVELS[grid]]
    g = int(O.GMAX[grid])

    def val(codes, scales, i, k):
        byte = int(codes[i, k // 2])
        n = (byte >> 4) if k % 2 else (byte & 0xF)
        return (-1 if n & 8 else 1) * L[n & 7] * Fraction(float(scales[i, k // 16])) / g

    for i in range(3):
        for j in range(4):
            exact = sum(val(ca, sa, i, k) * val(cb, sb, j, k) for k in range(kp))
            babs = sum(abs(val(ca, sa, i, k) * val(cb, sb, j, k)) for k in range(kp))
            assert abs(C[i, j] - float(exact)) <= 1e-13 * float(babs)
            assert abs(bound[i, j] - float(babs)) <= 1e-13 * float(babs)


def test_quantized_fprop_with_rht_matches_unrotated_product_to_noise_level():
    rng = np.random.default_rng(201)
    M, N, K = 64, 64, 1024
    a = rand_bits(rng, (M, K))
    b = rand_bits(rng, (N, K))
    af = O.bf16_bits_to_f32(a).astype(np.float64)
    bf = O.bf16_bits_to_f32(b).astype(np.float64)
    exact = af @ bf.T
    for rht in (False, True):
        ca, sa, _ = O.quantize(a, O.AXIS_COLS, rht, 0xC0DE, O.GRID_UNIFORM, O.ROUND_RTNE)
        cb, sb, _ = O.quantize(b, O.AXIS_COLS, rht, 0xC0DE, O.GRID_UNIFORM, O.ROUND_RTNE)
        C, _ = O.gemm_tn(ca, sa, cb, sb)
        err = C - exact
        # quantization noise: per element step s/7, error ~ U(-step/2, step/2);
        # product noise variance ~ K * (E|a|^2 var(eb) + E|b|^2 var(ea))
        step_a = np.repeat(sa, 16, axis=1) / 7.0
        step_b = np.repeat(sb, 16, axis=1) / 7.0
        pred = np.sqrt(((af ** 2) @ (step_b ** 2 / 12).T) + ((step_a ** 2 / 12) @ (bf ** 2).T))
        z = err / pred
        assert abs(z.mean()) < 5 / np.sqrt(z.size) * 1.5
        assert 0.5 < z.std() < 1.5
        assert np.abs(z).max() < 6


def test_grouped_forward_matches_dense_per_group_and_zero_groups():
    rng = np.random.default_rng(202)
    counts = [5, 0, 17, 1, 0, 9]
    off = np.concatenate([[0], np.cumsum(counts)])
    T, H, F, E = int(off[-1]), 48, 24, len(counts)
    x = rand_bits(rng, (T, H))
    w = rand_bits(rng, (E * F, H), 0.02)
    cx, sx, _ = O.quantize(x, O.AXIS_COLS, True, 7, O.GRID_UNIFORM, O.ROUND_RTNE)
    cw, sw, _ = O.quantize(w, O.AXIS_COLS, True, 7, O.GRID_UNIFORM, O.ROUND_RTNE)
    C, bound = O.grouped_gemm(0, off, cx, sx, cw, sw, F)
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        Ce, be = O.gemm_tn(cx[rows], sx[rows], cw[e * F:(e + 1) * F], sw[e * F:(e + 1) * F])
        assert (C[rows] == Ce).all() and (bound[rows] == be).all()


def test_grouped_weight_gradient_over_padded_segments():
    rng = np.random.default_rng(203)
    counts = [5, 0, 17, 16, 3]
    off = np.concatenate([[0], np.cumsum(counts)])
    T, H, F = int(off[-1]), 32, 16
    x = rand_bits(rng, (T, H))
    dy = rand_bits(rng, (T, F), 1e-4)
    cdy, sdy, kp = O.quantize(dy, O.AXIS_ROWS, True, 9, O.GRID_UNIFORM, O.ROUND_SR, 3, 1, off)
    cx, sx, kp2 = O.quantize(x, O.AXIS_ROWS, True, 9, O.GRID_UNIFORM, O.ROUND_RTNE, 0, 0, off)
    assert kp == kp2 == 16 + 0 + 32 + 16 + 16
    C, bound = O.grouped_gemm(2, off, cdy, sdy, cx, sx, 0)
    assert C.shape == (5, F, H)
    assert (C[1] == 0).all() and (bound[1] == 0).all()
    # each group equals the quantize-then-GEMM of that group alone
    poff = O.padded_offsets(off)
    for e in (0, 2, 3, 4):
        ce, se, _ = O.quantize(dy[off[e]:off[e + 1]], O.AXIS_ROWS, True, 9, O.GRID_UNIFORM,
                               O.ROUND_RTNE, 0, 0)
        cxe, sxe, _ = O.quantize(x[off[e]:off[e + 1]], O.AXIS_ROWS, True, 9, O.GRID_UNIFORM,
                                 O.ROUND_RTNE, 0, 0)
        A = O.dequantize64(cx, sx, O.GRID_UNIFORM)[:, poff[e]:poff[e + 1]]
        assert np.array_equal(A, O.dequantize64(cxe, sxe, O.GRID_UNIFORM))
        D = O.dequantize64(cdy, sdy, O.GRID_UNIFORM)[:, poff[e]:poff[e + 1]]
        assert np.allclose(C[e], D @ A.T, rtol=0, atol=0)


def test_wgrad_sr_uses_the_output_layout_index():
    """SR element index is row * K_p + k of the transposed output."""
    rng = np.random.default_rng(204)
    dy = rand_bits(rng, (48, 8), 1e-4)
    c1, s1, kp = O.quantize(dy, O.AXIS_ROWS, False, 0, O.GRID_UNIFORM, O.ROUND_SR, 5, 1)
    yt = O.bf16_bits_to_f32(dy).T.copy()            # [8, 48]
    c2, s2, _ = O.quantize((yt.view(np.uint32) >> 16).astype(np.uint16), O.AXIS_COLS, False, 0,
                           O.GRID_UNIFORM, O.ROUND_SR, 5, 1)
    assert kp == 48 and (c1 == c2).all() and (s1 == s2).all()
