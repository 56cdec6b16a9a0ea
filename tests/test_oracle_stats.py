"""Pins of the oracle's diagnostics (quant_stats, output_stats,
stats_summary) against closed forms and brute force written out from the
definitions: exact quantization of on-grid tensors, a hand-built underflow
block, element-by-element loops with the Sylvester matrix from its
(-1)^popcount(i & j) definition, and the entropy closed forms of the bucket
utilization."""
import itertools
import math

import numpy as np
import pytest

from oracle import ufp4_oracle as O


def to_bits(x):
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32) >> 16
    assert np.array_equal((bits << 16).view(np.float32), x), "inputs must be exact in bf16"
    return bits.astype(np.uint16)


LEVELS = {0: [0, 1, 2, 3, 4, 5, 6, 7], 1: [0, 0.5, 1, 1.5, 2, 3, 4, 6]}
G = {0: 7.0, 1: 6.0}


@pytest.mark.parametrize("grid", [0, 1])
@pytest.mark.parametrize("axis", [O.AXIS_COLS, O.AXIS_ROWS])
def test_on_grid_tensor_is_exact(grid, axis):
    rng = np.random.default_rng(1)
    L = np.array(LEVELS[grid])
    rows, k = 6, 48
    idx = rng.integers(0, 8, size=(rows, k))
    sgn = rng.choice([-1.0, 1.0], size=(rows, k))
    idx[:, ::16] = 7                      # every block reaches the top level
    scale = 2.0 ** rng.integers(-20, 20, size=(rows, k // 16))
    x = sgn * L[idx] * np.repeat(scale, 16, axis=1)
    x = x if axis == O.AXIS_COLS else x.T
    bits = to_bits(x)
    codes, scales, _ = O.quantize(bits, axis, False, 0, grid, O.ROUND_RTNE)
    st = O.quant_stats(bits, codes, scales, axis, False, 0, grid)
    xx = np.asarray(x, dtype=np.float64)
    assert st["sum_err2"] == 0.0
    assert st["sum_x_xhat"] == st["sum_x2"] == float((xx * xx).sum())
    assert st["sum_abs_xhat"] == st["sum_abs_x"]
    assert st["n_elems"] == rows * k
    assert st["n_underflow"] == 0 and st["n_nonzero"] == int((idx != 0).sum())
    nib = np.where(idx == 0, 0, idx + 8 * (sgn < 0))
    assert np.array_equal(st["hist"], np.bincount(nib.ravel(), minlength=16))
    sm = O.stats_summary(st)
    assert sm["sqnr_db"] == math.inf and sm["one_minus_alpha"] == 0.0 and sm["delta_mag"] == 0.0


def test_underflow_of_a_dominated_block():
    x = np.array([[100.0] + [2.0 ** -10] * 15 + [0.0] * 15 + [1.0]], dtype=np.float32)
    bits = to_bits(x)
    codes, scales, _ = O.quantize(bits, O.AXIS_COLS, False, 0, O.GRID_UNIFORM, O.ROUND_RTNE)
    st = O.quant_stats(bits, codes, scales, O.AXIS_COLS, False, 0, O.GRID_UNIFORM)
    # block 0: 15 tiny values under a 100 -> index 0; block 1: 15 zeros (y == 0) and 1.0
    assert st["n_nonzero"] == 17 and st["n_underflow"] == 15
    assert O.stats_summary(st)["underflow_ratio"] == 15 / 17
    assert st["hist"][0] == 30 and st["hist"][7] == 2


def brute_force(x, codes, scales, axis, rht, mask, grid):
    """Element-by-element sums from the definitions (small integer inputs,
    so the FP32 butterfly of the quantizer is exact and y != 0 is decided
    the same way)."""
    x = np.asarray(x, dtype=np.float64)
    if axis == O.AXIS_ROWS:
        x = x.T
    rows, k = x.shape
    d = [-1.0 if (mask >> j) & 1 else 1.0 for j in range(16)]
    H = [[(-1.0) ** bin(i & j).count("1") for j in range(16)] for i in range(16)]
    acc = dict(sum_x2=0.0, sum_err2=0.0, sum_x_xhat=0.0, sum_abs_x=0.0, sum_abs_xhat=0.0)
    n_nz = n_uf = 0
    hist = [0] * 16
    for r in range(rows):
        for kb in range((k + 15) // 16):
            xs = [x[r, 16 * kb + j] if 16 * kb + j < k else 0.0 for j in range(16)]
            nibs = []
            for j in range(16):
                byte = int(codes[r, (16 * kb + j) // 2])
                nibs.append((byte >> 4) if j % 2 else (byte & 15))
            s = float(scales[r, kb])
            yhat = [(-1.0 if n & 8 else 1.0) * LEVELS[grid][n & 7] * s / G[grid] for n in nibs]
            if rht:
                xhat = [0.25 * d[i] * sum(H[i][j] * yhat[j] for j in range(16)) for i in range(16)]
                y = [sum(H[i][j] * d[j] * xs[j] for j in range(16)) for i in range(16)]
            else:
                xhat, y = yhat, xs
            for j in range(16):
                if 16 * kb + j >= k:
                    continue
                xv, hv = xs[j], xhat[j]
                acc["sum_x2"] += xv * xv
                acc["sum_err2"] += (hv - xv) ** 2
                acc["sum_x_xhat"] += xv * hv
                acc["sum_abs_x"] += abs(xv)
                acc["sum_abs_xhat"] += abs(hv)
                hist[nibs[j]] += 1
                if y[j] != 0:
                    n_nz += 1
                    n_uf += (nibs[j] & 7) == 0
    return acc, n_nz, n_uf, hist


@pytest.mark.parametrize("grid,rht,axis", list(itertools.product([0, 1], [False, True],
                                                                  [O.AXIS_COLS, O.AXIS_ROWS])))
def test_brute_force(grid, rht, axis):
    rng = np.random.default_rng(7 + grid + 2 * rht + 4 * axis)
    x = rng.integers(-8, 9, size=(3, 37)).astype(np.float32)
    x[1, :16] = 0.0
    x[2, 16:20] = 96.0                                 # forces underflow in that block
    if axis == O.AXIS_ROWS:
        x = np.ascontiguousarray(x.T)
    bits = to_bits(x)
    mask = 0xB3C5
    for rnd in (O.ROUND_RTNE, O.ROUND_SR):
        codes, scales, _ = O.quantize(bits, axis, rht, mask, grid, rnd, seed=3)
        st = O.quant_stats(bits, codes, scales, axis, rht, mask, grid)
        acc, n_nz, n_uf, hist = brute_force(x, codes, scales, axis, rht, mask, grid)
        for key in O.STAT_KEYS:
            assert st[key] == pytest.approx(acc[key], rel=1e-12, abs=1e-12), key
        assert (st["n_nonzero"], st["n_underflow"]) == (n_nz, n_uf)
        assert list(st["hist"]) == hist
        assert st["n_elems"] == x.size


def test_error_identity_and_symmetry():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((40, 96)) * 3).astype(np.float32)
    x = np.concatenate([x, -x], axis=0)               # every value and its negation
    bits = to_bits((x.view(np.uint32) & 0xFFFF0000).view(np.float32))
    codes, scales, _ = O.quantize(bits, O.AXIS_COLS, True, 0x0F0F, 0, O.ROUND_RTNE)
    st = O.quant_stats(bits, codes, scales, O.AXIS_COLS, True, 0x0F0F, 0)
    xh = O.dequantize(codes, scales, 0, True, 0x0F0F).astype(np.float64)
    # sum (xh - x)^2 = sum x^2 - 2 <x, xh> + sum xh^2  (xh from the FP32 API path)
    ssq = float((xh * xh).sum())
    assert st["sum_err2"] == pytest.approx(st["sum_x2"] - 2 * st["sum_x_xhat"] + ssq, rel=1e-5)
    # negating the input mirrors the histogram (nibble i <-> i ^ 8, zero stays)
    h = st["hist"]
    assert all(h[i] == h[i ^ 8] for i in range(1, 8))


def test_bucket_utilization_closed_forms():
    base = dict(sum_x2=1.0, sum_err2=1.0, sum_x_xhat=1.0, sum_abs_x=1.0, sum_abs_xhat=1.0,
                n_elems=0, n_nonzero=0, n_underflow=0)
    h = np.ones(16, np.int64) * 5
    h[8] = 0
    assert O.stats_summary(dict(base, hist=h))["bucket_utilization"] == pytest.approx(1.0)
    h = np.zeros(16, np.int64)
    h[3] = 9
    assert O.stats_summary(dict(base, hist=h))["bucket_utilization"] == pytest.approx(1 / 15)
    h = np.zeros(16, np.int64)
    h[1] = h[9] = 4
    assert O.stats_summary(dict(base, hist=h))["bucket_utilization"] == pytest.approx(2 / 15)


def test_output_stats_closed_form():
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((17, 33))
    for eps in (1e-3, -2e-2):
        st = O.output_stats(ref, ref * (1 + eps))
        sm = O.stats_summary(st)
        assert sm["sqnr_db"] == pytest.approx(-20 * math.log10(abs(eps)), rel=1e-9)
        assert sm["one_minus_alpha"] == pytest.approx(-eps, rel=1e-9)
        assert sm["delta_mag"] == pytest.approx(eps, rel=1e-9)
