"""Pins for the oracle's blockwise absmax quantizer, grids and encoding.

Sources: paperlayer.ai summary of arXiv 2606.20381, section 2 "FP4 formats",
"Blockwise quantization", "Rounding rules"; section 5 "Q4: Recipe ablations"
(E2M1 magnitudes up to 2 are {0, 0.5, 1.0, 1.5, 2.0}); section 3.1 (the
neighbours of level 2 on E2M1 are 1.5 and 3).
"""
import numpy as np
import pytest

from oracle import ufp4_oracle as O


def to_bits(x):
    """float32 values that are exact in bf16 -> bf16 bit patterns."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert ((b & 0xFFFF) == 0).all(), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def brute_nearest_index(m, levels):
    """Independent nearest-level search: distances to all levels, the smallest
    wins, and between two equally near levels the even index wins."""
    m = np.asarray(m, dtype=np.float64)[:, None]
    L = np.asarray(levels, dtype=np.float64)[None, :]
    d = np.abs(m - L)
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    n_cand = cand.sum(axis=1)
    first = cand.argmax(axis=1)
    even_pick = np.where(cand & (np.arange(L.shape[1])[None, :] % 2 == 0), 1, 0).argmax(axis=1)
    return np.where(n_cand == 1, first, even_pick)


def test_e2m1_levels_match_pages():
    L = O.LEVELS[O.GRID_E2M1]
    assert list(L[L <= 2.0]) == [0.0, 0.5, 1.0, 1.5, 2.0]
    i2 = list(L).index(2.0)
    assert L[i2 - 1] == 1.5 and L[i2 + 1] == 3.0
    assert O.GMAX[O.GRID_E2M1] == 6.0


def test_uniform_levels_equally_spaced():
    L = O.LEVELS[O.GRID_UNIFORM]
    assert (np.diff(L) == 1.0).all() and O.GMAX[O.GRID_UNIFORM] == 7.0


@pytest.mark.parametrize("e", [-133, -126, -100, -70, -64, -30, -3, 0, 5, 60, 118])
def test_uniform_grid_round_trip(e):
    rng = np.random.default_rng(10 + abs(e))
    k = rng.integers(-7, 8, size=(64, 32))
    k[:, 0] = np.where(rng.random(64) < 0.5, 7, -7)
    k[:, 16] = 7
    x = (k * 2.0 ** e).astype(np.float32)
    if e < -126 + 3:   # bf16 subnormals still hold 7 * 2^e down to 2^-133 * 7
        assert (x != 0).any()
    codes, scales, kp = O.quantize(to_bits(x), O.AXIS_COLS, False, 0, O.GRID_UNIFORM, O.ROUND_RTNE)
    assert kp == 32
    nib = O.unpack_nibbles(codes).astype(np.int64)
    expect = np.where(k == 0, 0, ((k < 0).astype(np.int64) << 3) | np.abs(k))
    assert (nib == expect).all()
    assert (scales == np.float32(7 * 2.0 ** e)).all()


@pytest.mark.parametrize("e", [-130, -80, -10, 0, 7, 100])
def test_e2m1_grid_round_trip(e):
    L = O.LEVELS[O.GRID_E2M1]
    rng = np.random.default_rng(20 + abs(e))
    i = rng.integers(0, 8, size=(64, 16))
    sgn = np.where(rng.random((64, 16)) < 0.5, -1, 1)
    i[:, 3] = 7
    x = (sgn * L[i] * 2.0 ** e).astype(np.float32)
    codes, scales, _ = O.quantize(to_bits(x), O.AXIS_COLS, False, 0, O.GRID_E2M1, O.ROUND_RTNE)
    nib = O.unpack_nibbles(codes).astype(np.int64)
    expect = np.where(i == 0, 0, ((sgn < 0).astype(np.int64) << 3) | i)
    assert (nib == expect).all()
    assert (scales == np.float32(6 * 2.0 ** e)).all()


ALL_GRIDS = [O.GRID_UNIFORM, O.GRID_E2M1, O.GRID_E2M1_MAX2]


def test_range_restricted_e2m1_levels_match_pages():
    # section 5 Q4: the max_fpx = 2.0 variant keeps only {0, 0.5, 1.0, 1.5, 2.0}
    L = O.LEVELS[O.GRID_E2M1_MAX2]
    assert list(L) == [0.0, 0.5, 1.0, 1.5, 2.0] and O.GMAX[O.GRID_E2M1_MAX2] == 2.0
    full = O.LEVELS[O.GRID_E2M1]
    assert list(L) == list(full[full <= 2.0])      # the same E2M1 bit patterns


@pytest.mark.parametrize("e", [-130, -80, 0, 100])
def test_range_restricted_e2m1_round_trip(e):
    L = O.LEVELS[O.GRID_E2M1_MAX2]
    rng = np.random.default_rng(25 + abs(e))
    i = rng.integers(0, 5, size=(64, 16))
    sgn = np.where(rng.random((64, 16)) < 0.5, -1, 1)
    i[:, 5] = 4
    x = (sgn * L[i] * 2.0 ** e).astype(np.float32)
    codes, scales, _ = O.quantize(to_bits(x), O.AXIS_COLS, False, 0, O.GRID_E2M1_MAX2,
                                  O.ROUND_RTNE)
    nib = O.unpack_nibbles(codes).astype(np.int64)
    expect = np.where(i == 0, 0, ((sgn < 0).astype(np.int64) << 3) | i)
    assert (nib == expect).all() and (nib & 7).max() == 4
    assert (scales == np.float32(2 * 2.0 ** e)).all()


@pytest.mark.parametrize("grid", ALL_GRIDS)
def test_rtne_matches_brute_force(grid):
    L = O.LEVELS[grid]
    g = np.float32(O.GMAX[grid])
    mids = ((L[:-1] + L[1:]) / 2).astype(np.float32)
    pts = [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(10)),
           L.astype(np.float32), np.nextafter(L.astype(np.float32), np.float32(10))]
    rng = np.random.default_rng(30 + grid)
    pts.append((rng.random(2_000_000) * float(g)).astype(np.float32))
    m = np.minimum(np.concatenate(pts), g)
    assert (O.rtne_index(m, grid) == brute_nearest_index(m, L)).all()


def test_rtne_ties_go_to_even_index():
    # uniform: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, 6.5 -> 6
    u = O.rtne_index(np.array([0.5, 1.5, 2.5, 6.5], np.float32), O.GRID_UNIFORM)
    assert list(u) == [0, 2, 2, 6]
    # E2M1 ties: 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2.0, 2.5->2, 3.5->4, 5->4
    e = O.rtne_index(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32), O.GRID_E2M1)
    assert list(O.LEVELS[O.GRID_E2M1][e]) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    r = O.rtne_index(np.array([0.25, 0.75, 1.25, 1.75, 2.0], np.float32), O.GRID_E2M1_MAX2)
    assert list(O.LEVELS[O.GRID_E2M1_MAX2][r]) == [0.0, 1.0, 1.0, 2.0, 2.0]


@pytest.mark.parametrize("grid", ALL_GRIDS)
def test_every_bf16_value_in_a_block_with_unit_normalization(grid):
    """Block [x, g, 0, ...]: the scale is g so r = 1 and t = x exactly; the code
    of x must be the brute-force nearest level of |x| with x's sign.  Runs over
    every finite bf16 pattern with |x| <= g."""
    g = O.GMAX[grid]
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    xs = O.bf16_bits_to_f32(allb)
    keep = np.isfinite(xs) & (np.abs(xs) <= g)
    xs = xs[keep]
    n = xs.size
    blk = np.zeros((n, 16), np.float32)
    blk[:, 0] = xs
    blk[:, 1] = g
    codes, scales, _ = O.quantize(to_bits(blk), O.AXIS_COLS, False, 0, grid, O.ROUND_RTNE)
    assert (scales[:, 0] == np.float32(g)).all()
    nib = O.unpack_nibbles(codes)[:, 0].astype(np.int64)
    idx = brute_nearest_index(np.abs(xs), O.LEVELS[grid])
    expect = np.where(idx == 0, 0, ((xs < 0).astype(np.int64) << 3) | idx)
    assert (nib == expect).all()


def test_nibble_packing_low_first():
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 7.0     # code 7
    x[0, 1] = -3.0    # code 8 | 3 = 0xB
    x[0, 2] = -1.0    # 0x9
    codes, scales, _ = O.quantize(to_bits(x), O.AXIS_COLS, False, 0, O.GRID_UNIFORM, O.ROUND_RTNE)
    assert codes.shape == (1, 8)
    assert codes[0, 0] == (0x7 | (0xB << 4))
    assert codes[0, 1] == 0x9
    assert (codes[0, 2:] == 0).all() and scales[0, 0] == 7.0


def test_zero_block_and_negative_zero():
    x = np.zeros((2, 16), np.float32)
    x[1, :] = -0.0
    x[1, 5] = -2.0 ** -10     # rounds to level 0 in a block whose max is 1
    x[1, 6] = 1.0
    codes, scales, _ = O.quantize(to_bits(x), O.AXIS_COLS, False, 0, O.GRID_UNIFORM, O.ROUND_RTNE)
    assert (codes[0] == 0).all() and scales[0, 0] == 0.0
    nib = O.unpack_nibbles(codes)[1]
    assert nib[5] == 0 and nib[6] == 7 and (np.delete(nib, 6) == 0).all()


@pytest.mark.parametrize("rht", [False, True])
@pytest.mark.parametrize("grid", ALL_GRIDS)
def test_codes_invariant_under_power_of_two_scaling(rht, grid):
    """Absmax scaling makes codes invariant under exact power-of-two scaling
    of a block; the tiny-scale branch (s < 2^-64) must keep that property."""
    rng = np.random.default_rng(40)
    x = rng.standard_normal((200, 64)).astype(np.float32)
    b0 = (x.view(np.uint32) >> 16).astype(np.uint16)
    x0 = O.bf16_bits_to_f32(b0)
    c0, s0, _ = O.quantize(b0, O.AXIS_COLS, rht, 0x5A5A, grid, O.ROUND_RTNE)
    for e in (-100, -70, -40, 40, 100):
        xe = (x0.astype(np.float64) * 2.0 ** e).astype(np.float32)
        ce, se, _ = O.quantize(to_bits(xe), O.AXIS_COLS, rht, 0x5A5A, grid, O.ROUND_RTNE)
        assert (ce == c0).all(), e
        assert (se == (s0.astype(np.float64) * 2.0 ** e).astype(np.float32)).all()


def test_padding_and_column_wise_blocking_with_groups():
    x = np.arange(21 * 3, dtype=np.float32).reshape(21, 3) + 1
    off = [0, 5, 5, 21]       # group of 5, an empty group, a group of 16
    assert list(O.padded_offsets(off)) == [0, 16, 16, 32]
    xb = O.to_blocked_rows(x, O.AXIS_ROWS, off)
    assert xb.shape == (3, 32)
    assert (xb[:, :5] == x[:5].T).all() and (xb[:, 5:16] == 0).all()
    assert (xb[:, 16:32] == x[5:21].T).all()
    xr = O.to_blocked_rows(x, O.AXIS_COLS)
    assert xr.shape == (21, 16) and (xr[:, :3] == x).all() and (xr[:, 3:] == 0).all()


def test_dequantize_values():
    from fractions import Fraction
    rng = np.random.default_rng(50)
    x = rng.standard_normal((8, 32)).astype(np.float32)
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    for grid in ALL_GRIDS:
        codes, scales, _ = O.quantize(b, O.AXIS_COLS, True, 0x00FF, grid, O.ROUND_RTNE)
        v = O.dequantize(codes, scales, grid)
        nib = O.unpack_nibbles(codes)
        for (i, j) in [(0, 0), (3, 17), (7, 31), (5, 8)]:
            n = int(nib[i, j])
            lev = Fraction(O.LEVELS[grid][n & 7]).limit_denominator(4)
            exact = (-1 if n & 8 else 1) * lev * Fraction(float(scales[i, j // 16])) / int(O.GMAX[grid])
            assert float(v[i, j]) == float(np.float32(float(exact)))


@pytest.mark.parametrize("axis", [O.AXIS_COLS, O.AXIS_ROWS])
@pytest.mark.parametrize("rnd", [O.ROUND_RTNE, O.ROUND_SR])
def test_row_subset_equals_rows_of_full_result(axis, rnd):
    rng = np.random.default_rng(60)
    x = rng.standard_normal((48, 40)).astype(np.float32)
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    cf, sf, kp = O.quantize(b, axis, True, 0x2468, O.GRID_UNIFORM, rnd, 9, 2)
    rows = [0, 3, 17, cf.shape[0] - 1]
    cs, ss, kp2 = O.quantize(b, axis, True, 0x2468, O.GRID_UNIFORM, rnd, 9, 2, out_rows=rows)
    assert kp == kp2 and (cs == cf[rows]).all() and (ss == sf[rows]).all()
    # a larger caller-sized kpad only appends zero blocks
    ck, sk, kp3 = O.quantize(b, axis, True, 0x2468, O.GRID_UNIFORM, rnd, 9, 2, kpad=kp + 32)
    assert kp3 == kp + 32 and (sk[:, -2:] == 0).all() and (ck[:, -16:] == 0).all()
    if rnd == O.ROUND_RTNE:
        assert (ck[:, :kp // 2] == cf).all()


def test_stacked_axis_equals_per_group_transposes():
    rng = np.random.default_rng(61)
    x = rng.standard_normal((3 * 40, 24)).astype(np.float32)
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    for rnd in (O.ROUND_RTNE, O.ROUND_SR):
        cs, ss, kp = O.quantize(b, O.AXIS_ROWS_STACKED, True, 0x0A0A, O.GRID_UNIFORM, rnd, 4, 1,
                                n_stack=3)
        assert cs.shape == (3 * 24, 24) and kp == 48
        for e in range(3):
            rows = slice(e * 24, (e + 1) * 24)
            if rnd == O.ROUND_RTNE:
                ce, se, _ = O.quantize(b[e * 40:(e + 1) * 40], O.AXIS_ROWS, True, 0x0A0A,
                                       O.GRID_UNIFORM, rnd)
                assert (cs[rows] == ce).all() and (ss[rows] == se).all()
        # SR draws with the stacked output's row index: rows of the stacked
        # result equal a column-wise quantization whose row ids are offset
        xb = O.to_blocked_rows(O.bf16_bits_to_f32(b[40:80]), O.AXIS_ROWS)
        nib, s1 = O.quantize_blocked(xb, True, 0x0A0A, O.GRID_UNIFORM, rnd, 4, 1,
                                     row_ids=np.arange(24, 48))
        assert (O.pack_nibbles(nib) == cs[24:48]).all() and (s1 == ss[24:48]).all()
