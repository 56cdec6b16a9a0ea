"""Pins for the oracle's random Hadamard transform.

The transform (paperlayer.ai summary of arXiv 2606.20381, section 2
"Random Hadamard transforms") is a random sign diagonal followed by a
Sylvester Hadamard transform, norm preserving, applied along a GEMM's
reduction dimension so that it cancels.  Each test checks the oracle against
mathematics that does not come from the oracle itself.
"""
import numpy as np

from oracle import ufp4_oracle as O


def hadamard_closed_form(n=16):
    """Sylvester Hadamard entry H[i, j] = (-1)^popcount(i & j)."""
    i = np.arange(n)
    return np.array([[(-1.0) ** bin(int(a) & int(b)).count("1") for b in i] for a in i])


def test_sylvester_matrix_is_hadamard():
    H = O.sylvester_hadamard(4)
    assert (H @ H.T == 16 * np.eye(16)).all()
    assert (H == hadamard_closed_form()).all()


def test_butterfly_is_exact_matrix_product_on_small_integers():
    rng = np.random.default_rng(1)
    x = rng.integers(-1000, 1001, size=(2000, 16)).astype(np.float32)
    y = O.fwht16(x)
    ref = x.astype(np.float64) @ hadamard_closed_form().T
    assert (y.astype(np.float64) == ref).all()


def test_butterfly_float32_error_within_four_roundings():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((20000, 16)) *
         10.0 ** rng.uniform(-6, 6, size=(20000, 1))).astype(np.float32)
    y = O.fwht16(x).astype(np.float64)
    ref = x.astype(np.float64) @ hadamard_closed_form().T
    bound = 4 * 2.0 ** -24 * np.abs(x.astype(np.float64)).sum(-1, keepdims=True) * (1 + 1e-6)
    assert (np.abs(y - ref) <= bound).all()
    # and it is not trivially exact: some outputs do round
    assert (y != ref).any()


def test_sign_mask_bit_j_negates_coordinate_j():
    H = hadamard_closed_form()
    for j in range(16):
        e = np.zeros((1, 16), np.float32)
        e[0, j] = 1.0
        y = O.rht16(e, 1 << j).astype(np.float64)[0]
        assert (y == -0.25 * H[:, j]).all()
        y0 = O.rht16(e, 0).astype(np.float64)[0]
        assert (y0 == 0.25 * H[:, j]).all()


def test_rht_is_orthonormal_and_norm_preserving():
    mask = 0xA5C3
    d = O.signs_from_mask(mask).astype(np.float64)
    R = 0.25 * hadamard_closed_form() * d[None, :]
    assert (R @ R.T == np.eye(16)).all()
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5000, 16)).astype(np.float32)
    y = O.rht16(x, mask).astype(np.float64)
    n0 = np.linalg.norm(x.astype(np.float64), axis=-1)
    n1 = np.linalg.norm(y, axis=-1)
    assert np.allclose(n1, n0, rtol=2e-6, atol=0)
    assert np.allclose(y, x.astype(np.float64) @ R.T, rtol=0, atol=1e-6)


def test_rotation_cancels_along_the_reduction_dimension():
    rng = np.random.default_rng(4)
    a = rng.standard_normal((64, 128)).astype(np.float32)
    b = rng.standard_normal((48, 128)).astype(np.float32)
    mask = 0x3C5A
    ra = O.rht16(a.reshape(64, 8, 16), mask).reshape(64, 128).astype(np.float64)
    rb = O.rht16(b.reshape(48, 8, 16), mask).reshape(48, 128).astype(np.float64)
    exact = a.astype(np.float64) @ b.astype(np.float64).T
    bound = np.abs(a.astype(np.float64)) @ np.abs(b.astype(np.float64)).T
    assert np.abs(ra @ rb.T - exact).max() <= 1e-6 * bound.max()
    # different masks on the two sides do NOT cancel
    rb2 = O.rht16(b.reshape(48, 8, 16), mask ^ 1).reshape(48, 128).astype(np.float64)
    assert np.abs(ra @ rb2.T - exact).max() > 1e-2 * np.abs(exact).max()


def test_inverse_rht_in_dequantize_undoes_the_rotation():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)       # truncate to bf16
    xf = O.bf16_bits_to_f32(bits).astype(np.float64)
    mask = 0x1234
    codes, scales, kp = O.quantize(bits, O.AXIS_COLS, True, mask, O.GRID_UNIFORM, O.ROUND_RTNE)
    back = O.dequantize(codes, scales, O.GRID_UNIFORM, inverse_rht=True, sign_mask=mask)
    # per block the rotated error is at most half a step s/7/2 per coordinate;
    # the rotation preserves its norm, so ||x - back|| <= sqrt(16) * s / 14
    err = np.linalg.norm((back - xf).reshape(32, 4, 16), axis=-1)
    assert (err <= 4 * scales / 14 * (1 + 1e-5)).all()
    # without the inverse the values live in the rotated frame and are far off
    rot = O.dequantize(codes, scales, O.GRID_UNIFORM)
    assert np.abs(rot - xf).max() > 10 * np.abs(back - xf).max()
