"""GPU parity of the dual-axis quantizer (one read of x, the row-wise and the
transposed column-wise operand) through the C ABI: both outputs must equal
the oracle's single-axis quantizations bit for bit (codes and scales, SR
included), and the single-axis GPU calls with the same options.

Covers every grid / rounding / per-side RHT combination, ragged and
misaligned inputs (both the dword and the 16-bit load paths, paired and
unpaired row-wise stores), grouped and stacked column-wise layouts, and the
special values of the single-axis tests."""
import numpy as np
import pytest
import torch

from oracle import ufp4_oracle as O
from uniform_grid_fp4_amd import ufp4 as U
from uniform_grid_fp4_amd import workloads as W

from test_gpu_quantize import dev_bf16, special_values_tensor

pytestmark = pytest.mark.gpu
DEV = "cuda"


def host(t):
    return t.cpu().numpy()


def expect_equal(q, c, s, what):
    gc, gs = host(q.codes), host(q.scales)
    bad = np.argwhere(gc != c)
    assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first at {bad[:3].tolist()}"
    assert np.array_equal(gs.view(np.uint32), s.view(np.uint32)), f"{what}: scales differ"


def check_dual(x, rowwise, colwise, grid, rnd, seed=0, col_axis=U.BLOCKS_ALONG_ROWS,
               goff=None, n_groups=0, what=""):
    print(f"[dual] {what} shape={tuple(x.shape)} row={rowwise} col={colwise} grid={grid} "
          f"rnd={rnd} axis={col_axis} groups={n_groups or (0 if goff is None else len(goff) - 1)}",
          flush=True)
    goff_dev = torch.as_tensor(goff, dtype=torch.int64, device=DEV) if goff is not None else None
    qr, qc = U.ufp4_rht_quantize_dual(x, rowwise, colwise, col_axis, grid, rnd, seed,
                                      goff_dev, n_groups=n_groups)
    torch.cuda.synchronize()
    bits = W.bits_numpy(x)
    c, s, kp = O.quantize(bits, O.AXIS_COLS, rowwise[0], rowwise[1], grid, rnd, seed,
                          rowwise[2])
    assert qr.kpad == kp and qr.k == x.shape[1] and qr.rows == x.shape[0]
    expect_equal(qr, c, s, what + " row-wise")
    if col_axis == U.BLOCKS_ALONG_ROWS_STACKED:
        c, s, kp = O.quantize(bits, O.AXIS_ROWS_STACKED, colwise[0], colwise[1], grid, rnd, seed,
                              colwise[2], n_stack=n_groups)
    else:
        c, s, kp = O.quantize(bits, O.AXIS_ROWS, colwise[0], colwise[1], grid, rnd, seed,
                              colwise[2], goff, kpad=qc.kpad)
    assert qc.kpad == kp
    expect_equal(qc, c, s, what + " column-wise")
    # the single-axis GPU calls agree as well
    sr = U.ufp4_rht_quantize(x, U.BLOCKS_ALONG_COLS, rowwise[0], rowwise[1], grid, rnd, seed,
                             rowwise[2])
    sc = U.ufp4_rht_quantize(x, col_axis, colwise[0], colwise[1], grid, rnd, seed, colwise[2],
                             goff_dev, kpad=qc.kpad, n_groups=n_groups)
    assert torch.equal(sr.codes, qr.codes) and torch.equal(sr.scales, qr.scales)
    assert torch.equal(sc.codes, qc.codes) and torch.equal(sc.scales, qc.scales)
    assert (qr.rht, qr.sign_mask) == (int(rowwise[0]), rowwise[1] if rowwise[0] else 0)
    assert (qc.rht, qc.sign_mask) == (int(colwise[0]), colwise[1] if colwise[0] else 0)
    return qr, qc


SIDES = [((True, 0x1357, 0), (True, 0xBEEF, 1)), ((False, 0x1357, 0), (True, 0xBEEF, 1)),
         ((True, 0x00F0, 3), (False, 0, 0)), ((False, 0, 0), (False, 0, 2))]


@pytest.mark.parametrize("grid", [U.GRID_UNIFORM, U.GRID_E2M1, U.GRID_E2M1_MAX2])
@pytest.mark.parametrize("rnd", [U.ROUND_RTNE, U.ROUND_SR])
@pytest.mark.parametrize("sides", SIDES)
def test_tiny_layer_tensors(grid, rnd, sides):
    L = W.tiny(DEV)
    for name, x in (("x", L.x), ("dy", L.dy)):
        check_dual(x, sides[0], sides[1], grid, rnd, 7, what=f"tiny {name}")


@pytest.mark.parametrize("shape", [(37, 100), (300, 17), (1, 1), (5, 16), (513, 260), (16, 48),
                                   (40, 24), (257, 129)])
def test_ragged_shapes(shape):
    g = torch.Generator(device=DEV).manual_seed(21)
    x = torch.randn(shape, device=DEV, generator=g).to(torch.bfloat16)
    for grid, rnd in [(0, 0), (0, 1), (1, 0), (1, 1)]:
        check_dual(x, (True, 0xA5A5, 0), (True, 0x5A5A, 1), grid, rnd, 5, what="ragged")


def test_strided_and_misaligned_views():
    g = torch.Generator(device=DEV).manual_seed(22)
    base = torch.randn((200, 150), device=DEV, generator=g).to(torch.bfloat16)
    for view in (base[:, :96], base[:, 1:97], base[3:, 5:120], base[:, :129], base[1:, 1:]):
        check_dual(view, (True, 0x0F0F, 0), (True, 0xF0F0, 1), U.GRID_UNIFORM, U.ROUND_SR, 1,
                   what="view")
        check_dual(view, (False, 0, 0), (True, 0x3C3C, 0), U.GRID_E2M1, U.ROUND_RTNE,
                   what="view")


@pytest.mark.parametrize("counts", [
    [5, 0, 17, 1, 0, 9],
    [256, 255, 257, 0, 1],
    list(np.random.default_rng(3).integers(0, 40, size=300)),
])
@pytest.mark.parametrize("rnd", [U.ROUND_RTNE, U.ROUND_SR])
def test_grouped_columnwise(counts, rnd):
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    g = torch.Generator(device=DEV).manual_seed(23)
    x = torch.randn((T, 72), device=DEV, generator=g).to(torch.bfloat16)
    check_dual(x, (True, 0x1111, 0), (True, 0x2222, 1), U.GRID_UNIFORM, rnd, 8, goff=off,
               what=f"groups{len(counts)}")


@pytest.mark.parametrize("e,rows,cols", [(3, 40, 24), (5, 256, 130), (2, 300, 64)])
def test_stacked_columnwise(e, rows, cols):
    g = torch.Generator(device=DEV).manual_seed(24)
    x = torch.randn((e * rows, cols), device=DEV, generator=g).to(torch.bfloat16)
    check_dual(x, (True, 0x6666, 0), (True, 0x9999, 0), U.GRID_UNIFORM, U.ROUND_RTNE,
               col_axis=U.BLOCKS_ALONG_ROWS_STACKED, n_groups=e, what="stacked")


@pytest.mark.parametrize("grid", [U.GRID_UNIFORM, U.GRID_E2M1, U.GRID_E2M1_MAX2])
@pytest.mark.parametrize("rnd", [U.ROUND_RTNE, U.ROUND_SR])
def test_special_values(grid, rnd):
    xd = dev_bf16(special_values_tensor())
    check_dual(xd, (True, 0x8001, 0), (True, 0x7FFE, 1), grid, rnd, 21, what="special")


def test_outputs_reused_and_deterministic():
    L = W.tiny(DEV)
    a = U.ufp4_rht_quantize_dual(L.dy, (True, 3, 0), (True, 5, 1), rnd=U.ROUND_SR, seed=9)
    b = U.ufp4_rht_quantize_dual(L.dy, (True, 3, 0), (True, 5, 1), rnd=U.ROUND_SR, seed=9,
                                 out_rows=a[0], out_cols=a[1])
    c = U.ufp4_rht_quantize_dual(L.dy, (True, 3, 0), (True, 5, 1), rnd=U.ROUND_SR, seed=9)
    torch.cuda.synchronize()
    assert b[0].codes.data_ptr() == a[0].codes.data_ptr()
    for u, v in ((b[0], c[0]), (b[1], c[1])):
        assert torch.equal(u.codes, v.codes) and torch.equal(u.scales, v.scales)
