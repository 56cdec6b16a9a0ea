"""GPU parity of the fused RHT + 4-bit quantizer and the dequantizer against
the CPU oracle, through the C ABI.  Codes and scales must be bit-exact (SR
included); the dequantizer is bit-exact without the inverse RHT.

Sizes span several workgroup tiles and ragged tails; the special-value cases
cover zero blocks, bf16 subnormals, the tiny-scale branch, huge values,
negative zeros and every bf16 value in a unit-normalised block.
"""
import numpy as np
import pytest
import torch

from oracle import ufp4_oracle as O
from uniform_grid_fp4_amd import ufp4 as U
from uniform_grid_fp4_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"

GRIDS = (U.GRID_UNIFORM, U.GRID_E2M1, U.GRID_E2M1_MAX2)
COMBOS = [(g, r, h) for g in GRIDS for r in (U.ROUND_RTNE, U.ROUND_SR) for h in (False, True)]


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def check_quant(x_dev: torch.Tensor, axis, rht, mask, grid, rnd, seed=0, sid=0, goff=None,
                kpad=None, what=""):
    """Quantize on the GPU and compare every code and scale with the oracle."""
    print(f"[quant] {what} shape={tuple(x_dev.shape)} axis={axis} rht={rht} grid={grid} "
          f"rnd={rnd}", flush=True)
    goff_dev = torch.as_tensor(goff, dtype=torch.int64, device=DEV) if goff is not None else None
    q = U.ufp4_rht_quantize(x_dev, axis, rht, mask, grid, rnd, seed, sid, goff_dev, kpad)
    torch.cuda.synchronize()
    bits = W.bits_numpy(x_dev)
    c, s, kp = O.quantize(bits, axis, rht, mask, grid, rnd, seed, sid, goff, kpad=q.kpad)
    assert q.kpad == kp
    gc, gs = host(q.codes), host(q.scales)
    bad = np.argwhere(gc != c)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:3].tolist()}"
    assert np.array_equal(gs.view(np.uint32), s.view(np.uint32)), "scales differ"
    assert q.k == (x_dev.shape[1] if axis == U.BLOCKS_ALONG_COLS else x_dev.shape[0])
    return q


@pytest.mark.parametrize("grid,rnd,rht", COMBOS)
def test_rowwise_tiny_workload(grid, rnd, rht):
    L = W.tiny(DEV)
    check_quant(L.x, U.BLOCKS_ALONG_COLS, rht, L.masks[0], grid, rnd, 7, 0, what="tiny x")
    check_quant(L.w, U.BLOCKS_ALONG_COLS, rht, L.masks[0], grid, rnd, 7, 1, what="tiny w")


@pytest.mark.parametrize("grid,rnd,rht", COMBOS)
def test_colwise_tiny_workload(grid, rnd, rht):
    L = W.tiny(DEV)
    check_quant(L.dy, U.BLOCKS_ALONG_ROWS, rht, L.masks[2], grid, rnd, 3, 1, what="tiny dy^T")


@pytest.mark.parametrize("shape", [(37, 100), (300, 17), (1, 1), (5, 16), (513, 260)])
@pytest.mark.parametrize("axis", [U.BLOCKS_ALONG_COLS, U.BLOCKS_ALONG_ROWS])
def test_ragged_shapes(shape, axis):
    g = torch.Generator(device=DEV).manual_seed(11)
    x = torch.randn(shape, device=DEV, generator=g).to(torch.bfloat16)
    for grid, rnd, rht in [(0, 0, True), (0, 1, True), (1, 0, False), (1, 1, True), (2, 0, True),
                           (2, 1, False)]:
        check_quant(x, axis, rht, 0xB7E1, grid, rnd, 5, 2, what="ragged")


@pytest.mark.parametrize("axis", [U.BLOCKS_ALONG_COLS, U.BLOCKS_ALONG_ROWS])
def test_strided_and_misaligned_inputs(axis):
    g = torch.Generator(device=DEV).manual_seed(12)
    base = torch.randn((200, 130), device=DEV, generator=g).to(torch.bfloat16)
    for view in (base[:, :96], base[:, 1:97], base[3:, 5:120], base[:, :129]):
        check_quant(view, axis, True, 0x0F0F, U.GRID_UNIFORM, U.ROUND_SR, 1, 0, what="view")
        check_quant(view, axis, True, 0x0F0F, U.GRID_E2M1, U.ROUND_RTNE, what="view")


def special_values_tensor(rows=64, cols=256):
    rng = np.random.default_rng(13)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[0] = 0.0                                           # zero blocks
    x[1, :16] = -0.0
    x[2] = (rng.standard_normal(cols) * 2.0 ** -130).astype(np.float32)   # bf16 subnormals
    x[3] = (rng.standard_normal(cols) * 2.0 ** -80).astype(np.float32)    # tiny-scale branch
    x[4] = (rng.standard_normal(cols) * 2.0 ** -64).astype(np.float32)    # around the threshold
    x[5] = (rng.standard_normal(cols) * 2.0 ** 110).astype(np.float32)    # huge
    x[6] = np.tile(np.array([7, -3.5, 2.5, 0.5, 1.5, 6.5, -5.5, 4.5, 0, 0, 0, 0, 0, 0, 0, 0],
                            np.float32), cols // 16)                      # exact ties
    x[7] = np.tile(np.array([6, 5, -1.75, 0.25, 0.75, 3.5, 2.5, 1.25, 0, 0, 0, 0, 0, 0, 0, 0],
                            np.float32), cols // 16)
    x[8, ::16] = 1e-38                                   # one tiny value per block
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)   # truncate to bf16
    return bits


@pytest.mark.parametrize("grid,rnd,rht", COMBOS)
def test_special_values(grid, rnd, rht):
    xd = dev_bf16(special_values_tensor())
    check_quant(xd, U.BLOCKS_ALONG_COLS, rht, 0x8001, grid, rnd, 21, 0, what="special")
    check_quant(xd, U.BLOCKS_ALONG_ROWS, rht, 0x8001, grid, rnd, 21, 0, what="special^T")


@pytest.mark.parametrize("grid", GRIDS)
def test_every_bf16_value_in_a_unit_block(grid):
    g = O.GMAX[grid]
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    xs = O.bf16_bits_to_f32(allb)
    keep = np.isfinite(xs) & (np.abs(xs) <= g)
    xb = allb[keep]
    blk = np.zeros((xb.size, 16), np.uint16)
    blk[:, 0] = xb
    blk[:, 1] = (np.array([g], np.float32).view(np.uint32) >> 16).astype(np.uint16)[0]
    xd = dev_bf16(blk)
    for rnd in (U.ROUND_RTNE, U.ROUND_SR):
        check_quant(xd, U.BLOCKS_ALONG_COLS, False, 0, grid, rnd, 4, 0, what="all-bf16")
    # and every bf16 value through the RHT, 16 different values per block
    allf = allb[np.isfinite(xs) & (np.abs(xs) < 2.0 ** 120)]
    pad = (-allf.size) % 16
    blk2 = np.concatenate([allf, np.zeros(pad, np.uint16)]).reshape(-1, 16)
    check_quant(dev_bf16(blk2), U.BLOCKS_ALONG_COLS, True, 0x6D2B, grid, U.ROUND_RTNE,
                what="all-bf16 rht")


@pytest.mark.parametrize("counts", [
    [5, 0, 17, 1, 0, 9],
    [0, 0, 300, 16, 0],
    [256, 255, 257, 0, 1],
    list(np.random.default_rng(3).integers(0, 40, size=300)),   # more groups than threads
])
@pytest.mark.parametrize("rnd", [U.ROUND_RTNE, U.ROUND_SR])
def test_grouped_colwise(counts, rnd):
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    g = torch.Generator(device=DEV).manual_seed(14)
    x = torch.randn((T, 72), device=DEV, generator=g).to(torch.bfloat16)
    q = check_quant(x, U.BLOCKS_ALONG_ROWS, True, 0x1357, U.GRID_UNIFORM, rnd, 8, 1, goff=off,
                    what=f"groups{len(counts)}")
    assert q.kpad == U.padded_k_capacity(T, len(counts))


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("axis", [U.BLOCKS_ALONG_COLS, U.BLOCKS_ALONG_ROWS])
def test_dequantize(grid, axis):
    g = torch.Generator(device=DEV).manual_seed(15)
    x = torch.randn((130, 100), device=DEV, generator=g).to(torch.bfloat16)
    q = U.ufp4_rht_quantize(x, axis, True, 0x4242, grid, U.ROUND_RTNE)
    out = host(U.ufp4_dequantize(q))
    ref = O.dequantize(host(q.codes), host(q.scales), grid)
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    inv = host(U.ufp4_dequantize(q, inverse_rht=True))
    refi = O.dequantize(host(q.codes), host(q.scales), grid, True, 0x4242)
    tol = np.repeat(host(q.scales), 16, axis=1) * 1e-6
    assert (np.abs(inv - refi) <= tol + 1e-30).all()


def test_quantize_is_deterministic():
    L = W.tiny(DEV)
    a = U.ufp4_rht_quantize(L.dy, U.BLOCKS_ALONG_ROWS, True, 99, 0, U.ROUND_SR, 5, 1)
    b = U.ufp4_rht_quantize(L.dy, U.BLOCKS_ALONG_ROWS, True, 99, 0, U.ROUND_SR, 5, 1)
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)


@pytest.mark.parametrize("rnd", [U.ROUND_RTNE, U.ROUND_SR])
@pytest.mark.parametrize("e,rows,cols", [(3, 40, 24), (5, 256, 130), (2, 300, 64)])
def test_stacked_colwise(rnd, e, rows, cols):
    g = torch.Generator(device=DEV).manual_seed(16)
    x = torch.randn((e * rows, cols), device=DEV, generator=g).to(torch.bfloat16)
    print(f"[quant] stacked e={e} rows={rows} cols={cols} rnd={rnd}", flush=True)
    q = U.ufp4_rht_quantize(x, U.BLOCKS_ALONG_ROWS_STACKED, True, 0x5151, U.GRID_UNIFORM, rnd,
                            9, 1, n_groups=e)
    torch.cuda.synchronize()
    c, s, kp = O.quantize(W.bits_numpy(x), O.AXIS_ROWS_STACKED, True, 0x5151, O.GRID_UNIFORM,
                          rnd, 9, 1, n_stack=e)
    assert q.kpad == kp and q.rows == e * cols and q.k == rows
    assert np.array_equal(host(q.codes), c)
    assert np.array_equal(host(q.scales).view(np.uint32), s.view(np.uint32))
