"""GPU parity of the diagnostics kernels through the C ABI: the FP64 sums of
ufp4_quant_stats / ufp4_output_stats agree with the oracle's quant_stats /
output_stats to 1e-10 relative (only the summation order differs), the
counts and the nibble histogram are exact, and repeated calls are bitwise
identical."""
import numpy as np
import pytest
import torch

from oracle import ufp4_oracle as O
from uniform_grid_fp4_amd import ufp4 as U
from uniform_grid_fp4_amd import workloads as W

from test_gpu_quantize import dev_bf16, special_values_tensor

pytestmark = pytest.mark.gpu
DEV = "cuda"


def compare(gpu, ref, what):
    for k in U.STATS_SUMS:
        assert gpu[k] == pytest.approx(ref[k], rel=1e-10, abs=1e-300), f"{what}: {k}"
    for k in U.STATS_COUNTS:
        assert gpu[k] == ref[k], f"{what}: {k} {gpu[k]} != {ref[k]}"
    assert list(gpu["hist"]) == list(ref["hist"]), f"{what}: hist"


def check(x, axis, rht, mask, grid, rnd, what=""):
    print(f"[stats] {what} shape={tuple(x.shape)} axis={axis} rht={rht} grid={grid} rnd={rnd}",
          flush=True)
    q = U.ufp4_rht_quantize(x, axis, rht, mask, grid, rnd, 5, 1)
    got = U.ufp4_quant_stats(x, q, axis)
    ref = O.quant_stats(W.bits_numpy(x), q.codes.cpu().numpy(), q.scales.cpu().numpy(), axis,
                        rht, mask, grid)
    compare(got, ref, what)
    return got


@pytest.mark.parametrize("grid", [U.GRID_UNIFORM, U.GRID_E2M1, U.GRID_E2M1_MAX2])
@pytest.mark.parametrize("rnd", [U.ROUND_RTNE, U.ROUND_SR])
@pytest.mark.parametrize("rht", [False, True])
@pytest.mark.parametrize("axis", [U.BLOCKS_ALONG_COLS, U.BLOCKS_ALONG_ROWS])
def test_tiny_layer_tensors(grid, rnd, rht, axis):
    L = W.tiny(DEV)
    check(L.x, axis, rht, 0x6D2B, grid, rnd, "tiny x")
    check(L.dy, axis, rht, 0x6D2B, grid, rnd, "tiny dy")


@pytest.mark.parametrize("shape", [(37, 100), (300, 17), (1, 1), (513, 260)])
def test_ragged_and_strided(shape):
    g = torch.Generator(device=DEV).manual_seed(31)
    base = torch.randn((shape[0] + 3, shape[1] + 5), device=DEV, generator=g).to(torch.bfloat16)
    x = base[1:1 + shape[0], 2:2 + shape[1]]
    for axis in (U.BLOCKS_ALONG_COLS, U.BLOCKS_ALONG_ROWS):
        check(x, axis, True, 0x1234, U.GRID_UNIFORM, U.ROUND_SR, "ragged")
        check(x, axis, False, 0, U.GRID_E2M1, U.ROUND_RTNE, "ragged")


@pytest.mark.parametrize("grid", [U.GRID_UNIFORM, U.GRID_E2M1, U.GRID_E2M1_MAX2])
def test_special_values(grid):
    x = dev_bf16(special_values_tensor())
    for axis in (U.BLOCKS_ALONG_COLS, U.BLOCKS_ALONG_ROWS):
        check(x, axis, True, 0x8001, grid, U.ROUND_RTNE, "special")


def test_outlier_tensor_uniform_gains_under_rht():
    """The pages' Q1 pattern on a 1 % x 50 outlier-channel tensor (gist.science
    technical summary; paperlayer section 5 Q1): RHT lowers the underflow
    ratio on both grids."""
    L = W.dense_1p5b(DEV)
    x = L.x[:1024]
    st = {(grid, rht): check(x, U.BLOCKS_ALONG_COLS, rht, L.masks[0], grid, U.ROUND_RTNE,
                             "outliers")
          for grid in (U.GRID_UNIFORM, U.GRID_E2M1) for rht in (False, True)}
    for grid in (U.GRID_UNIFORM, U.GRID_E2M1):
        uf = {r: st[(grid, r)]["n_underflow"] / st[(grid, r)]["n_nonzero"] for r in (False, True)}
        assert uf[True] < uf[False]


def test_output_stats_against_oracle():
    L = W.tiny(DEV)
    xq = U.ufp4_rht_quantize(L.x, U.BLOCKS_ALONG_COLS, True, 0x55AA)
    wq = U.ufp4_rht_quantize(L.w, U.BLOCKS_ALONG_COLS, True, 0x55AA)
    y = U.ufp4_gemm_fprop(xq, wq)
    ref = torch.matmul(L.x.float(), L.w.float().t().contiguous())
    got = U.ufp4_output_stats(ref, y)
    exp = O.output_stats(ref.cpu().numpy(), y.cpu().numpy())
    compare(got, exp, "fprop output")
    # strided views
    got2 = U.ufp4_output_stats(ref[3:, 5:200], y[3:, 5:200])
    exp2 = O.output_stats(ref[3:, 5:200].cpu().numpy(), y[3:, 5:200].cpu().numpy())
    compare(got2, exp2, "fprop output view")


def test_bitwise_reproducible():
    g = torch.Generator(device=DEV).manual_seed(32)
    x = torch.randn((2048, 1024), device=DEV, generator=g).to(torch.bfloat16)
    q = U.ufp4_rht_quantize(x, U.BLOCKS_ALONG_ROWS, True, 77, U.GRID_E2M1, U.ROUND_SR, 3, 0)
    a = U.ufp4_quant_stats(x, q, U.BLOCKS_ALONG_ROWS)
    b = U.ufp4_quant_stats(x, q, U.BLOCKS_ALONG_ROWS)
    assert a == b
    r = torch.randn((1500, 700), device=DEV, generator=g)
    t = r + 1e-3 * torch.randn((1500, 700), device=DEV, generator=g)
    assert U.ufp4_output_stats(r, t) == U.ufp4_output_stats(r, t)
