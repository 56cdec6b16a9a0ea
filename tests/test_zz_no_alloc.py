"""The no-allocation diagnostics call, ufp4_quant_stats_noalloc, through the
C ABI: its partial sums live in the library's own per-device scratch array
instead of a caller's workspace, and its results equal ufp4_quant_stats's
bit for bit.  Two calls in a row, the second on a smaller input (fewer
partial records than the first left in the array), plus one on a
column-wise quantization; the GPU is one, so every call shares its array."""
import pytest
import torch

from uniform_grid_fp4_amd import ufp4 as U
from uniform_grid_fp4_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def same(a, b):
    return all(a[k] == b[k] for k in ("sum_x2", "sum_err2", "sum_x_xhat", "sum_abs_x",
                                      "sum_abs_xhat", "n_elems", "n_nonzero", "n_underflow",
                                      "hist"))


def test_noalloc_stats_equal_workspace_stats_two_calls():
    out = torch.empty(24, dtype=torch.int64, device=DEV)
    # first call: 4096 x 4096 (2^20 blocks: the grid's full 1024 partial records)
    x1 = W.bf16(W.laplace((4096, 4096), 1.0, 31, DEV))
    q1 = U.ufp4_rht_quantize(x1, U.BLOCKS_ALONG_COLS, True, 0xACE1, U.GRID_UNIFORM)
    print("[no-alloc] call 1: 4096 x 4096 row-wise", flush=True)
    got1 = U.ufp4_quant_stats_noalloc(x1, q1, U.BLOCKS_ALONG_COLS, out=out)
    ref1 = U.ufp4_quant_stats(x1, q1, U.BLOCKS_ALONG_COLS)
    assert same(got1, ref1), (got1, ref1)
    assert got1["n_elems"] == 4096 * 4096
    # second call, smaller: 100 x 200 (2 partial records; the array still
    # holds the first call's 1024)
    x2 = W.bf16(W.normal((100, 200), 1.0, 32, DEV))
    q2 = U.ufp4_rht_quantize(x2, U.BLOCKS_ALONG_COLS, True, 0x1357, U.GRID_E2M1)
    print("[no-alloc] call 2: 100 x 200 row-wise", flush=True)
    got2 = U.ufp4_quant_stats_noalloc(x2, q2, U.BLOCKS_ALONG_COLS, out=out)
    ref2 = U.ufp4_quant_stats(x2, q2, U.BLOCKS_ALONG_COLS)
    assert same(got2, ref2), (got2, ref2)
    assert got2["n_elems"] == 100 * 200
    # a column-wise quantization with stochastic rounding
    x3 = W.bf16(W.student_t3((333, 90), 33, DEV))
    q3 = U.ufp4_rht_quantize(x3, U.BLOCKS_ALONG_ROWS, True, 0x0F0F, U.GRID_UNIFORM, U.ROUND_SR,
                             5, 1)
    print("[no-alloc] call 3: 333 x 90 column-wise", flush=True)
    got3 = U.ufp4_quant_stats_noalloc(x3, q3, U.BLOCKS_ALONG_ROWS, out=out)
    assert same(got3, U.ufp4_quant_stats(x3, q3, U.BLOCKS_ALONG_ROWS))
    assert got3["n_elems"] == 333 * 90
