"""GPU parity of the quantizer at the sweep workload's full size: a 16384 x
16384 bf16 tensor (2^28 elements) drawn from a Gaussian, a Laplace and a
Student-t (nu = 3) distribution, quantized row-wise and column-wise
(transposed output), onto the uniform and the E2M1 grid, with RTNE and with
stochastic rounding, with and without the RHT -- the calls and arguments
`bench.py --workload quant-sweep` times.  The oracle recomputes sampled
output rows one by one (the first, the last and random ones; for the
column-wise output a row is a whole input column), and codes and scales must
match bit for bit, SR included (the sampled rows draw the SR bits of their
position in the full output).  One dual-axis call per tensor is checked the
same way.
"""
import numpy as np
import pytest
import torch

from oracle import ufp4_oracle as O
from uniform_grid_fp4_amd import ufp4 as U
from uniform_grid_fp4_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"
MASK, SEED, SID = 0xBEEF, 7, 0      # the sweep's sign mask, SR seed and stream


def sample(n, k, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, size=k)])).astype(np.int64)


def check_sampled(q, x, axis, rht, grid, rnd, rows, sid=SID, mask=MASK, what=""):
    """Output rows `rows` of q equal the oracle's quantization of the same
    input rows (row-wise) or input columns (column-wise)."""
    r = torch.as_tensor(rows, device=x.device)
    if axis == U.BLOCKS_ALONG_COLS:
        xb = O.to_blocked_rows(O.bf16_bits_to_f32(W.bits_numpy(x[r])), O.AXIS_COLS)
    else:
        xb = O.to_blocked_rows(O.bf16_bits_to_f32(W.bits_numpy(x[:, r])), O.AXIS_ROWS)
    assert xb.shape[1] == q.kpad
    nib, s = O.quantize_blocked(xb, rht, mask, grid, rnd, SEED, sid, row_ids=rows)
    gc = q.codes[r].cpu().numpy()
    gs = q.scales[r].cpu().numpy()
    assert np.array_equal(gc, O.pack_nibbles(nib)), f"{what}: codes differ"
    assert np.array_equal(gs.view(np.uint32), s.view(np.uint32)), f"{what}: scales differ"


@pytest.fixture(scope="module", params=W.SWEEP_DISTS)
def sweep(request):
    x = W.sweep_tensor(request.param, DEV)
    assert tuple(x.shape) == W.SWEEP_SHAPE == (16384, 16384)
    yield request.param, x
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("axis", [U.BLOCKS_ALONG_COLS, U.BLOCKS_ALONG_ROWS])
def test_sweep_quantizer_full_size(sweep, axis):
    dist, x = sweep
    n = x.shape[0]
    for grid in (U.GRID_UNIFORM, U.GRID_E2M1):
        for rnd in (U.ROUND_RTNE, U.ROUND_SR):
            for rht in (False, True):
                q = U.ufp4_rht_quantize(x, axis, rht, MASK, grid, rnd, SEED, SID)
                rows = sample(n, 6, 100 * grid + 10 * rnd + int(rht) + 7 * axis)
                what = f"{dist} axis={axis} grid={grid} rnd={rnd} rht={rht}"
                check_sampled(q, x, axis, rht, grid, rnd, rows, what=what)
                del q


def test_sweep_dual_quantizer_full_size(sweep):
    """The dual-axis kernel on the full sweep tensor (UFP4: uniform grid, RHT,
    SR; the two outputs on SR streams 0 and 1, different sign masks)."""
    dist, x = sweep
    q_r, q_c = U.ufp4_rht_quantize_dual(x, (True, MASK, 0), (True, 0x1234, 1),
                                        grid=U.GRID_UNIFORM, rnd=U.ROUND_SR, seed=SEED)
    rows = sample(x.shape[0], 6, 5)
    check_sampled(q_r, x, U.BLOCKS_ALONG_COLS, True, U.GRID_UNIFORM, U.ROUND_SR, rows, sid=0,
                  mask=MASK, what=f"{dist} dual row-wise")
    check_sampled(q_c, x, U.BLOCKS_ALONG_ROWS, True, U.GRID_UNIFORM, U.ROUND_SR, rows, sid=1,
                  mask=0x1234, what=f"{dist} dual column-wise")


@pytest.mark.parametrize("rnd", [U.ROUND_RTNE, U.ROUND_SR])
def test_sweep_single_and_dual_agree_whole_output(sweep, rnd):
    """Every code and scale of the full 16384 x 16384 outputs, not a sample:
    the column-wise single-axis call (four columns per lane, its XCD-major
    tile order) equals the dual-axis kernel's column-wise output (two columns
    per lane, its own tiles), and the row-wise single-axis call equals the
    dual-axis kernel's row-wise output, for RTNE and SR (same masks, seed and
    streams).  The oracle pins sampled rows of both in the tests above."""
    dist, x = sweep
    q_r, q_c = U.ufp4_rht_quantize_dual(x, (True, MASK, 0), (True, 0x1234, 1),
                                        grid=U.GRID_UNIFORM, rnd=rnd, seed=SEED)
    s_c = U.ufp4_rht_quantize(x, U.BLOCKS_ALONG_ROWS, True, 0x1234, U.GRID_UNIFORM, rnd, SEED, 1)
    assert torch.equal(s_c.codes, q_c.codes), f"{dist} rnd={rnd}: column-wise codes"
    assert torch.equal(s_c.scales.view(torch.int32), q_c.scales.view(torch.int32))
    del s_c
    s_r = U.ufp4_rht_quantize(x, U.BLOCKS_ALONG_COLS, True, MASK, U.GRID_UNIFORM, rnd, SEED, 0)
    assert torch.equal(s_r.codes, q_r.codes), f"{dist} rnd={rnd}: row-wise codes"
    assert torch.equal(s_r.scales.view(torch.int32), q_r.scales.view(torch.int32))
    del s_r, q_r, q_c
    torch.cuda.empty_cache()


@pytest.mark.parametrize("ld_extra", [0, 8, 2])
def test_column_wise_wide_tiles_ragged(ld_extra):
    """Large column-wise inputs take the kernel's four-columns-per-lane tiles
    (8-byte row loads) when rows are 8-byte aligned and the column count is a
    multiple of 4; ld_extra = 2 breaks that alignment and takes the two-column
    tiles at the same size.  Ragged rows (16380) and a ragged last column tile
    (8200 = 32 * 256 + 8 columns), contiguous and strided rows; sampled output
    rows (input columns, the last tile's all included) bit-exact against the
    oracle for the three grids, RTNE and SR."""
    n_rows, n_cols = 16380, 8200
    g = torch.Generator(device=DEV)
    g.manual_seed(11 + ld_extra)
    base = torch.randn(n_rows, n_cols + ld_extra, device=DEV, generator=g).to(torch.bfloat16)
    x = base[:, :n_cols]
    assert x.stride(0) == n_cols + ld_extra
    cols = np.unique(np.concatenate([sample(n_cols, 6, 3 + ld_extra),
                                     np.arange(8188, n_cols)])).astype(np.int64)
    for grid in (U.GRID_UNIFORM, U.GRID_E2M1, U.GRID_E2M1_MAX2):
        for rnd in (U.ROUND_RTNE, U.ROUND_SR):
            q = U.ufp4_rht_quantize(x, U.BLOCKS_ALONG_ROWS, True, MASK, grid, rnd, SEED, SID)
            assert q.rows == n_cols and q.kpad == 16384
            check_sampled(q, x, U.BLOCKS_ALONG_ROWS, True, grid, rnd, cols,
                          what=f"wide ld+{ld_extra} grid={grid} rnd={rnd}")
            del q


def test_column_wise_wide_tiles_grouped():
    """The four-column tiles in the grouped (per-expert padded) mode: 16000
    rows in 50 groups of ragged sizes, some empty, 8200 columns.  Sampled
    output rows bit-exact against the oracle (RTNE and SR), and the whole
    output equal to the dual-axis kernel's column-wise output, which tiles
    differently (two columns per lane, its own loads and tile order)."""
    n_rows, n_cols, n_groups = 16000, 8200, 50
    rng = np.random.default_rng(21)
    counts = rng.multinomial(n_rows, rng.dirichlet(np.ones(n_groups)))
    counts[[3, 17, 40]] = 0
    counts[0] += n_rows - counts.sum()
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    offd = torch.as_tensor(off, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(21)
    x = torch.randn(n_rows, n_cols, device=DEV, generator=g).to(torch.bfloat16)
    cols = np.unique(np.concatenate([sample(n_cols, 6, 22), np.arange(8190, n_cols)]))
    for rnd in (U.ROUND_RTNE, U.ROUND_SR):
        q = U.ufp4_rht_quantize(x, U.BLOCKS_ALONG_ROWS, True, MASK, U.GRID_UNIFORM, rnd, SEED, 1,
                                group_offsets=offd)
        assert q.kpad == U.padded_k_capacity(n_rows, n_groups)
        r = torch.as_tensor(cols, device=DEV)
        xb = O.to_blocked_rows(O.bf16_bits_to_f32(W.bits_numpy(x[:, r])), O.AXIS_ROWS, off)
        if xb.shape[1] < q.kpad:
            xb = np.concatenate([xb, np.zeros((xb.shape[0], q.kpad - xb.shape[1]), np.float32)], 1)
        nib, s = O.quantize_blocked(xb, True, MASK, O.GRID_UNIFORM, rnd, SEED, 1, row_ids=cols)
        assert np.array_equal(q.codes[r].cpu().numpy(), O.pack_nibbles(nib)), f"rnd={rnd} codes"
        assert np.array_equal(q.scales[r].cpu().numpy().view(np.uint32), s.view(np.uint32))
        _, qc = U.ufp4_rht_quantize_dual(x, (True, 0x1234, 0), (True, MASK, 1), rnd=rnd,
                                         seed=SEED, group_offsets=offd)
        assert torch.equal(qc.codes, q.codes) and torch.equal(qc.scales, q.scales)
        del q, qc
