"""The hot path captured as a HIP graph: the library's calls only launch
kernels on the caller's stream (no allocation, copy, memset or
synchronisation), so a whole UFP4 step -- the three dual-axis quantizations
and FPROP, DGRAD and WGRAD, dense and expert-grouped -- can be stream-captured
and replayed.  Each of several replays, with eager work and synchronisation
between them and its outputs overwritten with NaN first, must reproduce the
eager step bit for bit."""
import numpy as np
import pytest
import torch

from uniform_grid_fp4_amd import ufp4 as U
from uniform_grid_fp4_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dense_step(L, bufs):
    mf, md, mw = L.masks
    xq, xtq = U.ufp4_rht_quantize_dual(L.x, (True, mf, 0), (True, mw, 0),
                                       out_rows=bufs.get("xq"), out_cols=bufs.get("xtq"))
    wq, wtq = U.ufp4_rht_quantize_dual(L.w, (True, mf, 0), (True, md, 0),
                                       out_rows=bufs.get("wq"), out_cols=bufs.get("wtq"))
    dq, dtq = U.ufp4_rht_quantize_dual(L.dy, (True, md, 0), (True, mw, 1), rnd=U.ROUND_SR,
                                       seed=9, out_rows=bufs.get("dq"), out_cols=bufs.get("dtq"))
    bufs.update(xq=xq, xtq=xtq, wq=wq, wtq=wtq, dq=dq, dtq=dtq)
    bufs["y"] = U.ufp4_gemm_fprop(xq, wq, out=bufs.get("y"))
    bufs["dx"] = U.ufp4_gemm_out(U.DGRAD, dq, wtq, torch.bfloat16, out=bufs.get("dx"))
    bufs["dw"] = U.ufp4_gemm_wgrad(dtq, xtq, out=bufs.get("dw"))
    return [bufs["y"], bufs["dx"], bufs["dw"], xq.codes, dtq.codes, dtq.scales]


def moe_step(L, offd, E, bufs):
    mf, md, mw = L.masks
    xq, xtq = U.ufp4_rht_quantize_dual(L.x, (True, mf, 0), (True, mw, 0), group_offsets=offd,
                                       out_rows=bufs.get("xq"), out_cols=bufs.get("xtq"))
    wq, wtq = U.ufp4_rht_quantize_dual(L.w, (True, mf, 0), (True, md, 0),
                                       col_axis=U.BLOCKS_ALONG_ROWS_STACKED, n_groups=E,
                                       out_rows=bufs.get("wq"), out_cols=bufs.get("wtq"))
    dq, dtq = U.ufp4_rht_quantize_dual(L.dy, (True, md, 0), (True, mw, 1), rnd=U.ROUND_SR,
                                       seed=9, group_offsets=offd,
                                       out_rows=bufs.get("dq"), out_cols=bufs.get("dtq"))
    bufs.update(xq=xq, xtq=xtq, wq=wq, wtq=wtq, dq=dq, dtq=dtq)
    bufs["y"] = U.ufp4_grouped_gemm(U.FPROP, offd, xq, wq, out=bufs.get("y"))
    bufs["dx"] = U.ufp4_grouped_gemm(U.DGRAD, offd, dq, wtq, out=bufs.get("dx"))
    bufs["dw"] = U.ufp4_grouped_gemm(U.WGRAD, offd, dtq, xtq, out=bufs.get("dw"))
    return [bufs["y"], bufs["dx"], bufs["dw"], xtq.codes, dtq.scales]


def check_replays(step, replays=4):
    outs = step()                      # eager: allocates every buffer once
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = step()
    assert all(a.data_ptr() == b.data_ptr() for a, b in zip(outs, captured))
    for i in range(replays):
        step()                         # eager work between the replays
        torch.cuda.synchronize()
        ref = [t.clone() for t in outs]
        for t in outs:
            if t.is_floating_point():
                t.fill_(float("nan"))
            else:
                t.fill_(0xA5)
        g.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), f"replay {i}: output {k} differs from the eager step"


def test_graph_dense_step():
    L = W.dense_layer(512, 384, 640, 0.01, 50.0, 5, DEV, "graph-dense")
    bufs = {}
    check_replays(lambda: dense_step(L, bufs))


def test_graph_moe_step():
    E, H, F, T = 8, 256, 192, 2000
    L = W.moe_layer(E, H, F, T, 0.01, 50.0, 6, DEV, "graph-moe")
    offd = torch.as_tensor(L.offsets, device=DEV)
    assert int(np.diff(L.offsets).min()) >= 0
    bufs = {}
    check_replays(lambda: moe_step(L, offd, E, bufs))
