"""Split-K WGRAD: a weight gradient with few output tiles and a long token
contraction (a MoE-124B expert's 149170 routed tokens; paperlayer.ai summary,
section 2 "Random Hadamard transforms": WGRAD contracts over the tokens) is
split along K into the caller's workspace and summed in a fixed order.  The
split and unsplit results both match the oracle element by element on
sampled outputs (|C - C_ref| <= 1e-5 * sum_k |a_k||b_k|), and the split
result is bitwise reproducible."""
import numpy as np
import pytest
import torch

from oracle import ufp4_oracle as O
from uniform_grid_fp4_amd import ufp4 as U
from uniform_grid_fp4_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-5


@pytest.mark.parametrize("M,N", [(256, 256), (384, 200)])
def test_split_k_wgrad_long_contraction(M, N):
    T = 149170
    print(f"[splitk] T={T} M={M} N={N}", flush=True)
    dy = W.bf16(W.normal((T, M), 1e-4, 11, DEV))
    x = W.bf16(W.normal((T, N), 1.0, 12, DEV))
    mw, seed = 0x5A3C, 77
    dytq = U.ufp4_rht_quantize(dy, U.BLOCKS_ALONG_ROWS, True, mw, U.GRID_UNIFORM, U.ROUND_SR,
                               seed, 1)
    xtq = U.ufp4_rht_quantize(x, U.BLOCKS_ALONG_ROWS, True, mw)
    need = U.ufp4_workspace_size(U.WGRAD, M, N, dytq.kpad)
    assert need > 0
    ws = torch.empty(need // 4, dtype=torch.float32, device=DEV)
    plain = U.ufp4_gemm_wgrad(dytq, xtq)
    split = U.ufp4_gemm_wgrad(dytq, xtq, workspace=ws)
    again = torch.full_like(split, float("nan"))
    U.ufp4_gemm_wgrad(dytq, xtq, out=again, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(split, again)
    # the oracle on sampled rows and columns of dW (its own quantization of
    # the sampled columns of dY and X, SR bits of their output positions)
    rows = np.array([0, 1, 37, M // 2, M - 2, M - 1])
    cols = np.array([0, 5, 64, N // 3, N - 1])
    dyb, xb = W.bits_numpy(dy), W.bits_numpy(x)
    ca, sa, _ = O.quantize(dyb, O.AXIS_ROWS, True, mw, O.GRID_UNIFORM, 1, seed, 1, out_rows=rows)
    cb, sb, _ = O.quantize(xb, O.AXIS_ROWS, True, mw, O.GRID_UNIFORM, 0, out_rows=cols)
    C, bound = O.gemm_tn(ca, sa, cb, sb)
    for name, out in (("split", split), ("plain", plain)):
        got = out.cpu().numpy()[np.ix_(rows, cols)].astype(np.float64)
        err = np.abs(got - C)
        assert (err <= TOL * bound).all(), (name, (err / (TOL * bound)).max())


def test_no_split_without_enough_workspace():
    """A workspace smaller than ufp4_workspace_size leaves the call unsplit:
    the output equals the plain call's bit for bit."""
    T, M, N = 40000, 128, 128
    dy = W.bf16(W.normal((T, M), 1.0, 21, DEV))
    x = W.bf16(W.normal((T, N), 1.0, 22, DEV))
    dytq = U.ufp4_rht_quantize(dy, U.BLOCKS_ALONG_ROWS, True, 0x0F0F)
    xtq = U.ufp4_rht_quantize(x, U.BLOCKS_ALONG_ROWS, True, 0x0F0F)
    need = U.ufp4_workspace_size(U.WGRAD, M, N, dytq.kpad)
    assert need > 0
    small = torch.empty(need // 8, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    assert torch.equal(U.ufp4_gemm_wgrad(dytq, xtq, workspace=small),
                       U.ufp4_gemm_wgrad(dytq, xtq))
