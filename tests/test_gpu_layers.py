"""The linear and MoE expert layer wrappers: forward and backward equal the
explicit sequence of C-ABI calls bit for bit (dual-axis quantizations with
the layer's masks and SR seed, GEMMs with the bf16 epilogue), and stay within
4-bit quantization noise of the unquantized product."""
import numpy as np
import pytest
import torch

from uniform_grid_fp4_amd import ufp4 as U
from uniform_grid_fp4_amd.layers import UFP4ExpertLinear, UFP4Linear

pytestmark = pytest.mark.gpu
DEV = "cuda"


def rel_rms(a, b):
    a, b = a.detach().float(), b.detach().float()
    return float(((a - b) ** 2).mean().sqrt() / (b ** 2).mean().sqrt())


def test_linear_layer():
    torch.manual_seed(0)
    layer = UFP4Linear(256, 384, seed=3, device=DEV)
    x = torch.randn((2, 64, 256), device=DEV).to(torch.bfloat16).requires_grad_(True)
    g = torch.randn((2, 64, 384), device=DEV).to(torch.bfloat16)
    y = layer(x)
    y.backward(g)
    assert y.dtype == x.grad.dtype == layer.weight.grad.dtype == torch.bfloat16
    # the same computation through the library calls
    mf, md, mw = layer.masks
    x2, w, g2 = x.detach().reshape(-1, 256), layer.weight.detach(), g.reshape(-1, 384)
    xq, xtq = U.ufp4_rht_quantize_dual(x2, (True, mf, 0), (True, mw, 0))
    wq, wtq = U.ufp4_rht_quantize_dual(w, (True, mf, 0), (True, md, 0))
    dq, dtq = U.ufp4_rht_quantize_dual(g2, (True, md, 0), (True, mw, 1), rnd=U.ROUND_SR,
                                       seed=layer.sr_seed)
    assert torch.equal(y.reshape(-1, 384), U.ufp4_gemm_out(U.FPROP, xq, wq))
    assert torch.equal(x.grad.reshape(-1, 256), U.ufp4_gemm_out(U.DGRAD, dq, wtq))
    assert torch.equal(layer.weight.grad, U.ufp4_gemm_out(U.WGRAD, dtq, xtq))
    # and it is the product it stands for, up to 4-bit noise
    xf, wf, gf = x2.float(), w.float(), g2.float()
    assert rel_rms(y.reshape(-1, 384), xf @ wf.t()) < 0.2
    assert rel_rms(x.grad.reshape(-1, 256), gf @ wf) < 0.25
    assert rel_rms(layer.weight.grad, gf.t() @ xf) < 0.25
    # the SR seed advances per call
    s0 = layer.sr_seed
    layer(x)
    assert layer.sr_seed != s0


def test_linear_layer_rejects_other_dtypes():
    layer = UFP4Linear(32, 32, device=DEV)
    with pytest.raises(TypeError):
        layer(torch.zeros((4, 32), device=DEV))


def test_expert_layer():
    torch.manual_seed(1)
    counts = [40, 0, 70, 18, 1]
    E, H, F = len(counts), 128, 96
    off = torch.as_tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int64, device=DEV)
    T = sum(counts)
    layer = UFP4ExpertLinear(E, H, F, seed=5, device=DEV)
    x = torch.randn((T, H), device=DEV).to(torch.bfloat16).requires_grad_(True)
    g = torch.randn((T, F), device=DEV).to(torch.bfloat16)
    y = layer(x, off)
    y.backward(g)
    mf, md, mw = layer.masks
    w = layer.weight.detach()
    xq, xtq = U.ufp4_rht_quantize_dual(x.detach(), (True, mf, 0), (True, mw, 0),
                                       group_offsets=off)
    wq, wtq = U.ufp4_rht_quantize_dual(w, (True, mf, 0), (True, md, 0),
                                       col_axis=U.BLOCKS_ALONG_ROWS_STACKED, n_groups=E)
    dq, dtq = U.ufp4_rht_quantize_dual(g, (True, md, 0), (True, mw, 1), rnd=U.ROUND_SR,
                                       seed=layer.sr_seed, group_offsets=off)
    assert torch.equal(y, U.ufp4_grouped_gemm_out(U.FPROP, off, xq, wq))
    assert torch.equal(x.grad, U.ufp4_grouped_gemm_out(U.DGRAD, off, dq, wtq))
    dw = U.ufp4_grouped_gemm_out(U.WGRAD, off, dtq, xtq).reshape(E * F, H)
    assert torch.equal(layer.weight.grad, dw)
    assert (layer.weight.grad[F:2 * F] == 0).all()            # the expert with no tokens
    o = off.tolist()
    for e in range(E):
        if counts[e] == 0:
            continue
        xe, ge = x.detach()[o[e]:o[e + 1]].float(), g[o[e]:o[e + 1]].float()
        we = w[e * F:(e + 1) * F].float()
        assert rel_rms(y[o[e]:o[e + 1]], xe @ we.t()) < 0.25
        if counts[e] >= 16:
            assert rel_rms(x.grad[o[e]:o[e + 1]], ge @ we) < 0.3
            assert rel_rms(layer.weight.grad[e * F:(e + 1) * F], ge.t() @ xe) < 0.3
