"""The linear and MoE expert layer wrappers: forward and backward equal the
explicit sequence of C-ABI calls bit for bit (dual-axis quantizations with
the layer's masks and SR seed, GEMMs with the bf16 epilogue), match the
oracle element by element (its quantizer on the same bf16 inputs, masks and
SR seed, then its FP64 GEMMs: |out - C| <= 1e-5 * sum_k |a_k||b_k| plus half a
bf16 ulp of the output for the epilogue's rounding), and stay within 4-bit
quantization noise of the unquantized product.  The recipe the layers follow
is the paperlayer.ai summary's section 4 "UFP4 Recipe" (RHT on all three
GEMMs along their contraction dimensions, stochastic rounding on dY only);
its section 5 "Q4" ablations (RHT on a subset of the GEMMs, dY without SR)
are layer options checked the same way."""
import numpy as np
import pytest
import torch

from oracle import ufp4_oracle as O
from uniform_grid_fp4_amd import ufp4 as U
from uniform_grid_fp4_amd import workloads as W
from uniform_grid_fp4_amd.layers import UFP4ExpertLinear, UFP4Linear

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-5


def assert_bf16_close(out, C, bound, what):
    """out: bf16 GEMM output (the FP32 result v rounded to nearest even);
    C, bound: the oracle's FP64 product and sum |a||b|.  |v - C| <= TOL*bound,
    and the rounding adds at most half a bf16 ulp of v, <= 2^-8 |v|."""
    o = out.detach().float().cpu().numpy().astype(np.float64)
    lim = TOL * bound + 2.0 ** -8 * (np.abs(C) + TOL * bound)
    err = np.abs(o - C)
    bad = err > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside, worst ratio "
                           f"{(err / np.maximum(lim, 1e-300)).max():.3g}")


def oracle_linear(x, w, g, masks, seed, grid=O.GRID_UNIFORM, rht=(True, True, True), rnd_dy=1):
    """The oracle's three GEMMs of a linear layer: the six quantized operands
    (X and W along H, dY along F with stream 0, W^T along F, dY^T with stream
    1 and X^T along the tokens; each GEMM's pair with its RHT flag, dY with
    rounding rnd_dy) and FP64 products."""
    mf, md, mw = masks
    rf, rd, rw = rht
    xb, wb, gb = W.bits_numpy(x), W.bits_numpy(w), W.bits_numpy(g)
    q = lambda b, axis, r, mask, rnd=0, sid=0: O.quantize(b, axis, r, mask, grid, rnd, seed, sid)
    cx, sx, _ = q(xb, O.AXIS_COLS, rf, mf)
    cw, sw, _ = q(wb, O.AXIS_COLS, rf, mf)
    cg, sg, _ = q(gb, O.AXIS_COLS, rd, md, rnd_dy, 0)
    cwt, swt, _ = q(wb, O.AXIS_ROWS, rd, md)
    cgt, sgt, _ = q(gb, O.AXIS_ROWS, rw, mw, rnd_dy, 1)
    cxt, sxt, _ = q(xb, O.AXIS_ROWS, rw, mw)
    return (O.gemm_tn(cx, sx, cw, sw, grid), O.gemm_tn(cg, sg, cwt, swt, grid),
            O.gemm_tn(cgt, sgt, cxt, sxt, grid))


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
    # the oracle, element by element, on the same inputs, masks and SR seed
    (Cy, By), (Cdx, Bdx), (Cdw, Bdw) = oracle_linear(x2, w, g2, layer.masks, layer.sr_seed)
    assert_bf16_close(y.reshape(-1, 384), Cy, By, "linear fprop")
    assert_bf16_close(x.grad.reshape(-1, 256), Cdx, Bdx, "linear dgrad")
    assert_bf16_close(layer.weight.grad, Cdw, Bdw, "linear wgrad")
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
    # the oracle, element by element: grouped quantizations (per-expert
    # padding along the tokens, stacked per-expert W^T) and grouped FP64 GEMMs
    o = off.tolist()
    xb, wb, gb = W.bits_numpy(x.detach()), W.bits_numpy(w), W.bits_numpy(g)
    seed, grid = layer.sr_seed, O.GRID_UNIFORM
    kp = U.padded_k_capacity(T, E)
    q = lambda b, axis, mask, rnd=0, sid=0, **kw: O.quantize(b, axis, True, mask, grid, rnd,
                                                             seed, sid, **kw)
    cx, sx, _ = q(xb, O.AXIS_COLS, mf)
    cw, sw, _ = q(wb, O.AXIS_COLS, mf)
    cg, sg, _ = q(gb, O.AXIS_COLS, md, 1, 0)
    cwt, swt, _ = q(wb, O.AXIS_ROWS_STACKED, md, n_stack=E)
    cgt, sgt, _ = q(gb, O.AXIS_ROWS, mw, 1, 1, group_offsets=o, kpad=kp)
    cxt, sxt, _ = q(xb, O.AXIS_ROWS, mw, group_offsets=o, kpad=kp)
    Cy, By = O.grouped_gemm(0, o, cx, sx, cw, sw, F, grid)
    Cdx, Bdx = O.grouped_gemm(1, o, cg, sg, cwt, swt, H, grid)
    Cdw, Bdw = O.grouped_gemm(2, o, cgt, sgt, cxt, sxt, H, grid)
    assert_bf16_close(y, Cy, By, "expert fprop")
    assert_bf16_close(x.grad, Cdx, Bdx, "expert dgrad")
    assert_bf16_close(layer.weight.grad, Cdw.reshape(E * F, H), Bdw.reshape(E * F, H),
                      "expert wgrad")
    assert not Cdw[1].any()
    for e in range(E):
        if counts[e] == 0:
            continue
        xe, ge = x.detach()[o[e]:o[e + 1]].float(), g[o[e]:o[e + 1]].float()
        we = w[e * F:(e + 1) * F].float()
        assert rel_rms(y[o[e]:o[e + 1]], xe @ we.t()) < 0.25
        if counts[e] >= 16:
            assert rel_rms(x.grad[o[e]:o[e + 1]], ge @ we) < 0.3
            assert rel_rms(layer.weight.grad[e * F:(e + 1) * F], ge.t() @ xe) < 0.3


@pytest.mark.parametrize("rht,sr_dy", [((False, False, True), True), ((True, False, True), True),
                                       ((False, True, True), True), ((True, True, True), False),
                                       ((False, False, False), False)])
def test_linear_layer_recipe_ablations(rht, sr_dy):
    """The recipe ablations of the paperlayer.ai summary, section 5 "Q4":
    RHT on WGRAD only, on FPROP and WGRAD, on DGRAD and WGRAD, full RHT
    without SR on dY, and neither.  Each GEMM's operands carry that GEMM's
    flag; forward and both gradients equal the explicit C-ABI sequence and
    match the oracle element by element."""
    torch.manual_seed(2)
    layer = UFP4Linear(128, 96, seed=4, device=DEV, rht=rht, sr_dy=sr_dy)
    x = torch.randn((80, 128), device=DEV).to(torch.bfloat16).requires_grad_(True)
    g = torch.randn((80, 96), device=DEV).to(torch.bfloat16)
    y = layer(x)
    y.backward(g)
    mf, md, mw = layer.masks
    rf, rd, rw = rht
    rnd = U.ROUND_SR if sr_dy else U.ROUND_RTNE
    w = layer.weight.detach()
    xq, xtq = U.ufp4_rht_quantize_dual(x.detach(), (rf, mf, 0), (rw, mw, 0))
    wq, wtq = U.ufp4_rht_quantize_dual(w, (rf, mf, 0), (rd, md, 0))
    dq, dtq = U.ufp4_rht_quantize_dual(g, (rd, md, 0), (rw, mw, 1), rnd=rnd, seed=layer.sr_seed)
    assert (xq.rht, xtq.rht, dq.rht, dtq.rht) == (int(rf), int(rw), int(rd), int(rw))
    assert torch.equal(y, U.ufp4_gemm_out(U.FPROP, xq, wq))
    assert torch.equal(x.grad, U.ufp4_gemm_out(U.DGRAD, dq, wtq))
    assert torch.equal(layer.weight.grad, U.ufp4_gemm_out(U.WGRAD, dtq, xtq))
    (Cy, By), (Cdx, Bdx), (Cdw, Bdw) = oracle_linear(x.detach(), w, g, layer.masks,
                                                     layer.sr_seed, rht=rht,
                                                     rnd_dy=1 if sr_dy else 0)
    assert_bf16_close(y, Cy, By, "fprop")
    assert_bf16_close(x.grad, Cdx, Bdx, "dgrad")
    assert_bf16_close(layer.weight.grad, Cdw, Bdw, "wgrad")


def test_expert_layer_recipe_ablation():
    """The expert layer with RHT on WGRAD only and round-to-nearest dY."""
    torch.manual_seed(3)
    counts = [30, 0, 50, 17]
    E, H, F = len(counts), 64, 48
    off = torch.as_tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int64, device=DEV)
    T = sum(counts)
    layer = UFP4ExpertLinear(E, H, F, seed=6, device=DEV, rht=(False, False, True), sr_dy=False)
    x = torch.randn((T, H), device=DEV).to(torch.bfloat16).requires_grad_(True)
    g = torch.randn((T, F), device=DEV).to(torch.bfloat16)
    y = layer(x, off)
    y.backward(g)
    mf, md, mw = layer.masks
    o = off.tolist()
    w = layer.weight.detach()
    xb, wb, gb = W.bits_numpy(x.detach()), W.bits_numpy(w), W.bits_numpy(g)
    grid = O.GRID_UNIFORM
    kp = U.padded_k_capacity(T, E)
    cx, sx, _ = O.quantize(xb, O.AXIS_COLS, False, mf, grid, 0)
    cw, sw, _ = O.quantize(wb, O.AXIS_COLS, False, mf, grid, 0)
    cg, sg, _ = O.quantize(gb, O.AXIS_COLS, False, md, grid, 0)
    cwt, swt, _ = O.quantize(wb, O.AXIS_ROWS_STACKED, False, md, grid, 0, n_stack=E)
    cgt, sgt, _ = O.quantize(gb, O.AXIS_ROWS, True, mw, grid, 0, layer.sr_seed, 1,
                             group_offsets=o, kpad=kp)
    cxt, sxt, _ = O.quantize(xb, O.AXIS_ROWS, True, mw, grid, 0, group_offsets=o, kpad=kp)
    Cy, By = O.grouped_gemm(0, o, cx, sx, cw, sw, F, grid)
    Cdx, Bdx = O.grouped_gemm(1, o, cg, sg, cwt, swt, H, grid)
    Cdw, Bdw = O.grouped_gemm(2, o, cgt, sgt, cxt, sxt, H, grid)
    assert_bf16_close(y, Cy, By, "expert fprop")
    assert_bf16_close(x.grad, Cdx, Bdx, "expert dgrad")
    assert_bf16_close(layer.weight.grad, Cdw.reshape(E * F, H), Bdw.reshape(E * F, H),
                      "expert wgrad")
