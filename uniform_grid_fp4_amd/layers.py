"""Linear and MoE expert layers whose three training GEMMs run in UFP4.

The recipe (paperlayer.ai summary of "Rethinking Shrinkage Bias in LLM FP4
Pretraining", section 4 "UFP4 Recipe"): every GEMM contracts operands that
were rotated by the 16-point RHT along its reduction dimension and quantized
onto the uniform 4-bit grid; dY uses stochastic rounding, X and W
round-to-nearest-even.  One sign mask per GEMM is shared by its two operands
so the rotation cancels (section 2 "Random Hadamard transforms").

Everything runs in libufp4's kernels through the C ABI: per tensor one
dual-axis quantization (both of its operands from one read), the GEMMs write
bf16 directly (the epilogue rounds to nearest even), and only the 4-bit
operands the backward pass needs (X^T and W^T, 0.75 B per element) are kept
between forward and backward.  Masks are drawn once per layer from its seed;
the SR seed advances every forward call, so each step's rounding noise is
independent.

The recipe ablations of the same summary (section 5 "Q4: Recipe
ablations": RHT on the weight-gradient GEMM only, on FPROP and WGRAD, on
DGRAD and WGRAD; stochastic rounding of dY on or off) are layer options:
`rht` = (FPROP, DGRAD, WGRAD) flags, each applied to both operands of that
GEMM, and `sr_dy`.
"""
from __future__ import annotations

import numpy as np
import torch

from . import ufp4 as U


def draw_sign_masks(seed: int):
    """Three 16-bit RHT sign masks (FPROP, DGRAD, WGRAD) from a seed."""
    m = np.random.default_rng(seed).integers(0, 1 << 16, size=3)
    return int(m[0]), int(m[1]), int(m[2])


def _rows(t: torch.Tensor) -> torch.Tensor:
    t = t.reshape(-1, t.shape[-1])
    return t if t.stride(-1) == 1 else t.contiguous()


def _recipe(rht, sr_dy):
    """(FPROP, DGRAD, WGRAD) RHT flags as bools and the rounding of dY."""
    rf, rd, rw = (bool(r) for r in rht)
    return (rf, rd, rw), (U.ROUND_SR if sr_dy else U.ROUND_RTNE)


class _LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, masks, grid, seed, rht, rnd_dy):
        mf, md, mw = masks
        rf, rd, rw = rht
        xq, xtq = U.ufp4_rht_quantize_dual(x, (rf, mf, 0), (rw, mw, 0), grid=grid)
        wq, wtq = U.ufp4_rht_quantize_dual(w, (rf, mf, 0), (rd, md, 0), grid=grid)
        y = U.ufp4_gemm_out(U.FPROP, xq, wq, torch.bfloat16)
        ctx.q = (xtq, wtq)
        ctx.masks, ctx.grid, ctx.seed, ctx.rht, ctx.rnd_dy = masks, grid, seed, rht, rnd_dy
        return y

    @staticmethod
    def backward(ctx, dy):
        _, md, mw = ctx.masks
        _, rd, rw = ctx.rht
        dyq, dytq = U.ufp4_rht_quantize_dual(_bf16_rows(dy), (rd, md, 0), (rw, mw, 1),
                                             grid=ctx.grid, rnd=ctx.rnd_dy, seed=ctx.seed)
        xtq, wtq = ctx.q
        ctx.q = None
        dx = U.ufp4_gemm_out(U.DGRAD, dyq, wtq, torch.bfloat16)
        dw = U.ufp4_gemm_out(U.WGRAD, dytq, xtq, torch.bfloat16)
        return dx, dw, None, None, None, None, None


def _bf16_rows(t: torch.Tensor) -> torch.Tensor:
    if t.dtype != torch.bfloat16:
        raise TypeError(f"UFP4 layers take bf16 activations and gradients, got {t.dtype}")
    return _rows(t)


class UFP4Linear(torch.nn.Module):
    """y = x W^T, weight [out_features, in_features] in bf16; x is bf16
    [..., in_features]; the output and both gradients are bf16.  `rht`
    (FPROP, DGRAD, WGRAD) and `sr_dy` select the recipe; the default is the
    UFP4 recipe (RHT on all three GEMMs, SR on dY)."""

    def __init__(self, in_features: int, out_features: int, seed: int = 0,
                 grid: int = U.GRID_UNIFORM, device=None, rht=(True, True, True),
                 sr_dy: bool = True):
        super().__init__()
        w = torch.empty((out_features, in_features), device=device, dtype=torch.bfloat16)
        torch.nn.init.normal_(w, std=in_features ** -0.5)
        self.weight = torch.nn.Parameter(w)
        self.masks = draw_sign_masks(seed)
        self.grid = grid
        self.rht, self.rnd_dy = _recipe(rht, sr_dy)
        self.sr_seed = (seed * 0x9E3779B97F4A7C15) & ((1 << 64) - 1)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        self.sr_seed = (self.sr_seed + 1) & ((1 << 64) - 1)
        y = _LinearFn.apply(_bf16_rows(x), self.weight, self.masks, self.grid, self.sr_seed,
                            self.rht, self.rnd_dy)
        return y.reshape(*lead, y.shape[-1])


class _ExpertFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, offsets, n_experts, masks, grid, seed, rht, rnd_dy):
        mf, md, mw = masks
        rf, rd, rw = rht
        xq, xtq = U.ufp4_rht_quantize_dual(x, (rf, mf, 0), (rw, mw, 0), grid=grid,
                                           group_offsets=offsets)
        wq, wtq = U.ufp4_rht_quantize_dual(w, (rf, mf, 0), (rd, md, 0), grid=grid,
                                           col_axis=U.BLOCKS_ALONG_ROWS_STACKED,
                                           n_groups=n_experts)
        y = U.ufp4_grouped_gemm_out(U.FPROP, offsets, xq, wq, torch.bfloat16)
        ctx.q = (xtq, wtq)
        ctx.offsets, ctx.masks, ctx.grid, ctx.seed = offsets, masks, grid, seed
        ctx.rht, ctx.rnd_dy = rht, rnd_dy
        return y

    @staticmethod
    def backward(ctx, dy):
        _, md, mw = ctx.masks
        _, rd, rw = ctx.rht
        dyq, dytq = U.ufp4_rht_quantize_dual(_bf16_rows(dy), (rd, md, 0), (rw, mw, 1),
                                             grid=ctx.grid, rnd=ctx.rnd_dy, seed=ctx.seed,
                                             group_offsets=ctx.offsets)
        xtq, wtq = ctx.q
        ctx.q = None
        dx = U.ufp4_grouped_gemm_out(U.DGRAD, ctx.offsets, dyq, wtq, torch.bfloat16)
        dw = U.ufp4_grouped_gemm_out(U.WGRAD, ctx.offsets, dytq, xtq, torch.bfloat16)
        dw = dw.reshape(-1, dw.shape[-1])
        return dx, dw, None, None, None, None, None, None, None


class UFP4ExpertLinear(torch.nn.Module):
    """The expert layer of an MoE block: tokens arrive sorted by expert with
    device int64 offsets [n_experts + 1] (first 0, last = tokens; empty
    experts allowed) and expert e applies its own weight W_e [out, in]:
    y[off_e:off_{e+1}] = x[off_e:off_{e+1}] W_e^T.  Weights are stored
    stacked, [n_experts * out_features, in_features], in bf16.  `rht` and
    `sr_dy` as for UFP4Linear."""

    def __init__(self, n_experts: int, in_features: int, out_features: int, seed: int = 0,
                 grid: int = U.GRID_UNIFORM, device=None, rht=(True, True, True),
                 sr_dy: bool = True):
        super().__init__()
        w = torch.empty((n_experts * out_features, in_features), device=device,
                        dtype=torch.bfloat16)
        torch.nn.init.normal_(w, std=in_features ** -0.5)
        self.weight = torch.nn.Parameter(w)
        self.n_experts = n_experts
        self.masks = draw_sign_masks(seed)
        self.grid = grid
        self.rht, self.rnd_dy = _recipe(rht, sr_dy)
        self.sr_seed = (seed * 0x9E3779B97F4A7C15) & ((1 << 64) - 1)

    def forward(self, x: torch.Tensor, offsets: torch.Tensor) -> torch.Tensor:
        assert offsets.dtype == torch.int64 and offsets.numel() == self.n_experts + 1
        self.sr_seed = (self.sr_seed + 1) & ((1 << 64) - 1)
        return _ExpertFn.apply(_bf16_rows(x), self.weight, offsets, self.n_experts, self.masks,
                               self.grid, self.sr_seed, self.rht, self.rnd_dy)
