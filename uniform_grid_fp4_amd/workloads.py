"""Seeded synthetic workloads shaped like the pages' dense and MoE layers.

This module only draws random inputs; it holds none of the quantizer's or the
GEMM's arithmetic, so tests can feed the same tensors to the HIP library and
to the CPU oracle.

Shapes follow the dense 1.5B and MoE 7.9B / 124B models the paper trains
(paperlayer.ai summary, section 5 "Q2-Q3: Long-run training and scaling");
the pages give no tensor statistics, so the value distributions are synthetic
stand-ins: activations N(0, 1) with a few outlier input channels (the pages
call linear_fc2 inputs outlier heavy, section 5 "Q1: Grid geometry and RHT"),
weights N(0, 0.02), output gradients N(0, 1e-4).  All draws use torch
generators seeded per tensor, on the device the caller names, and are rounded
to bf16 by torch (round to nearest even).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

SEED = 0


@dataclass
class Layer:
    """One linear (or expert-grouped) layer's operands, all bf16 tensors.

    x  [tokens, hidden]     activations (FPROP A, WGRAD B after transpose)
    w  [experts*ffn, hidden] weights, experts stacked (FPROP B, DGRAD B^T)
    dy [tokens, ffn]        output gradient (DGRAD A, WGRAD A after transpose)
    offsets: int64 group offsets over tokens (len experts+1), [0, T] if dense.
    masks: RHT sign masks for FPROP, DGRAD, WGRAD.
    """
    name: str
    x: torch.Tensor
    w: torch.Tensor
    dy: torch.Tensor
    offsets: np.ndarray
    masks: tuple
    experts: int
    hidden: int
    ffn: int
    seed: int = SEED
    extra: dict = field(default_factory=dict)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std: float, seed: int, device="cpu") -> torch.Tensor:
    out = torch.empty(shape, dtype=torch.float32, device=device)
    out.normal_(0.0, std, generator=_gen(device, seed))
    return out


def laplace(shape, b: float, seed: int, device="cpu") -> torch.Tensor:
    """Laplace(0, b) as the difference of two unit exponentials."""
    g = _gen(device, seed)
    e1 = torch.empty(shape, device=device).exponential_(1.0, generator=g)
    e2 = torch.empty(shape, device=device).exponential_(1.0, generator=g)
    return (e1 - e2) * b


def student_t3(shape, seed: int, device="cpu") -> torch.Tensor:
    """Student t with 3 degrees of freedom: z0 / sqrt((z1^2 + z2^2 + z3^2)/3)."""
    g = _gen(device, seed)
    z = [torch.empty(shape, device=device).normal_(0.0, 1.0, generator=g) for _ in range(4)]
    chi = (z[1] * z[1] + z[2] * z[2] + z[3] * z[3]) / 3.0
    return z[0] / torch.sqrt(chi)


def with_outlier_channels(x: torch.Tensor, frac: float, factor: float, seed: int) -> torch.Tensor:
    """Scale round(frac * hidden) input channels, picked by a seeded permutation."""
    h = x.shape[1]
    n = int(round(frac * h))
    rng = np.random.default_rng(seed + 1000)
    ch = np.sort(rng.permutation(h)[:n])
    x[:, torch.as_tensor(ch, device=x.device)] *= factor
    return x


def zipf_counts(experts: int, total: int, s: float, seed: int) -> np.ndarray:
    """Per-expert token counts: a multinomial of `total` picks over
    p_e ~ e^-s (e = 1..E), expert 0 the heaviest; counts may be zero."""
    p = np.arange(1, experts + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    return np.random.default_rng(seed).multinomial(total, p).astype(np.int64)


def sign_masks(seed: int):
    """16-bit RHT sign masks for FPROP, DGRAD and WGRAD, drawn from the seed."""
    rng = np.random.default_rng(seed + 77)
    return tuple(int(v) for v in rng.integers(0, 1 << 16, size=3))


def bf16(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.bfloat16)


def bits_numpy(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dense_layer(tokens: int, hidden: int, ffn: int, outlier_frac: float,
                outlier_factor: float, seed: int = SEED, device="cpu", name="dense") -> Layer:
    x = normal((tokens, hidden), 1.0, seed + 1, device)
    if outlier_frac > 0:
        x = with_outlier_channels(x, outlier_frac, outlier_factor, seed)
    w = normal((ffn, hidden), 0.02, seed + 2, device)
    dy = normal((tokens, ffn), 1e-4, seed + 3, device)
    return Layer(name, bf16(x), bf16(w), bf16(dy), np.array([0, tokens], dtype=np.int64),
                 sign_masks(seed), 1, hidden, ffn, seed)


def moe_layer(experts: int, hidden: int, ffn: int, tokens_routed: int,
              outlier_frac: float, outlier_factor: float, seed: int = SEED,
              device="cpu", name="moe", counts=None) -> Layer:
    if counts is None:
        counts = zipf_counts(experts, tokens_routed, 1.1, seed)
    counts = np.asarray(counts, dtype=np.int64)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    t = int(off[-1])
    x = normal((t, hidden), 1.0, seed + 1, device)
    if outlier_frac > 0:
        x = with_outlier_channels(x, outlier_frac, outlier_factor, seed)
    w = normal((experts * ffn, hidden), 0.02, seed + 2, device)
    dy = normal((t, ffn), 1e-4, seed + 3, device)
    return Layer(name, bf16(x), bf16(w), bf16(dy), off, sign_masks(seed), experts,
                 hidden, ffn, seed, {"counts": counts})


# The five workloads.  `tiny` is the small case the oracle finishes in
# seconds; `dense_1p5b` is one linear layer of the dense 1.5B model
# (4 x 2048 tokens, hidden 2048, FFN 8192); `sweep` is the 2^28-element
# quantizer sweep; `moe_7p9b` and `moe_124b` are expert layers (the latter is
# one GPU's share: 32 resident experts, all 65536 x top-8 routed rows).
def tiny(device="cpu", seed: int = SEED) -> Layer:
    return dense_layer(256, 256, 256, 0.0, 1.0, seed, device, "tiny-256")


def dense_1p5b(device="cpu", seed: int = SEED) -> Layer:
    return dense_layer(8192, 2048, 8192, 0.01, 50.0, seed, device, "dense-1.5B-fc1")


def moe_7p9b(device="cpu", seed: int = SEED) -> Layer:
    return moe_layer(64, 2048, 1408, 16384 * 6, 0.01, 50.0, seed, device, "moe-7.9B-experts")


def moe_124b(device="cpu", seed: int = SEED) -> Layer:
    return moe_layer(32, 6144, 2048, 65536 * 8, 0.005, 100.0, seed, device, "moe-124B-experts-1gpu")


SWEEP_SHAPE = (16384, 16384)
SWEEP_DISTS = ("gaussian", "laplace", "student_t3")


def sweep_tensor(dist: str, device="cpu", shape=SWEEP_SHAPE) -> torch.Tensor:
    """Quantizer sweep input: Gaussian (seed 0), Laplace b=1 (seed 1),
    Student-t nu=3 (seed 2)."""
    if dist == "gaussian":
        x = normal(shape, 1.0, 0, device)
    elif dist == "laplace":
        x = laplace(shape, 1.0, 1, device)
    elif dist == "student_t3":
        x = student_t3(shape, 2, device)
    else:
        raise ValueError(dist)
    return bf16(x)
