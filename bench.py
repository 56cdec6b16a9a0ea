"""Throughput of the UFP4 hot path on one MI355X.

A step is one pass of the whole path over one layer: the six quantized
operands of the UFP4 recipe (X and W along H for FPROP; dY along F with
stochastic rounding and W along F for DGRAD; dY and X along the tokens for
WGRAD, dY with stochastic rounding) and the three block-scaled 4-bit GEMMs.
By default the layer is the MoE-124B expert layer at one GPU's share (32
resident experts, hidden 6144, expert FFN 2048, 65536 tokens routed top-8
with Zipf(1.1) counts: 524288 expert rows), with the grouped GEMMs;
`--workload dense-1.5b` runs the dense 1.5B-model linear layer (tokens 8192,
hidden 2048, FFN 8192) and `moe-7.9b` the 7.9B expert layer.  The operands
come from three dual-axis quantizations (one read of X, W and dY each, both
of the tensor's operands out; bit-identical to the six single-axis calls,
which `--quantizer single` runs instead).  Inputs are synthetic (seeded, see
uniform_grid_fp4_amd/workloads.py) and resident in HBM before the timed
region.

Prints one JSON line.  `value` is the whole step's throughput in GEMM
TFLOP/s (3 x 2*T*H*F FLOP per step over the wall time of the step, the
quantizations included).  The step is captured once as a HIP graph and the
timed steps are replays of it (checked bit-identical to the eager step
first; `--eager` times eager launches instead).  Each kernel is also timed on
its own: an eager pass of back-to-back steps records HIP events around every
launch, on the stream the library launches on, and the reported durations
are medians over the steps.  The per-kernel figures are labelled "cold" when
every input tensor the quantizers read is at least twice the 256 MB MALL (so
each step streams it from HBM, and each launch also pays for writing back the
previous launch's outputs, as in a real step), else "warm".
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_MFMA_PEAK_TFLOPS = 5000.0  # dense FP8 MFMA
# The GEMM's work per unit of one 32x32 output tile and one 16-element block
# (32768 FLOP): one v_mfma_f32_32x32x16_fp8_fp8 for the exact block product
# (32 matrix-core cycles), half of one v_mfma_f32_32x32x1_2b_f32 for the FP32
# scale products of a 32 x 64 wave tile (64 cycles for both 32x32 halves) and
# 16 vector FMAs acc += S * P (4 issue cycles per wave64 instruction).  The
# matrix core and the vector ALU each need 64 cycles per unit, so the ceiling
# of this instruction mix is 32768 FLOP / 64 cycles x 1024 SIMDs x 2.4 GHz =
# 1258.3 TFLOP/s (a quarter of the 5.0 PFLOP/s FP8 MFMA peak).
SIMDS = 256 * 4
GEMM_UNIT_CYCLES = 64
GEMM_PIPE_PEAK_TFLOPS = 32 * 32 * 16 * 2 / GEMM_UNIT_CYCLES * SIMDS * 2.4e9 / 1e12
BYTES_PER_QUANT_ELEM = 2.0 + 0.5 + 0.25
BYTES_PER_DUAL_ELEM = 2.0 + 2 * (0.5 + 0.25)

# HBM bytes from the rocprofv3 FETCH_SIZE and WRITE_SIZE counters, each
# scaled by the factor that makes the same counter read the known size of a
# plain 1 GiB device copy: per GEMM launch (averaged over the FPROP, DGRAD
# and WGRAD launches of one step) and per step of quantizations.  A figure
# holds for the sources whose SHA-256 is recorded with it; after any change to
# them the bench reports null until the counters are taken again.
TRAFFIC = {
    "moe-124B-experts-1gpu": {
        "gemm": {"sha256": "b3756901f52a1a4c3c0785f07446f908dc12bacf7b04ccc17bb3e0d119e6a19f",
                 "bytes_per_launch": 22459143930},
        "quantize": {"sha256": "9bc2220e9251f951c8558751186c15ffbc050a44615921d8983718693798e53f",
                     "bytes_per_step": 16904243057},
    },
}
# The kernels, the host code that launches them and chooses split-K, the
# binding that sets the output layouts (the grouped row length) and the
# workload shapes: a change to any of them can change the bytes moved.
_HOST_SOURCES = ("uniform_grid_fp4_amd/csrc/api.hip", "uniform_grid_fp4_amd/ufp4.py",
                 "uniform_grid_fp4_amd/workloads.py")
GEMM_SOURCES = ("uniform_grid_fp4_amd/csrc/gemm.hip", "uniform_grid_fp4_amd/csrc/ufp4_device.h",
                "uniform_grid_fp4_amd/csrc/ufp4_kernels.h") + _HOST_SOURCES
QUANT_SOURCES = ("uniform_grid_fp4_amd/csrc/quantize.hip",
                 "uniform_grid_fp4_amd/csrc/ufp4_device.h",
                 "uniform_grid_fp4_amd/csrc/ufp4_kernels.h") + _HOST_SOURCES
MALL_BYTES = 256 << 20          # MI355X Infinity Cache


def source_sha256(sources) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def gemm_source_sha256() -> str:
    return source_sha256(GEMM_SOURCES)


def measured_traffic(workload: str, part: str):
    """Counter-measured bytes of `part` ("gemm": per launch, "quantize": per
    step) for the current sources, or None."""
    rec = TRAFFIC.get(workload, {}).get(part)
    if rec is None:
        return None
    srcs = GEMM_SOURCES if part == "gemm" else QUANT_SOURCES
    if rec["sha256"] != source_sha256(srcs):
        return None
    return rec["bytes_per_launch"] if part == "gemm" else rec["bytes_per_step"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time the step as eager launches instead of replays of the step "
                         "captured once as a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--quantizer", default="dual", choices=["single", "dual"],
                    help="single: six single-axis quantizations per step; dual: three dual-axis "
                         "quantizations (one read of X, W and dY each, both operands out)")
    ap.add_argument("--workload", default="moe-124b",
                    choices=["moe-124b", "dense-1.5b", "moe-7.9b", "quant-sweep", "quant-2p28",
                             "copy", "q1-outputs", "mfma-peak"],
                    help="moe-124b: the timed step on the MoE-124B expert layer, one GPU's "
                         "share (default); dense-1.5b, moe-7.9b: the same step on the dense "
                         "1.5B linear layer or the MoE-7.9B expert layer; quant-sweep: the "
                         "2^28-element quantizer sweep, one JSON line per case; quant-2p28: the "
                         "UFP4 quantizer kernels alone on the sweep's Gaussian tensor (row- and "
                         "column-wise, RTNE and SR, and dual-axis), back to back; copy: a plain "
                         "1 GiB device copy, the "
                         "streaming ceiling and the calibration run of the HBM traffic "
                         "counters; q1-outputs: GEMM-output SQNR of each recipe against the "
                         "unquantized product, one JSON line per GEMM; mfma-peak: measured "
                         "rates of the candidate MFMA instructions")
    return ap.parse_args()


class Step:
    """Buffers and calls of one pass of the hot path."""

    def __init__(self, L, U, torch, dual=False):
        self.L, self.U, self.torch = L, U, torch
        self.dual = dual
        self.quant_names = self.QUANT_DUAL if dual else self.QUANT
        T, H, F = L.x.shape[0], L.hidden, L.ffn
        self.T, self.H, self.F = T, H, F
        self.mf, self.md, self.mw = L.masks
        dev = L.x.device
        self.y = torch.empty((T, F), dtype=torch.float32, device=dev)
        self.dx = torch.empty((T, H), dtype=torch.float32, device=dev)
        self.dw = torch.empty((F, H), dtype=torch.float32, device=dev)
        self.q = {}
        self.seed = 1234
        self.run(None)   # allocates the quantized buffers once

    def _start(self, ev, name):
        """Record the start event of launch `name` (per-kernel timing pass)."""
        if ev is not None:
            ev[name][0].record()

    def inputs_cold(self):
        """Whether every quantized input is at least twice the MALL."""
        L = self.L
        return all(t.numel() * t.element_size() >= 2 * MALL_BYTES for t in (L.x, L.w, L.dy))

    def quant(self, name, x, axis, mask, rnd, sid, ev):
        U = self.U
        self._start(ev, name)
        q = U.ufp4_rht_quantize(x, axis, True, mask, U.GRID_UNIFORM, rnd, self.seed, sid,
                                out=self.q.get(name))
        if ev is not None:
            ev[name][1].record()
        self.q[name] = q
        return q

    def quant2(self, name, x, rowwise, colwise, rnd, ev, **kw):
        """Both operands of x from one read (dual-axis quantizer)."""
        U = self.U
        self._start(ev, name)
        prev = self.q.get(name, (None, None))
        q = U.ufp4_rht_quantize_dual(x, rowwise, colwise, grid=U.GRID_UNIFORM, rnd=rnd,
                                     seed=self.seed, out_rows=prev[0], out_cols=prev[1], **kw)
        if ev is not None:
            ev[name][1].record()
        self.q[name] = q
        return q

    def gemm(self, name, fn, a, b, out, ev):
        self._start(ev, name)
        fn(a, b, out=out)
        if ev is not None:
            ev[name][1].record()

    def run(self, ev):
        U, L = self.U, self.L
        C, R = U.BLOCKS_ALONG_COLS, U.BLOCKS_ALONG_ROWS
        if self.dual:
            xq, xtq = self.quant2("q_x_dual", L.x, (True, self.mf, 0), (True, self.mw, 0),
                                  U.ROUND_RTNE, ev)
            wq, wtq = self.quant2("q_w_dual", L.w, (True, self.mf, 0), (True, self.md, 0),
                                  U.ROUND_RTNE, ev)
            self.gemm("fprop", U.ufp4_gemm_fprop, xq, wq, self.y, ev)
            dyq, dytq = self.quant2("q_dy_dual", L.dy, (True, self.md, 0), (True, self.mw, 1),
                                    U.ROUND_SR, ev)
            self.gemm("dgrad", U.ufp4_gemm_dgrad, dyq, wtq, self.dx, ev)
            self.gemm("wgrad", U.ufp4_gemm_wgrad, dytq, xtq, self.dw, ev)
            return
        xq = self.quant("q_x_fprop", L.x, C, self.mf, U.ROUND_RTNE, 0, ev)
        wq = self.quant("q_w_fprop", L.w, C, self.mf, U.ROUND_RTNE, 0, ev)
        self.gemm("fprop", U.ufp4_gemm_fprop, xq, wq, self.y, ev)
        dyq = self.quant("q_dy_dgrad", L.dy, C, self.md, U.ROUND_SR, 0, ev)
        wtq = self.quant("q_wt_dgrad", L.w, R, self.md, U.ROUND_RTNE, 0, ev)
        self.gemm("dgrad", U.ufp4_gemm_dgrad, dyq, wtq, self.dx, ev)
        dytq = self.quant("q_dyt_wgrad", L.dy, R, self.mw, U.ROUND_SR, 1, ev)
        xtq = self.quant("q_xt_wgrad", L.x, R, self.mw, U.ROUND_RTNE, 0, ev)
        self.gemm("wgrad", U.ufp4_gemm_wgrad, dytq, xtq, self.dw, ev)

    def outputs(self):
        """The step's GEMM outputs (they depend on every quantized operand)."""
        return [self.y, self.dx, self.dw]

    QUANT = ("q_x_fprop", "q_w_fprop", "q_dy_dgrad", "q_wt_dgrad", "q_dyt_wgrad", "q_xt_wgrad")
    QUANT_DUAL = ("q_x_dual", "q_w_dual", "q_dy_dual")
    GEMMS = ("fprop", "dgrad", "wgrad")

    def quant_elems(self):
        T, H, F = self.T, self.H, self.F
        return {"q_x_fprop": T * H, "q_w_fprop": F * H, "q_dy_dgrad": T * F,
                "q_wt_dgrad": F * H, "q_dyt_wgrad": T * F, "q_xt_wgrad": T * H,
                "q_x_dual": T * H, "q_w_dual": F * H, "q_dy_dual": T * F}

    def quant_bytes(self):
        """Algorithmic bytes of each quantizer call of the step: 2 B read and
        0.75 B written per element and output (two outputs for a dual call)."""
        el = self.quant_elems()
        return {n: el[n] * (BYTES_PER_DUAL_ELEM if n.endswith("_dual") else BYTES_PER_QUANT_ELEM)
                for n in self.quant_names}

    def gemm_flops(self):
        return 2.0 * self.T * self.H * self.F


def host_cpu_info():
    """Host CPU model, os.cpu_count() and the BLAS/OpenMP thread pools."""
    from threadpoolctl import threadpool_info
    pools = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in pools] + [1])
    blas = ", ".join(f"{i.get('internal_api', '?')} x{i.get('num_threads', '?')}" for i in pools)
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return int(threads), model, blas


def cpu_baseline(L, st, target_s: float):
    """The oracle on the host, on a bounded sample of the same workload.

    Quantizer: 64 sampled rows of X and dY quantized row-wise (RTNE and SR),
    and the first 4096 token rows x 64 columns of X and dY quantized
    column-wise (along the tokens); the oracle's elements per second are
    scaled to the step's 2 x (T*H + E*F*H + T*F) quantized elements.  GEMM:
    the FP64 FPROP of the first expert (or the dense layer) on 32-row samples
    of its output rows, scaled to the step's 3 x 2*T*H*F FLOP.  Inputs are
    copied to the host in slices only."""
    import numpy as np
    from oracle import ufp4_oracle as O
    from uniform_grid_fp4_amd import workloads as W

    mf, md, mw = L.masks
    H, F = L.hidden, L.ffn
    T = int(L.offsets[-1])
    c0 = int(L.offsets[1] - L.offsets[0])          # rows of the first group
    rows = np.arange(64)
    xr, dyr = W.bits_numpy(L.x[:64]), W.bits_numpy(L.dy[:64])
    tk = min(4096, c0)
    xc, dyc = W.bits_numpy(L.x[:tk, :64]), W.bits_numpy(L.dy[:tk, :64])
    t0 = time.perf_counter()
    n_el = 0
    for bits, axis, rnd in ((xr, 0, 0), (dyr, 0, 1), (xc, 1, 0), (dyc, 1, 1)):
        c, s, kp = O.quantize(bits, axis, True, mf, O.GRID_UNIFORM, rnd, 1234, 0,
                              out_rows=rows if axis == 0 else None)
        n_el += c.shape[0] * kp
        if time.perf_counter() - t0 > target_s / 2:
            break
    tq = time.perf_counter() - t0
    q_rate = n_el / tq
    # FP64 GEMM rate: FPROP of group 0 (B = that group's whole quantized W)
    cw, sw, _ = O.quantize(W.bits_numpy(L.w[:F]), 0, True, mf, O.GRID_UNIFORM, 0)
    nr = min(256, c0)
    cx, sx, _ = O.quantize(W.bits_numpy(L.x[:nr]), 0, True, mf, O.GRID_UNIFORM, 0)
    t1 = time.perf_counter()
    flops = 0.0
    done = 0
    while True:
        r0 = done % max(nr - 31, 1)
        _ = O.gemm_tn_rows(cx, sx, cw, sw, np.arange(r0, min(r0 + 32, nr)))
        flops += 2.0 * min(32, nr - r0) * F * H
        done += 32
        if time.perf_counter() - t1 > target_s / 2:
            break
    tg = time.perf_counter() - t1
    g_rate = flops / tg
    elems_step = 2 * sum(v for k, v in st.quant_elems().items() if k.endswith("_dual"))
    step_flop = 3 * st.gemm_flops()
    step_s = elems_step / q_rate + step_flop / g_rate
    threads, model, blas = host_cpu_info()
    return {
        "value": step_flop / step_s / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"oracle quantizer on {n_el} elements (64-row samples of X and dY row-wise, "
                   f"{tk} token rows x 64 columns of X and dY column-wise; RTNE and SR: "
                   f"{q_rate / 1e6:.2f} M elem/s) and FP64 FPROP of the first "
                   f"{'expert' if L.experts > 1 else 'layer'} on {done} output rows "
                   f"({g_rate / 1e9:.1f} GFLOP/s), scaled to one step of {elems_step:.3g} "
                   f"quantized elements and {step_flop:.3g} FLOP ({step_s:.1f} s); host {model}, "
                   f"cpu_count={os.cpu_count()}, thread pools: {blas or 'none'}"),
    }


class MoeStep(Step):
    """One pass of the hot path over an expert layer: X, W, dY quantized as in
    the dense step, W^T per expert by the stacked column-wise quantization,
    dY^T and X^T column-wise with per-expert padding, then the three grouped
    GEMMs."""

    def __init__(self, L, U, torch, dual=False):
        self.offd = torch.as_tensor(L.offsets, device=L.x.device)
        self.E = L.experts
        self.tokens = int(L.offsets[-1])
        super().__init__(L, U, torch, dual)

    def quant(self, name, x, axis, mask, rnd, sid, ev, **kw):
        U = self.U
        self._start(ev, name)
        q = U.ufp4_rht_quantize(x, axis, True, mask, U.GRID_UNIFORM, rnd, self.seed, sid,
                                out=self.q.get(name), **kw)
        if ev is not None:
            ev[name][1].record()
        self.q[name] = q
        return q

    def gemm(self, name, kind, a, b, out, ev):
        self._start(ev, name)
        self.U.ufp4_grouped_gemm(kind, self.offd, a, b, out=out)
        if ev is not None:
            ev[name][1].record()

    def run(self, ev):
        U, L = self.U, self.L
        C, R, S = U.BLOCKS_ALONG_COLS, U.BLOCKS_ALONG_ROWS, U.BLOCKS_ALONG_ROWS_STACKED
        if not hasattr(self, "dwg"):
            T, H, F, E = self.tokens, self.H, self.F, self.E
            dev = L.x.device
            self.y = self.torch.empty((T, F), dtype=self.torch.float32, device=dev)
            self.dx = self.torch.empty((T, H), dtype=self.torch.float32, device=dev)
            self.dwg = self.torch.empty((E, F, H), dtype=self.torch.float32, device=dev)
        if self.dual:
            xq, xtq = self.quant2("q_x_dual", L.x, (True, self.mf, 0), (True, self.mw, 0),
                                  U.ROUND_RTNE, ev, group_offsets=self.offd)
            wq, wtq = self.quant2("q_w_dual", L.w, (True, self.mf, 0), (True, self.md, 0),
                                  U.ROUND_RTNE, ev, col_axis=S, n_groups=self.E)
            self.gemm("fprop", U.FPROP, xq, wq, self.y, ev)
            dyq, dytq = self.quant2("q_dy_dual", L.dy, (True, self.md, 0), (True, self.mw, 1),
                                    U.ROUND_SR, ev, group_offsets=self.offd)
            self.gemm("dgrad", U.DGRAD, dyq, wtq, self.dx, ev)
            self.gemm("wgrad", U.WGRAD, dytq, xtq, self.dwg, ev)
            return
        xq = self.quant("q_x_fprop", L.x, C, self.mf, U.ROUND_RTNE, 0, ev)
        wq = self.quant("q_w_fprop", L.w, C, self.mf, U.ROUND_RTNE, 0, ev)
        self.gemm("fprop", U.FPROP, xq, wq, self.y, ev)
        dyq = self.quant("q_dy_dgrad", L.dy, C, self.md, U.ROUND_SR, 0, ev)
        wtq = self.quant("q_wt_dgrad", L.w, S, self.md, U.ROUND_RTNE, 0, ev, n_groups=self.E)
        self.gemm("dgrad", U.DGRAD, dyq, wtq, self.dx, ev)
        dytq = self.quant("q_dyt_wgrad", L.dy, R, self.mw, U.ROUND_SR, 1, ev,
                          group_offsets=self.offd)
        xtq = self.quant("q_xt_wgrad", L.x, R, self.mw, U.ROUND_RTNE, 0, ev,
                         group_offsets=self.offd)
        self.gemm("wgrad", U.WGRAD, dytq, xtq, self.dwg, ev)

    def outputs(self):
        return [self.y, self.dx, self.dwg]

    def quant_elems(self):
        T, H, F, E = self.tokens, self.H, self.F, self.E
        return {"q_x_fprop": T * H, "q_w_fprop": E * F * H, "q_dy_dgrad": T * F,
                "q_wt_dgrad": E * F * H, "q_dyt_wgrad": T * F, "q_xt_wgrad": T * H,
                "q_x_dual": T * H, "q_w_dual": E * F * H, "q_dy_dual": T * F}

    def gemm_flops(self):
        return 2.0 * self.tokens * self.H * self.F


def diag_summary(st: dict) -> dict:
    """Reported metrics from the diagnostics kernel's sums and counts (the
    formulas of ufp4_stats in include/ufp4.h)."""
    out = {"sqnr_db": (10.0 * math.log10(st["sum_x2"] / st["sum_err2"])
                       if st["sum_err2"] > 0 else None),
           "one_minus_alpha": 1.0 - st["sum_x_xhat"] / st["sum_x2"],
           "delta_mag": (st["sum_abs_xhat"] - st["sum_abs_x"]) / st["sum_abs_x"]}
    if st["n_nonzero"]:
        out["underflow_ratio"] = st["n_underflow"] / st["n_nonzero"]
        h = list(st["hist"])
        h[0] += h[8]
        h[8] = 0
        tot = float(sum(h))
        ent = -sum((c / tot) * math.log(c / tot) for c in h if c)
        out["bucket_utilization"] = math.exp(ent) / 15.0
    return out


def quant_sweep(args):
    """The quantizer sweep: 16384 x 16384 bf16 (Gaussian, Laplace, Student-t3)
    x {row-wise, column-wise} x {uniform, E2M1} x {RTNE, SR} x {none, RHT}.
    Each case is timed with HIP events over `steps` calls after `warmup`; the
    tensor (512 MiB) does not fit the 256 MiB MALL, so every call streams from
    HBM.  Each case also reports the pages' quantization diagnostics from the
    library's diagnostics kernel (SQNR, 1 - alpha, delta_mag, underflow ratio,
    bucket utilization) and, for the RHT case, the SQNR change RHT brings.
    Per tensor, the dual-axis quantizer (uniform grid, RHT on both outputs,
    RTNE and SR) is timed too, over its 3.5 algorithmic bytes per element."""
    import torch
    from uniform_grid_fp4_amd import ufp4 as U
    from uniform_grid_fp4_amd import workloads as W
    dev = torch.device("cuda:0")
    n = W.SWEEP_SHAPE[0] * W.SWEEP_SHAPE[1]
    ws = torch.empty(U.ufp4_stats_workspace_size() // 8, dtype=torch.int64, device=dev)
    for dist in W.SWEEP_DISTS:
        x = W.sweep_tensor(dist, dev)
        for axis in (U.BLOCKS_ALONG_COLS, U.BLOCKS_ALONG_ROWS):
            for grid in (U.GRID_UNIFORM, U.GRID_E2M1):
                for rnd in (U.ROUND_RTNE, U.ROUND_SR):
                    sqnr_plain = None
                    for rht in (False, True):
                        q = U.ufp4_rht_quantize(x, axis, rht, 0xBEEF, grid, rnd, 7, 0)
                        for _ in range(args.warmup):
                            U.ufp4_rht_quantize(x, axis, rht, 0xBEEF, grid, rnd, 7, 0, out=q)
                        e0 = torch.cuda.Event(enable_timing=True)
                        e1 = torch.cuda.Event(enable_timing=True)
                        e0.record()
                        for _ in range(args.steps):
                            U.ufp4_rht_quantize(x, axis, rht, 0xBEEF, grid, rnd, 7, 0, out=q)
                        e1.record()
                        torch.cuda.synchronize()
                        ms = e0.elapsed_time(e1) / args.steps
                        diag = diag_summary(U.ufp4_quant_stats(x, q, axis, workspace=ws))
                        if rht and sqnr_plain is not None and diag["sqnr_db"] is not None:
                            diag["delta_sqnr_db"] = diag["sqnr_db"] - sqnr_plain
                        else:
                            sqnr_plain = diag["sqnr_db"]
                        gbs = n * BYTES_PER_QUANT_ELEM / (ms * 1e-3) / 1e9
                        print(json.dumps({
                            "workload": "quant-sweep", "dist": dist,
                            "layout": ("colwise-transposed" if axis == U.BLOCKS_ALONG_ROWS
                                       else "rowwise"),
                            "rht": rht, "grid": "uniform" if grid == 0 else "e2m1",
                            "rounding": "sr" if rnd else "rtne", "us": round(ms * 1e3, 2),
                            "gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                            **diag}), flush=True)
                        del q
        # the dual-axis quantizer (both operands of the tensor from one read),
        # uniform grid with RHT on both outputs, as the UFP4 recipe uses it
        for rnd in (U.ROUND_RTNE, U.ROUND_SR):
            sides = ((True, 0xBEEF, 0), (True, 0x1DEA, 1))
            qr, qc = U.ufp4_rht_quantize_dual(x, *sides, grid=U.GRID_UNIFORM, rnd=rnd, seed=7)
            for _ in range(args.warmup):
                U.ufp4_rht_quantize_dual(x, *sides, grid=U.GRID_UNIFORM, rnd=rnd, seed=7,
                                         out_rows=qr, out_cols=qc)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                U.ufp4_rht_quantize_dual(x, *sides, grid=U.GRID_UNIFORM, rnd=rnd, seed=7,
                                         out_rows=qr, out_cols=qc)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            gbs = n * BYTES_PER_DUAL_ELEM / (ms * 1e-3) / 1e9
            print(json.dumps({"workload": "quant-sweep", "dist": dist, "layout": "dual-axis",
                              "rht": True, "grid": "uniform", "rounding": "sr" if rnd else "rtne",
                              "us": round(ms * 1e3, 2), "gbs": round(gbs, 1),
                              "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}), flush=True)
            del qr, qc
        del x
        torch.cuda.empty_cache()


# Recipes of the single-GEMM output comparison: grid, and which GEMMs'
# operands get the RHT (paperlayer summary section 4 and section 5 Q4: UFP4
# applies it to all three; the E2M1 reference recipe to WGRAD only; the
# range-restricted E2M1 variant keeps {0, .5, 1, 1.5, 2} with full RHT).
Q1_RECIPES = (
    ("uniform, no RHT", 0, (False, False, False)),
    ("UFP4: uniform, RHT on all GEMMs", 0, (True, True, True)),
    ("E2M1, no RHT", 1, (False, False, False)),
    ("E2M1, RHT on WGRAD only (reference recipe)", 1, (False, False, True)),
    ("E2M1, RHT on all GEMMs", 1, (True, True, True)),
    ("E2M1 max 2.0, RHT on all GEMMs", 2, (True, True, True)),
)


def q1_outputs(args):
    """The pages' single-GEMM output test on the dense 1.5B layer: the three
    GEMM outputs of each recipe (grid and RHT placement; stochastic rounding
    on dY) against the unquantized product of the bf16 operands (FP32 torch
    matmul, the reference only), as SQNR and 1 - alpha -- measured with the
    library's diagnostics kernel.  One JSON line per (recipe, GEMM)."""
    import torch
    from uniform_grid_fp4_amd import ufp4 as U
    from uniform_grid_fp4_amd import workloads as W
    dev = torch.device("cuda:0")
    L = W.dense_1p5b(dev)
    mf, md, mw = L.masks
    x, w, dy = L.x.float(), L.w.float(), L.dy.float()
    refs = {"fprop": torch.matmul(x, w.t().contiguous()),
            "dgrad": torch.matmul(dy, w),
            "wgrad": torch.matmul(dy.t().contiguous(), x)}
    del x, w, dy
    ws = torch.empty(U.ufp4_stats_workspace_size() // 8, dtype=torch.int64, device=dev)
    C, R = U.BLOCKS_ALONG_COLS, U.BLOCKS_ALONG_ROWS
    for name, grid, (hf, hd, hw) in Q1_RECIPES:
        qx = U.ufp4_rht_quantize(L.x, C, hf, mf, grid)
        qw = U.ufp4_rht_quantize(L.w, C, hf, mf, grid)
        qdy = U.ufp4_rht_quantize(L.dy, C, hd, md, grid, U.ROUND_SR, 1234, 0)
        qwt = U.ufp4_rht_quantize(L.w, R, hd, md, grid)
        qdyt = U.ufp4_rht_quantize(L.dy, R, hw, mw, grid, U.ROUND_SR, 1234, 1)
        qxt = U.ufp4_rht_quantize(L.x, R, hw, mw, grid)
        outs = {"fprop": U.ufp4_gemm_fprop(qx, qw), "dgrad": U.ufp4_gemm_dgrad(qdy, qwt),
                "wgrad": U.ufp4_gemm_wgrad(qdyt, qxt)}
        for gemm, y in outs.items():
            d = diag_summary(U.ufp4_output_stats(refs[gemm], y, workspace=ws))
            print(json.dumps({"workload": "q1-outputs", "layer": L.name, "recipe": name,
                              "gemm": gemm, "sqnr_db": d["sqnr_db"],
                              "one_minus_alpha": d["one_minus_alpha"]}), flush=True)
        del outs, qx, qw, qdy, qwt, qdyt, qxt
        torch.cuda.empty_cache()


MFMA_KINDS = ("v_mfma_f32_32x32x16_fp8_fp8", "v_mfma_i32_32x32x16_i8",
              "v_mfma_scale_f32_32x32x64_f8f6f4 (fp8)", "v_mfma_scale_f32_32x32x64_f8f6f4 (fp6)",
              "v_mfma_scale_f32_32x32x64_f8f6f4 (fp4)", "v_mfma_f32_32x32x16_bf16",
              "v_mfma_f32_32x32x1_2b_f32", "v_mfma_f32_32x32x8_bf16")
# The block-product candidates (kinds 0-5): a K = 16 instruction yields one
# useful 16-element block product per output, and so does a K = 64 one
# (zero-padded, or four blocks placed block-diagonally along M), since the
# per-16 FP32 scales must be applied to each block's partial sum.  Kinds 6
# and 7 are candidates for the scale products: the FP32 outer product the
# GEMM uses, and the K = 8 bf16 form a three-way bf16 split of the scales
# would use.
MFMA_BLOCK_PRODUCT_KINDS = 6
MIX_MODES = ("2 FP8 MFMA + 1 FP32 outer-product MFMA + 32 FMA", "32 FMA only",
             "2 FP8 MFMA + 1 FP32 outer-product MFMA only")
OVERLAP_KINDS = ("2 x v_mfma_f32_32x32x16_fp8_fp8", "1 x v_mfma_f32_32x32x1_2b_f32",
                 "2 x v_mfma_f32_32x32x8_bf16")


def probe_lib():
    import ctypes
    path = os.path.join(ROOT, "uniform_grid_fp4_amd", "libufp4_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with python -m uniform_grid_fp4_amd.build")
    L = ctypes.CDLL(path)
    L.ufp4_probe_mfma_tflops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.ufp4_probe_mfma_tflops.restype = ctypes.c_double
    L.ufp4_probe_mfma_flops.argtypes = [ctypes.c_int]
    L.ufp4_probe_mfma_flops.restype = ctypes.c_double
    L.ufp4_probe_mix_ms.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.ufp4_probe_mix_ms.restype = ctypes.c_double
    L.ufp4_probe_overlap_ms.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.ufp4_probe_overlap_ms.restype = ctypes.c_double
    return L


def mfma_peak_tflops(kind: int) -> float:
    """Sustained rate of one MFMA kind on this GPU (4096 workgroups x 4 waves
    x 4 independent chains)."""
    v = probe_lib().ufp4_probe_mfma_tflops(kind, 4096, 2000)
    if v <= 0:
        raise RuntimeError(f"MFMA probe failed ({v})")
    return v


def instruction_mix_tflops() -> float:
    """Rate of the GEMM's per-block instruction mix run on its own (two FP8
    MFMAs, one FP32 outer-product MFMA and 32 FMAs per wave-iteration = two
    32x32x16 units, 4 waves per SIMD, no memory traffic): the ceiling this
    instruction mix reaches on this GPU, given how little matrix-core and
    vector work overlap on one SIMD."""
    wgs, reps = 4096, 2000
    ms = probe_lib().ufp4_probe_mix_ms(0, wgs, reps)
    if ms <= 0:
        raise RuntimeError(f"mix probe failed ({ms})")
    return wgs * 4 * reps * 2 * (2.0 * 32 * 32 * 16) / (ms * 1e-3) / 1e12


def mfma_peaks(args):
    """The candidate MFMA instructions for the block-scaled GEMM, measured:
    the rate, and the rate of useful 16-element block products (the GEMM
    needs each block's partial sum on its own to apply the FP32 scales)."""
    import torch
    assert torch.cuda.is_available()
    L = probe_lib()
    for kind, name in enumerate(MFMA_KINDS):
        tf = mfma_peak_tflops(kind)
        flops = L.ufp4_probe_mfma_flops(kind)
        line = {"workload": "mfma-peak", "instruction": name, "tflops": round(tf, 1),
                "cycles_per_instruction_2p4ghz": round(flops / (tf * 1e12 / SIMDS / 2.4e9), 1)}
        if kind < MFMA_BLOCK_PRODUCT_KINDS:
            k = 16 if flops == 2.0 * 32 * 32 * 16 else 64
            line.update(k=k, block_products_tflops_equiv=round(tf * 16 / k, 1))
        print(json.dumps(line), flush=True)
    # Co-execution: the GEMM's per-block mix of one wave against its parts,
    # in SIMD cycles per wave-iteration at the nominal 2.4 GHz (4096
    # workgroups x 4 waves = 4 waves per SIMD).  If matrix-core and vector
    # work overlapped, the mix would take the larger of its parts; if they
    # serialised, their sum.
    wgs, reps = 4096, 2000
    cyc = []
    for mode, name in enumerate(MIX_MODES):
        ms = L.ufp4_probe_mix_ms(mode, wgs, reps)
        if ms <= 0:
            raise RuntimeError(f"mix probe failed ({ms})")
        cyc.append(ms * 1e-3 * SIMDS * 2.4e9 / (wgs * 4 * reps))
        print(json.dumps({"workload": "mfma-vs-valu", "loop": name,
                          "simd_cycles_per_wave_iteration": round(cyc[-1], 1)}), flush=True)
    print(json.dumps({"workload": "mfma-vs-valu", "mix_over_max_of_parts": round(cyc[0] / max(cyc[1:]), 3),
                      "mix_over_sum_of_parts": round(cyc[0] / (cyc[1] + cyc[2]), 3)}), flush=True)
    # Cross-wave overlap: on every SIMD half of the waves issue one kind of
    # matrix-core work (about 64 matrix-core cycles per iteration), the other
    # half 32 FMAs per iteration; timed with each half alone and both
    # together.  overlap = (alone + alone - together) / the shorter alone:
    # 1 when the vector work hides entirely under the matrix-core work (or the
    # reverse), 0 when the two serialise.
    wgs, reps = 1024, 4000
    for kind, name in enumerate(OVERLAP_KINDS):
        t = []
        for roles in (1, 2, 3):
            ms = L.ufp4_probe_overlap_ms(kind, roles, wgs, reps)
            if ms <= 0:
                raise RuntimeError(f"overlap probe failed ({ms})")
            t.append(ms)
        print(json.dumps({"workload": "mfma-vs-valu-waves", "mfma": name,
                          "mfma_waves_ms": round(t[0], 3), "fma_waves_ms": round(t[1], 3),
                          "together_ms": round(t[2], 3),
                          "overlap": round((t[0] + t[1] - t[2]) / min(t[0], t[1]), 3)}),
              flush=True)


def quant_kernels(args):
    """The UFP4 quantizer kernels on the 16384 x 16384 Gaussian sweep tensor
    (uniform grid, RHT): row-wise and column-wise single-axis calls with RTNE
    and SR, and the dual-axis call with RTNE and SR.  Each is timed with HIP
    events over `steps` back-to-back calls after `warmup` (the 512 MiB input
    streams from HBM every call); one JSON line per kernel, over the
    algorithmic bytes (2.75 B per element per output, 2 B read once)."""
    import torch
    from uniform_grid_fp4_amd import ufp4 as U
    from uniform_grid_fp4_amd import workloads as W
    dev = torch.device("cuda:0")
    x = W.sweep_tensor("gaussian", dev)
    n = x.numel()
    cases = [("rowwise", "rtne"), ("colwise-transposed", "rtne"), ("rowwise", "sr"),
             ("colwise-transposed", "sr"), ("dual-axis", "rtne"), ("dual-axis", "sr")]
    for layout, r in cases:
        rnd = U.ROUND_SR if r == "sr" else U.ROUND_RTNE
        if layout == "dual-axis":
            sides = ((True, 0xBEEF, 0), (True, 0x1DEA, 1))
            qr, qc = U.ufp4_rht_quantize_dual(x, *sides, rnd=rnd, seed=7)
            call = lambda: U.ufp4_rht_quantize_dual(x, *sides, rnd=rnd, seed=7, out_rows=qr,
                                                    out_cols=qc)
            nbytes = n * BYTES_PER_DUAL_ELEM
        else:
            axis = U.BLOCKS_ALONG_COLS if layout == "rowwise" else U.BLOCKS_ALONG_ROWS
            q = U.ufp4_rht_quantize(x, axis, True, 0xBEEF, U.GRID_UNIFORM, rnd, 7, 0)
            call = lambda: U.ufp4_rht_quantize(x, axis, True, 0xBEEF, U.GRID_UNIFORM, rnd, 7, 0,
                                               out=q)
            nbytes = n * BYTES_PER_QUANT_ELEM
        for _ in range(args.warmup):
            call()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / args.steps * 1e3
        gbs = nbytes / (us * 1e-6) / 1e9
        print(json.dumps({"workload": "quant-2p28", "layout": layout, "rounding": r,
                          "grid": "uniform", "rht": True, "us": round(us, 2),
                          "gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}),
              flush=True)


def copy_ceiling(args):
    """A plain contiguous 1 GiB device-to-device copy (torch's copy kernel):
    the streaming ceiling the quantizer is compared with, and the run whose
    FETCH_SIZE / WRITE_SIZE counters calibrate the traffic figures (it reads
    and writes exactly 1 GiB per launch)."""
    import torch
    n = 1 << 29
    a = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(args.warmup):
        b.copy_(a)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = 2 * a.numel() * a.element_size()
    print(json.dumps({"workload": "copy", "bytes_read": nbytes // 2, "bytes_written": nbytes // 2,
                      "us": round(ms * 1e3, 2), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                      "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}),
          flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the UFP4 hot path is "
              "data parallel and what is measured is one GPU's share of it.", file=sys.stderr)
        sys.exit(2)
    if args.workload == "quant-sweep":
        return quant_sweep(args)
    if args.workload == "quant-2p28":
        return quant_kernels(args)
    if args.workload == "copy":
        return copy_ceiling(args)
    if args.workload == "q1-outputs":
        return q1_outputs(args)
    if args.workload == "mfma-peak":
        return mfma_peaks(args)
    import torch
    from uniform_grid_fp4_amd import ufp4 as U
    from uniform_grid_fp4_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.workload == "moe-7.9b":
        L = W.moe_7p9b(dev)
        st = MoeStep(L, U, torch, args.quantizer == "dual")
    elif args.workload == "moe-124b":
        L = W.moe_124b(dev)
        st = MoeStep(L, U, torch, args.quantizer == "dual")
    else:
        L = W.dense_1p5b(dev)
        st = Step(L, U, torch, args.quantizer == "dual")
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        st.run(None)
    torch.cuda.synchronize()

    # Step time: the step captured once as a HIP graph (stream capture of the
    # same library calls on the same buffers) and replayed back to back, no
    # per-launch host work or gaps.  Each of three checking replays first has
    # its outputs overwritten with NaN and must reproduce the eager step bit
    # for bit.
    ms_step_eager = None
    graph_checked = None
    if not args.eager:
        outs = st.outputs()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st.run(None)
        for _ in range(3):
            st.run(None)
            torch.cuda.synchronize()
            ref = [t.clone() for t in outs]
            for t in outs:
                t.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert all(torch.equal(a, b) for a, b in zip(outs, ref)), \
                "graph replay differs from the eager step"
            del ref
        graph_checked = 3
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # Eager steps, back to back (also the step time with --eager).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        st.run(None)
    torch.cuda.synchronize()
    ms_step_eager = (time.perf_counter() - t0) * 1e3 / args.steps
    if args.eager:
        ms_step = ms_step_eager

    # Per-kernel durations: an eager pass of back-to-back steps with HIP
    # events around every launch; medians over the steps.
    names = st.quant_names + Step.GEMMS
    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for n in names} for _ in range(args.steps)]
    for k in range(args.steps):
        st.run(evs[k])
    torch.cuda.synchronize()
    cache = "cold" if st.inputs_cold() else "warm"

    def median(v):
        v = sorted(v)
        n = len(v)
        return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])

    dur = {n: median([e[n][0].elapsed_time(e[n][1]) for e in evs]) for n in names}
    q_ms = sum(dur[n] for n in st.quant_names)
    qb = st.quant_bytes()
    q_bytes = sum(qb.values())
    q_gbs = q_bytes / (q_ms * 1e-3) / 1e9
    g_ms = sum(dur[n] for n in Step.GEMMS)
    g_flop = 3 * st.gemm_flops()
    gemm_avg_ms = g_ms / 3
    gemm_tflops = st.gemm_flops() / (gemm_avg_ms * 1e-3) / 1e12
    used_peak = mfma_peak_tflops(0)   # measured after the timed region
    mix_peak = instruction_mix_tflops()
    step_tflops = g_flop / (ms_step * 1e-3) / 1e12
    gemm_traffic = measured_traffic(L.name, "gemm")
    quant_traffic = measured_traffic(L.name, "quantize")

    out = {
        "metric": "RHT+UFP4 quantize GB/s (% HBM peak); UFP4 GEMM TFLOP/s (% MFMA peak)",
        "value": round(step_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "timing": (("HIP graph replays of the captured step (%d checking replays bit-identical "
                    "to the eager step)" % graph_checked) if graph_checked
                   else "eager launches") +
                  "; per-kernel durations: medians of HIP events on the launch stream over an "
                  "eager pass of back-to-back steps (%s: the quantized inputs %s the 256 MB "
                  "MALL)" % (cache, "are all >= 2x" if cache == "cold" else "can sit in"),
        "ms_per_step_eager": round(ms_step_eager, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 MFMA operands (exact 4-bit levels), fp32 accumulate/scales",
        "data": "synthetic",
        "config": {"workload": L.name, "tokens": int(L.offsets[-1]), "hidden": st.H,
                   "ffn": st.F, "experts": L.experts,
                   "recipe": "UFP4: uniform grid, RHT-16 on all 3 GEMMs, SR on dY",
                   "block": 16, "scale": "fp32 absmax"},
        "quantize": {"gbs": round(q_gbs, 1),
                     "frac_hbm": round(q_gbs / HBM_PEAK_GBS, 4),
                     "ms_per_step": round(q_ms, 4),
                     "per_call_ms": {n: round(dur[n], 4) for n in st.quant_names},
                     "per_call_gbs": {n: round(qb[n] / (dur[n] * 1e-3) / 1e9, 1)
                                      for n in st.quant_names},
                     "kernels": "dual-axis" if st.dual else "single-axis",
                     "bytes_per_step": q_bytes,
                     "cache": cache},
        "gemm": {"tflops": round(gemm_tflops, 2),
                 "frac_fp8_mfma_peak": round(gemm_tflops / FP8_MFMA_PEAK_TFLOPS, 4),
                 "used_instruction": MFMA_KINDS[0],
                 "used_instruction_peak_tflops": round(used_peak, 1),
                 "frac_used_instruction_peak": round(gemm_tflops / used_peak, 4),
                 "mix_ceiling_tflops": round(GEMM_PIPE_PEAK_TFLOPS, 1),
                 "frac_mix_ceiling": round(gemm_tflops / GEMM_PIPE_PEAK_TFLOPS, 4),
                 "instruction_mix_tflops": round(mix_peak, 1),
                 "frac_instruction_mix": round(gemm_tflops / mix_peak, 4),
                 "ms_per_step": round(g_ms, 4),
                 "per_call_ms": {n: round(dur[n], 4) for n in Step.GEMMS}},
        "roofline": {"kernel": ("ufp4::gemm_kernel<0, 1|2>" if isinstance(st, MoeStep)
                                else "ufp4::gemm_kernel<0, 0>"),
                     "bound": "mfma",
                     "achieved": round(gemm_tflops, 2), "peak": FP8_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / FP8_MFMA_PEAK_TFLOPS, 4),
                     "traffic": gemm_traffic},
        "roofline_quantize": {"kernel": ("ufp4::quant_dual_kernel" if st.dual
                                         else "ufp4::quant_{rows_contig,cols}_kernel"),
                              "bound": "hbm", "achieved": round(q_gbs, 1),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(q_gbs / HBM_PEAK_GBS, 4),
                              "cache": cache, "traffic": quant_traffic},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(L, st, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
