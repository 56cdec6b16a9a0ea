"""Pins for the oracle's Philox4x32-10 generator and its stochastic rounding.

Philox4x32-10 is the counter-based generator of Salmon et al., "Parallel
Random Numbers: As Easy as 1, 2, 3" (SC'11).  The oracle's implementation is
checked against an independent one: PyTorch's installed C++ header
ATen/core/PhiloxRNGEngine.h, compiled here into a small host program.

Stochastic rounding (paperlayer.ai summary of arXiv 2606.20381, section 2
"Rounding rules") samples the two adjacent levels and is unbiased in
expectation; the test bound is statistical.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

from oracle import ufp4_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))

HARNESS = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  // stdin: lines "seed subsequence offset"; stdout: the 4 words
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    at::philox_engine e(seed, sub, off);
    unsigned a = e(), b = e(), c = e(), d = e();
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def torch_philox():
    gxx = shutil.which("g++")
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    if gxx is None or not os.path.exists(os.path.join(inc, "ATen/core/PhiloxRNGEngine.h")):
        pytest.skip("g++ or torch's Philox header is not available")
    d = tempfile.mkdtemp()
    src = os.path.join(d, "h.cpp")
    exe = os.path.join(d, "h")
    open(src, "w").write(HARNESS)
    subprocess.check_call([gxx, "-O1", "-std=c++17", "-I", inc, src, "-o", exe])

    def run(triples):
        inp = "".join(f"{s} {b} {o}\n" for s, b, o in triples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return np.array([[int(v) for v in ln.split()] for ln in out.strip().splitlines()],
                        dtype=np.uint64)
    yield run
    shutil.rmtree(d)


def test_philox_matches_pytorch_header(torch_philox):
    rng = np.random.default_rng(0)
    triples = [(0, 0, 0), (1, 0, 0), (0, 1, 0), (0, 0, 1),
               ((1 << 64) - 1, (1 << 32) - 1, (1 << 64) - 1)]
    for _ in range(300):
        triples.append((int(rng.integers(0, 1 << 63)) * 2 + int(rng.integers(0, 2)),
                        int(rng.integers(0, 1 << 32)),
                        int(rng.integers(0, 1 << 62))))
    ref = torch_philox(triples)
    for (seed, sub, off), want in zip(triples, ref):
        got = O.philox4x32_10(off & 0xFFFFFFFF, off >> 32, sub & 0xFFFFFFFF, sub >> 32,
                              seed & 0xFFFFFFFF, seed >> 32)
        assert [int(w) for w in got] == [int(w) for w in want], (seed, sub, off)


def test_sr_word_selection_matches_pytorch_engine_stream(torch_philox):
    """Element idx takes word idx & 3 of block idx >> 2 in subsequence stream_id."""
    seed, stream = 0x123456789ABCDEF, 7
    idx = np.array([0, 1, 2, 3, 4, 5, 1 << 33, (1 << 33) + 3, 12345678901], dtype=np.uint64)
    ref = torch_philox([(seed, stream, int(i) >> 2) for i in idx])
    got = O.sr_random_u32(idx, seed, stream)
    for i, g, r in zip(idx, got, ref):
        assert int(g) == int(r[int(i) & 3])


@pytest.mark.parametrize("grid,ts", [(O.GRID_UNIFORM, [0.3, 2.5, 6.9]),
                                     (O.GRID_E2M1, [0.3, 1.2, 2.4, 5.0]),
                                     (O.GRID_E2M1_MAX2, [0.3, 1.2, 1.9])])
def test_sr_is_unbiased(grid, ts):
    N = 10_000_000
    L = O.LEVELS[grid]
    for j, t in enumerate(ts):
        t32 = float(np.float32(t))
        m = np.full(N, np.float32(t))
        idx = np.arange(N, dtype=np.uint64) + np.uint64(N * j)
        u = O.sr_random_u32(idx, seed=2024 + grid, stream_id=3)
        k = O.sr_index(m, grid, u)
        lo = L[L <= t32].max()
        hi = L[L > t32].min()
        assert set(np.unique(k)) <= {int(np.where(L == lo)[0][0]), int(np.where(L == hi)[0][0])}
        f = (t32 - lo) / (hi - lo)
        sigma = np.sqrt(f * (1 - f) / N) * (hi - lo)
        mean = L[k].mean()
        assert abs(mean - t32) <= 6 * sigma + 2.0 ** -32 * (hi - lo), (t, mean)


def test_sr_on_a_level_never_moves():
    for grid in (O.GRID_UNIFORM, O.GRID_E2M1, O.GRID_E2M1_MAX2):
        L = O.LEVELS[grid].astype(np.float32)
        m = np.repeat(L, 1000)
        u = O.sr_random_u32(np.arange(m.size, dtype=np.uint64), 5, 0)
        assert (O.LEVELS[grid][O.sr_index(m, grid, u)] == m).all()


def test_sr_quantizer_is_unbiased_per_element():
    """Averaged over many seeds, the SR-dequantized tensor equals the RHT of
    the input (the normalized value times s/g) up to the statistical bound."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 32)).astype(np.float32)
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    xf = O.bf16_bits_to_f32(b)
    y = O.rht16(xf.reshape(4, 2, 16), 0x0F0F).reshape(4, 32).astype(np.float64)
    acc = np.zeros_like(y)
    S = 4000
    for seed in range(S):
        c, s, _ = O.quantize(b, O.AXIS_COLS, True, 0x0F0F, O.GRID_UNIFORM, O.ROUND_SR, seed, 1)
        acc += O.dequantize64(c, s, O.GRID_UNIFORM)
    step = np.repeat(s, 16, axis=1) / 7.0
    assert (np.abs(acc / S - y) <= 6 * 0.5 * step / np.sqrt(S) + 1e-12).all()


def test_sr_streams_and_seeds_are_distinct():
    idx = np.arange(4096, dtype=np.uint64)
    a = O.sr_random_u32(idx, 1, 0)
    b = O.sr_random_u32(idx, 1, 1)
    c = O.sr_random_u32(idx, 2, 0)
    assert (a != b).mean() > 0.99 and (a != c).mean() > 0.99
    assert (O.sr_random_u32(idx, 1, 0) == a).all()
