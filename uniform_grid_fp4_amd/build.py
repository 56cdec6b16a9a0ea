"""Build libufp4.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m uniform_grid_fp4_amd.build   (or call build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libufp4.so")
SOURCES = ["api.hip", "quantize.hip", "gemm.hip", "stats.hip"]
# The bench's MFMA issue-rate probe: a separate library, not part of the ABI.
PROBE_LIB = os.path.join(HERE, "libufp4_probe.so")
PROBE_SOURCES = ["probe.hip"]

# -ffp-contract=off: no multiply-add fusion anywhere (the quantizer's two
#   roundings r = RN(g/s), t = RN(y*r) must stay separate).
# -fno-gpu-flush-denormals-to-zero: FP32 subnormals are kept (bf16 inputs and
#   butterfly outputs can be subnormal).
# -packed-fp32-ops disabled: no v_pk_* FP32 instructions are generated.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libufp4.so")


def _compile(sources, out, verbose):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    noise = [ln for ln in res.stderr.splitlines()
             if "packed-fp32-ops" not in ln and ln.strip()]
    if noise and verbose:
        print("\n".join(noise), file=sys.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source: libufp4.so and the probe library."""
    _compile(SOURCES, LIB, verbose)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
