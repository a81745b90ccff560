"""Build librs_hip.so (the layout library) and librs_bench.so (the
benchmark's streaming-copy ceiling and the square-root self-check) for gfx950
with hipcc, in-tree next to this file.

    python -m structure_aware_grouped_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librs_hip.so")
SOURCES = ["planner.cpp", "plan.cpp", "transform.hip", "quant.hip", "gather.hip", "adam.hip"]
BENCH_LIB = os.path.join(HERE, "librs_bench.so")
BENCH_SOURCES = ["stream_copy.hip", "selftest.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",                          # no FMA contraction anywhere
    "-fhip-fp32-correctly-rounded-divide-sqrt",   # IEEE fp32 division for the block scales
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(sources, lib, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", INCLUDE, *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile both libraries; returns the layout library's path. Always recompiles."""
    _compile(BENCH_SOURCES, BENCH_LIB, verbose)
    return _compile(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
