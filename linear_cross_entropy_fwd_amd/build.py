"""Builds the gfx950 shared library ``libflce.so`` in-tree with hipcc.

    python -m linear_cross_entropy_fwd_amd.build        # or build() from Python

The library exports the C ABI declared in include/flce.h.  Device code is
compiled for gfx950 only, without floating-point contraction (so the loss
does not depend on which optional metrics a kernel variant also computes)
and without the packed-fp32 target feature.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libflce.so")

SOURCES = ["flce_kernels.hip", "flce_small.hip", "flce_api.cpp"]
HEADERS = ["flce_device.h", "flce_plan.h"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source into ``libflce.so`` (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
