"""Build libhc.so (the HIP library) in-tree for gfx950.

    python -m transformer_hyper_connection_amd.build

Runs hipcc on csrc/hc.hip with the repository's include/ directory and writes
transformer_hyper_connection_amd/libhc.so.  No GPU is needed to build.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "hc.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhc.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-shared",
    # the stream arithmetic is a fixed sequence of separately rounded fp32 ops
    "-ffp-contract=off",
    # no packed-fp32 instructions are generated
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wextra",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libhc)")


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile libhc.so; returns its path.  Always recompiles."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-I", INCLUDE, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-6000:]}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
