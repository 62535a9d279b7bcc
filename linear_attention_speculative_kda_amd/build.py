"""Build libkda.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m linear_attention_speculative_kda_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "kda.hip")
HOST_SRC = os.path.join(PKG, "csrc", "check_rows.cpp")   # host-only C++
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkda.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Every FMA is written out; nothing is contracted or reassociated, so the
    # commit and the plain recurrence round identically.
    "-ffp-contract=off",
    # No packed fp32 instructions in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def build(verbose: bool = False) -> str:
    """Compile libkda.so next to this file and return its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, SRC, HOST_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
