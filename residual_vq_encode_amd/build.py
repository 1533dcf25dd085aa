"""Builds libkvq.so in place with hipcc for gfx950 (MI355X).

    python -m residual_vq_encode_amd.build

Sources: csrc/kernels.hip (device code), csrc/api.cpp (C ABI, launches), csrc/codebooks.cpp
(host codebook builder). All HIP code is compiled with packed-FP32 instruction selection
off (``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass warns that
it does not know that feature, which is harmless.
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
LIB = os.path.join(HERE, "libkvq.so")
ARCH = "gfx950"

SOURCES = ["kernels.hip", "api.cpp", "codebooks.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkvq)")


def command(out: str = LIB) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I", INCLUDE, "-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False) -> str:
    """Compile libkvq.so next to this file (atomically replaced). Returns its path."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
