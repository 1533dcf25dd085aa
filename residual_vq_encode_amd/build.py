"""Builds libkvq.so in place with hipcc for gfx950 (MI355X).

    python -m residual_vq_encode_amd.build

Sources: csrc/kernels.hip and csrc/kernels_ragged.hip (codec kernels of csrc/codec.h, for
head dimensions whose rows are and are not 16-byte aligned), csrc/attend.hip (attention over the packed
cache), csrc/qjl.hip (1-bit sign-sketch encoder), csrc/api.cpp (C ABI, launches),
csrc/codebooks.cpp (host codebook builder). Each
is compiled to an object file in parallel (in a private temporary directory), then the
objects are linked into the shared library, which replaces the previous one atomically.
All HIP code is compiled with packed-FP32 instruction selection off
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass warns that it
does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkvq.so")
ARCH = "gfx950"

SOURCES = ["kernels.hip", "kernels_ragged.hip", "attend.hip", "qjl.hip", "api.cpp", "codebooks.cpp"]
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument"]
NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkvq)")


def compile_command(src: str, obj: str) -> list[str]:
    return [hipcc()] + FLAGS + ["-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj]


def link_command(objs: list[str], out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out] + objs


def _run(cmd: list[str], verbose: bool) -> str:
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in proc.stderr.splitlines() if NOISE not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile libkvq.so next to this file (atomically replaced). Returns its path."""
    with tempfile.TemporaryDirectory(prefix="kvq_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as pool:
            errs = list(pool.map(lambda so: _run(compile_command(*so), verbose), zip(SOURCES, objs)))
        tmp = LIB + ".tmp"
        errs.append(_run(link_command(objs, tmp), verbose))
        warnings = "\n".join(e for e in errs if e.strip())
        if warnings and verbose:
            print(warnings, file=sys.stderr)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
