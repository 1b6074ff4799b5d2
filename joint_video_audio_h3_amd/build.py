"""Build libh3dit.so (gfx950) in-tree with hipcc.

Every HIP translation unit is compiled for gfx950 only, with packed-FP32
instruction generation disabled, then linked into one shared library next to
this file.  ``build()`` always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(os.path.dirname(PKG), "_build")
LIB_PATH = os.path.join(PKG, "libh3dit.so")
SOURCES = ["adaln_rope.hip", "gemm.hip", "attention.hip", "io.hip", "scratch.hip", "h3dit.cpp"]
ARCH = "gfx950"


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the H3 HIP library)")


def _flags():
    return [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
            "-I", CSRC, "-I", os.path.join(os.path.dirname(PKG), "include")]


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc] + _flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-6000:]}")
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
