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
SOURCES = ["adaln_rope.hip", "gemm.hip", "attention.hip", "io.hip", "unfused.hip", "scratch.hip", "h3dit.cpp"]
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


def _compile_one(hipcc: str, src: str, verbose: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc] + _flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-6000:]}")
    if verbose and r.stderr.strip():
        print(r.stderr)
    return obj


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile_one(hipcc, src, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


SAN_LIB_PATH = os.path.join(BUILD, "san", "libh3dit_san.so")


def build_host_sanitized() -> str:
    """The same library with its host code (the C ABI, argument checks, workspace
    carving: ``h3dit.cpp``) built by g++ under AddressSanitizer and
    UndefinedBehaviorSanitizer; the kernel objects are the ordinary hipcc ones.
    For the CPU ABI tests only (load it with ``$H3DIT_LIB`` and GCC's libasan
    preloaded).  Returns the library's path."""
    gxx = shutil.which("g++")
    if gxx is None:
        raise RuntimeError("g++ not found")
    hipcc = _hipcc()
    os.makedirs(os.path.dirname(SAN_LIB_PATH), exist_ok=True)
    kernels = [s for s in SOURCES if s.endswith(".hip")]
    # the kernel objects of the last build() are reused when no source is newer
    newest = max(os.path.getmtime(os.path.join(d, f))
                 for d in (CSRC, os.path.join(os.path.dirname(PKG), "include")) for f in os.listdir(d))

    def kernel_obj(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        if os.path.exists(obj) and os.path.getmtime(obj) >= newest:
            return obj
        return _compile_one(hipcc, src)

    with cf.ThreadPoolExecutor(max_workers=len(kernels)) as ex:
        objs = list(ex.map(kernel_obj, kernels))
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    obj = os.path.join(os.path.dirname(SAN_LIB_PATH), "h3dit_san.o")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer", "-Wall",
           "-Wno-unused-function", "-fvisibility=hidden", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", CSRC,
           "-I", os.path.join(os.path.dirname(PKG), "include")] + san + \
          ["-c", os.path.join(CSRC, "h3dit.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed on h3dit.cpp:\n{r.stderr[-6000:]}")
    tmp = SAN_LIB_PATH + ".tmp"
    cmd = [gxx, "-shared"] + san + ["-o", tmp, obj] + objs + \
          ["-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, SAN_LIB_PATH)
    return SAN_LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
