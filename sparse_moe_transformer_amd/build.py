"""Build libmoe_ffn.so (HIP kernels + C ABI) for gfx950 with hipcc.

Usage: ``python -m sparse_moe_transformer_amd.build`` (or ``build()``).
Objects go to ``_build/`` at the repository root; the shared library is
written next to this file so it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_ffn.so")

SOURCES = ["route.hip", "gemm.hip", "fp4mm.hip", "fp4stream.hip", "stream.hip", "combine.hip", "quant.hip", "api.cpp"]
ARCH = "gfx950"

# -packed-fp32-ops: keep hipcc from forming v_pk_{add,mul,fma}_f32 (the host
# pass warns that it does not know the feature; that is harmless).
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
         "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build")
    return p


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


SAN_DIR = os.path.join(OBJDIR, "asan")
SAN_LIB = os.path.join(SAN_DIR, "libmoe_ffn_asan.so")


def asan_runtime():
    """Path of the compiler's AddressSanitizer runtime (it also carries the
    UndefinedBehaviorSanitizer handlers), or None."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    hits = sorted(glob.glob(os.path.join(root, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")) +
                  glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def build_sanitized(verbose: bool = False) -> str:
    """The library with its host code (the C ABI layer, api.cpp) built with
    AddressSanitizer and UndefinedBehaviorSanitizer, for the CPU tests of the
    ABI; device code is the regular build.  Load it with the sanitizer
    runtime preloaded (asan_runtime()).  Returns its path."""
    os.makedirs(SAN_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        if src == "api.cpp":
            continue
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(os.path.join(CSRC, src)):
            obj = _compile(src)
        objs.append(obj)
    api_obj = os.path.join(SAN_DIR, "api.o")
    # sanitizers on the host pass only (each -fsanitize= behind -Xarch_host)
    cmd = [hipcc(), "-xhip", *[f for f in FLAGS if f != "-O3"], "-O1", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-c", os.path.join(CSRC, "api.cpp"), "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc (sanitized api.cpp) failed:\n{r.stdout}\n{r.stderr}")
    # the sanitizer runtime is preloaded at run time, so the link needs no flag
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", api_obj, *objs, "-o", SAN_LIB],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (sanitized) failed:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
