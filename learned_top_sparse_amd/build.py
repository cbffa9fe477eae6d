"""Build liblsa.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: ``python -m learned_top_sparse_amd.build`` or ``build()`` from Python.
Object files go to ``_build/`` at the repository root (git-ignored); the
shared library lands next to this file so the binding finds it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblsa.so")
SOURCES = ["lsa_indexer.hip", "lsa_topk.hip", "lsa_attn.hip", "lsa_semantic.hip", "lsa_api.cpp", "lsa_noalloc.hip", "lsa_peaks.hip"]
# sources whose arithmetic decides integers (merges, kept buckets): no fused multiply-add
# unless written out, so every value is rounded in the order the source gives
NO_CONTRACT = {"lsa_semantic.hip"}

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden",
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    return os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


# host code under AddressSanitizer (device code is built as usual)
ASAN_DIR = os.path.join(BUILD_DIR, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "liblsa_asan.so")
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, verbose: bool, out_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + list(extra)
    if src in NO_CONTRACT:
        cmd.append("-ffp-contract=off")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every HIP source for gfx950 and link liblsa.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def build_host_asan(verbose: bool = False, jobs: int = 4) -> str:
    """liblsa with its host code built under AddressSanitizer, for tests of the host-side
    validation and planning; returns its path.  The process that loads it must have the
    ASan runtime (asan_runtime()) preloaded."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, ASAN_DIR, ASAN_HOST), SOURCES))
    tmp = ASAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + ASAN_HOST
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"asan link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


def asan_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (to preload)."""
    r = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no shared AddressSanitizer runtime found")
    return hits[-1]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
