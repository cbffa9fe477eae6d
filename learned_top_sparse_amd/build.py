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


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON
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


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
