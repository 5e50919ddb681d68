"""Builds libsparse_attn.so (gfx950) in-tree with hipcc.

    python block_sparse_attention_hilbert_amd/build.py

(run by path: importing the package loads the library this script builds)
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsparse_attn.so")
SOURCES = ["sa_api.cpp", "hilbert.cpp", "k_select.hip", "k_attn.hip", "k_permute.hip", "k_route.hip",
           "k_cluster.hip", "k_tiles.hip", "sa_noalloc.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            # keep the compiler from forming packed fp32 instructions
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include")]


# Per-source extra flags.  The attention kernel keeps its softmax operands in
# VGPRs: the matrix-core accumulators of S are read by VALU code every tile, so
# the VGPR form of the MFMA instructions avoids AGPR<->VGPR copies.
EXTRA = {"k_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = ([_hipcc()] + common_flags() + EXTRA.get(src, []) + lang +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
