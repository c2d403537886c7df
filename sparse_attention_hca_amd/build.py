"""Build libhca.so (all HIP kernels + the C-ABI layer) for gfx950 with hipcc.

Usage: python -m sparse_attention_hca_amd.build   (or build() from Python)
The library is written in-tree next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhca.so")
ARCH = os.environ.get("HCA_OFFLOAD_ARCH", "gfx950")

SOURCES = [
    "compress.hip",
    "append.hip",
    "attn_generic.hip",
    "attn_f32mfma.hip",
    "attn_bf16mfma.hip",
    "attn_prefill512.hip",
    "attn_decode512.hip",
    "dsa_index_topk.hip",
    "dsa_attn256.hip",
    "attn_bwd.hip",
    "attn_bwd512.hip",
    "epilogue.hip",
    "dsa_bwd256.hip",
    "hca_abi.cpp",
]

# Packed-fp32 VALU forms are disabled for all device code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _compile(src: str, outdir: str) -> str:
    obj = os.path.join(outdir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    outdir = os.path.join(HERE, "_build")
    os.makedirs(outdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, outdir), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
