"""Build libcacheblend.so in-tree with hipcc for gfx950.

    python -m selective_recompute_amd.build          # compile every source
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
LIB = os.path.join(PKG, "libcacheblend.so")
PEAKS = os.path.join(PKG, "cb_peaks")    # attainable-peak probe run by bench.py

SOURCES = ["api.cpp", "stream_kernels.hip", "attn_kernels.hip", "scratch.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _flags():
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
        "-Wall", "-Wno-unused-result",
        # keep the compiler from forming packed fp32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [_hipcc(), *_flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source and link libcacheblend.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-fvisibility=hidden", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    cmd = [_hipcc(), *_flags(), "-x", "hip", os.path.join(CSRC, "peaks.hip"), "-o", PEAKS + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on peaks.hip:\n{res.stdout}\n{res.stderr}")
    os.replace(PEAKS + ".tmp", PEAKS)
    if verbose:
        print(f"built {LIB} and {PEAKS}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
