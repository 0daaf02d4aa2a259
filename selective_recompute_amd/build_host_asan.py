"""The library with AddressSanitizer on its host code only (argument checks,
planner, launch order); the device code is not instrumented.

    python -m selective_recompute_amd.build_host_asan DIR

Load the result with CB_LIBRARY=DIR/libcacheblend.so,
LD_PRELOAD=<clang's libclang_rt.asan-x86_64.so> and
ASAN_OPTIONS=detect_leaks=0, e.g. to run the host tests (tests/test_abi.py).
A CPU-side check: no GPU run uses this build.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

from selective_recompute_amd import build as B

# -fsanitize follows -Xarch_host each time, so no GPU code is built with it.
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, out_dir: str) -> str:
    obj = os.path.join(out_dir, src + ".o")
    cmd = [B._hipcc(), *B._flags(), *HOST_ASAN, "-x", "hip", "-c",
           os.path.join(B.CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build_host_asan(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(B.SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, out_dir), B.SOURCES))
    lib = os.path.join(out_dir, "libcacheblend.so")
    cmd = [B._hipcc(), "-shared", f"--offload-arch={B.ARCH}", "-fvisibility=hidden",
           "-Xarch_host", "-fsanitize=address", "-shared-libasan", *objs, "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    return lib


if __name__ == "__main__":
    if len(sys.argv) != 2:
        sys.exit("usage: python -m selective_recompute_amd.build_host_asan DIR")
    print(build_host_asan(sys.argv[1]))
