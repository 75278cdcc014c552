"""Build libmsq.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m memory_streamed_qlora_amd.build   (or build_library() from Python)

Every HIP translation unit is compiled with packed-fp32 instruction selection
disabled and fp32 denormals preserved (the NF4 dequantization is bit-exact for
subnormal products too).  Objects go to _build/ (not committed); the shared
library lands next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmsq.so")
BUILD = os.path.join(ROOT, "_build", "msq")
ARCH = os.environ.get("MSQ_OFFLOAD_ARCH", "gfx950")

SOURCES = ["abi.cpp", "codebook.cpp", "window.cpp", "loader.cpp", "timing.cpp", "quant.hip",
           "gemm.hip", "lora.hip", "glue.hip", "noalloc.hip", "optim.hip", "hostcopy.hip", "small.hip"]

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MI355X build needs ROCm's hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        sys.stderr.write(msg + "\n")
    return obj


def build_library(verbose: bool = True) -> str:
    """Compile every source and link libmsq.so; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    t0 = time.time()
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"[msq build] {OUT} ({os.path.getsize(OUT) / 1e6:.1f} MB) in {time.time() - t0:.1f}s")
    return OUT


if __name__ == "__main__":
    build_library()
