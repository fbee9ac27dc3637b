"""Build libcpr_gdn.so in place (hipcc, gfx950).

Usage: python bitwise_aligned_gated_amd/build.py   (run by path: importing the package needs the
library to exist already).
Every HIP translation unit is compiled with the flags that pin the arithmetic: no FMA
contraction beyond the explicit fmaf calls, no fast-math, IEEE fp32 denormals, and packed fp32
instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libcpr_gdn.so")
BUILD_DIR = os.environ.get("CPR_BUILD_DIR", os.path.join(ROOT, "_build"))

SOURCES = ["cpr_prefill.hip", "cpr_overlap.hip", "cpr_decode.hip", "cpr_backward.hip", "cpr_chunked.hip",
           "cpr_chunked_bwd.hip",
           "cpr_static.hip", "cpr_host.cpp"]
EXTRA_FLAGS = os.environ.get("CPR_EXTRA_HIPCC_FLAGS", "").split()
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build_library(verbose: bool = False) -> str:
    """Compile every source and link libcpr_gdn.so next to this file; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
