"""Build libqmoe.so in-tree with hipcc for gfx950.

    python -m quantized_moe_02_amd.build        (or __graft_entry__.build())

Every source is compiled on each call; objects go to _build/ at the repository
root and the shared library next to this file, where the binding loads it.
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
OUT = os.path.join(PKG, "libqmoe.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["qmoe_api.cpp", "route.hip", "permute.hip", "gemv.hip", "decode.hip", "gemm.hip",
           "gemm_i8.hip", "noalloc.hip", "expert_cache.cpp"]

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Wall", "-Wno-unused-function",
          # keep the compiler from forming packed fp32 VALU ops
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    # counter-calibration kernels, a library of their own (benchmark only)
    cal = os.path.join(PKG, "libqmoe_calib.so")
    cmd = [HIPCC, *COMMON, "-shared", os.path.join(CSRC, "calib.hip"), "-o", cal + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for calib.hip:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(cal + ".tmp", cal)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
