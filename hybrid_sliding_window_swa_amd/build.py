"""Build libswa_attn.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m hybrid_sliding_window_swa_amd.build

Every source is compiled on each call (the build is the "does it compile"
check); objects go to ``_build/`` next to this file and the shared library
to ``libswa_attn.so`` beside it.  The same call builds ``swa_peaks``, a small
program that measures the HBM and MFMA ceilings the kernels are compared with.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libswa_attn.so")
PEAKS = os.path.join(PKG, "swa_peaks")
ARCH = os.environ.get("SWA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.hip", "validate.c", "prefill_bf16.hip", "verify_bf16.hip", "fp32_kernels.hip", "append.hip",
           "accept.hip", "rope.hip", "backward_bf16.hip", "noalloc.hip"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".c"):
        cmd = [hipcc(), "-x", "c", "-std=c99", "-O2", "-fPIC", "-fvisibility=hidden", "-Wall", "-I", INCLUDE, "-I", CSRC,
               "-c", path, "-o", obj]
    else:
        cmd = [hipcc(), *HIP_FLAGS, "-fPIC", "-fvisibility=hidden", "-I", INCLUDE, "-I", CSRC, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{r.stdout}\n{r.stderr}")
    return obj


HIP_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build_peaks() -> str:
    cmd = [hipcc(), *HIP_FLAGS, os.path.join(CSRC, "peaks.hip"), "-o", PEAKS + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of peaks.hip failed:\n{r.stdout}\n{r.stderr}")
    os.replace(PEAKS + ".tmp", PEAKS)
    return PEAKS


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        peaks = ex.submit(build_peaks)
        objs = list(ex.map(_compile, SOURCES))
        peaks.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, "and", PEAKS)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
