"""Builds libhc.so in-tree from csrc/ with hipcc for gfx950.

Flags: -O3, -ffp-contract=off (no fused multiply-add contraction: every hop is
one IEEE add), no fast-math, no flush-to-zero, packed-fp32 instructions
disabled on the device (-Xclang -target-feature -Xclang -packed-fp32-ops).
Objects go to _build/ at the repository root; the library lands next to this
file so that it travels with the tree.  The two measurement programs of
measure/ at the repository root are built there: dma_contention (linked
against libhc and rocBLAS from the system ROCm) and hbm_ceiling.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhc.so")
MEASURE = os.path.join(ROOT, "measure")
DMA_TOOL = os.path.join(MEASURE, "dma_contention")
CEILING_TOOL = os.path.join(MEASURE, "hbm_ceiling")
ARCH = os.environ.get("HC_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["hc_api.cpp", "schedule.cpp", "ring_kernels.hip", "codec_kernels.hip", "car_chain.hip",
           "entropy_kernels.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    tmp = DMA_TOOL + ".tmp"
    cmd = [HIPCC, *COMMON, *DEVICE, "-x", "hip", os.path.join(MEASURE, "dma_contention.hip"), "-o", tmp,
           "-L", PKG, "-lhc", "-Wl,-rpath,$ORIGIN/../collective_communication_amd", "-L/opt/rocm/lib", "-lrocblas", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"dma_contention build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, DMA_TOOL)
    tmp = CEILING_TOOL + ".tmp"
    cmd = [HIPCC, *COMMON, *DEVICE, "-x", "hip", os.path.join(MEASURE, "hbm_ceiling.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hbm_ceiling build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, CEILING_TOOL)
    if verbose:
        print(f"built {LIB}, {DMA_TOOL} and {CEILING_TOOL}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
