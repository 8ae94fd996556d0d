"""Builds libqmv.so (the HIP kernels and the C ABI of include/qmv.h) in-tree
for gfx950 with hipcc.  `python -m block_quant_weight_amd.build` runs it."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libqmv.so")
ARCH = "gfx950"

# Packed float32 VALU forms are turned off for all device code (the compiler
# may otherwise pair float32 operations into v_pk_* instructions).
HIP_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]
HIP_SOURCES = ["gemv.hip", "gemv_mfma.hip", "gemm.hip", "gemm_i8.hip", "misc.hip", "writer.hip",
               "qmv_api.cpp"]
HOST_SOURCES = ["qmv_host.cpp"]  # no HIP: plain g++
# Per-file flags.  The int8 product reads every matrix-core result with
# vector instructions; in the accumulation-register form each result would
# first be copied out (one extra instruction per output per block).
FILE_FLAGS = {"gemm_i8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    return p


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmd = ["hipcc", *HIP_FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = ["hipcc", *HIP_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        jobs.append((obj, cmd))
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append((obj, ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE,
                           "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for obj, cmd in jobs:
            if verbose:
                print(" ".join(cmd), file=sys.stderr)
        list(ex.map(lambda j: _run(j[1]), jobs))
    tmp = LIB_PATH + ".tmp"
    _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
          *[o for o, _ in jobs]])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
