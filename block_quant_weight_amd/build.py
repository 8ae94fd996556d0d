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


def _stale(obj: str, src: str) -> bool:
    """True when obj is missing or older than its source or any header."""
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [src] + [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".h")]
    deps += [os.path.join(INCLUDE, h) for h in os.listdir(INCLUDE)]
    return any(os.path.getmtime(dp) > t for dp in deps)


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compiles every source (incremental=True: only those whose object is
    older than the source or a header) and links libqmv.so."""
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
    todo = [j for j in jobs if not incremental or _stale(j[0], j[1][-3])]
    with ThreadPoolExecutor(max_workers=max(1, min(8, len(todo)))) as ex:
        for obj, cmd in todo:
            if verbose:
                print(" ".join(cmd), file=sys.stderr)
        list(ex.map(lambda j: _run(j[1]), todo))
    tmp = LIB_PATH + ".tmp"
    _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
          *[o for o, _ in jobs]])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv))
