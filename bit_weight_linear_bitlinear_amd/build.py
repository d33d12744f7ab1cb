"""Build liblowbit.so in-tree with hipcc for gfx950.

Every HIP file is compiled with -ffp-contract=off (the quantiser and the
epilogues are specified operation by operation), without fast-math, with
denormals kept, and with the packed-fp32 target feature switched off.
"""
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
LIB = os.path.join(HERE, "liblowbit.so")
ARCH = os.environ.get("LOWBIT_OFFLOAD_ARCH", "gfx950")

SOURCES = ["act_quant.hip", "hadamard.hip", "bitnet_v1.hip", "onebit.hip", "sparse8.hip", "gemv.hip", "gemv_ternary.hip", "gemv_int4.hip", "gemv_binary.hip", "gemm.hip",
           "decode_model.hip",
           "gemm_mfma.hip", "calib.hip", "lowbit_host.cpp"]

COMMON = ["-std=c++17", "-O3", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
          "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]
DEVICE = [f"--offload-arch={ARCH}", "-fno-gpu-flush-denormals-to-zero",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# the decode GEMV keeps its MFMA accumulators in ordinary VGPRs (its group
# epilogue reads them every few MFMAs; no accumulation-register copies)
EXTRA = {f"gemv_{f}.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"] for f in ("ternary", "int4", "binary")}


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, *DEVICE, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-pthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
