"""Build ``libbitnet_hip.so`` (the C-ABI library) in-tree with hipcc for gfx950.

Each HIP translation unit is compiled to an object in ``_build/`` (in parallel)
and the objects are linked into ``bit_gemm_ternary_amd/libbitnet_hip.so``.
Floating-point flags: no FMA contraction and IEEE-correct float32 division and
square root, so the kernels' float operations match their definitions; packed
FP32 instructions are disabled.

Run ``python -m bit_gemm_ternary_amd.build`` or call :func:`build`.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbitnet_hip.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "pack.hip", "quant_act.hip", "hadamard_quant.hip", "hadamard_decode.hip", "gemv.hip", "gemm_mfma.hip",
           "backward.hip", "base3.hip", "dequant.hip", "stream_read.hip", "blend.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj


def build(jobs: int = 6) -> str:
    """Compile every source and link the shared library; return its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        objs = list(pool.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
