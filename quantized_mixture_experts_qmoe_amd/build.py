"""Builds libqmoe.so (the HIP library behind include/qmoe.h) in-tree for gfx950.

    python -m quantized_mixture_experts_qmoe_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqmoe.so")

ARCH = "gfx950"
# Packed-FP32 VALU instructions are disabled in every kernel.
# MFMA results are kept in architectural VGPRs (the grouped GEMMs scale them
# with VALU FMAs every group; AGPR placement would add a read per element).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    steps = [
        ("qmoe_kernels.hip", ["-x", "hip"] + HIP_FLAGS),
        # the device quantizer: the host quantizer's arithmetic, no contraction
        ("qmoe_quant.hip", ["-x", "hip"] + HIP_FLAGS + ["-ffp-contract=off"]),
        ("qmoe_api.cpp", HOST_FLAGS),
        # the host quantizer: plain IEEE fp32, no contraction, no fast-math
        ("qmoe_pack.cpp", HOST_FLAGS + ["-ffp-contract=off", "-fno-fast-math"]),
    ]
    for src, flags in steps:
        obj = os.path.join(BUILD, src.rsplit(".", 1)[0] + ".o")
        cmd = ["hipcc"] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        _run(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = ["hipcc", "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd))
    _run(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
