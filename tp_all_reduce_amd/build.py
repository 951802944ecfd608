"""Builds libarrms.so in-tree: the host-only plan/validation unit with the host
C++ compiler, the HIP unit with hipcc for gfx950, linked by hipcc.

    python -m tp_all_reduce_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libarrms.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CXX = os.environ.get("CXX_HOST") or shutil.which("g++") or "c++"

# Packed-fp32 VALU ops are disabled for every HIP unit; hipcc's host pass warns
# that it does not know the feature, which is harmless.
# Kernel arguments: the first eight of every kernel (at most 14 dwords) are
# preloaded into SGPRs at wave launch (the code object keeps a loading prologue
# for firmware without it).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-kernarg-preload-count=8",
             "-I", INCLUDE]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    plan_o = os.path.join(BUILD, "plan.o")
    hip_o = os.path.join(BUILD, "arrms.o")
    _run([CXX, *HOST_FLAGS, "-c", os.path.join(CSRC, "plan.cpp"), "-o", plan_o])
    _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "arrms.hip"), "-o", hip_o])
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", plan_o, hip_o, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
