"""Builds libarrms.so in-tree: the host-only plan/validation unit with the host
C++ compiler, the run unit and the six kernel units (each instantiates one
slice of the kernel variants) with hipcc for gfx950, all compiled in
parallel, then linked by hipcc.

    python -m tp_all_reduce_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

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


# The run unit (entry points, no device code) and the kernel units.
HIP_UNITS = ["arrms", "rms_bf16", "rms_bf16_fp8", "rms_fp16", "rms_fp16_fp8", "qk_bf16", "qk_fp16"]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def _jobs() -> int:
    for var in ("MAX_JOBS", "CMAKE_BUILD_PARALLEL_LEVEL"):
        if os.environ.get(var, "").isdigit() and int(os.environ[var]) > 0:
            return int(os.environ[var])
    return os.cpu_count() or 1


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    cmds = [[CXX, *HOST_FLAGS, "-c", os.path.join(CSRC, "plan.cpp"),
             "-o", os.path.join(BUILD, "plan.o")]]
    cmds += [[HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, u + ".hip"),
              "-o", os.path.join(BUILD, u + ".o")] for u in HIP_UNITS]
    with ThreadPoolExecutor(max_workers=max(1, min(_jobs(), len(cmds)))) as pool:
        for f in [pool.submit(_run, c) for c in cmds]:
            f.result()
    objs = [c[-1] for c in cmds]
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
