"""Builds the native C++ check of the C ABI (tests/host/native_check.cpp): host
code only (HIP runtime API, libarrms, the C oracle), compiled with the host C++
compiler into tests/host/bin/, which build() calls on the CPU; the GPU test only
runs what is built."""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "bin", "native_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cxx = shutil.which("g++") or "c++"
    os.makedirs(os.path.dirname(BIN), exist_ok=True)
    cmd = [cxx, "-std=c++17", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "native_check.cpp"),
           "-L", os.path.join(ROOT, "tp_all_reduce_amd"), "-larrms",
           "-L", os.path.join(ROOT, "oracle"), "-loracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           # found again relative to the binary wherever the tree is copied
           "-Wl,-rpath,$ORIGIN/../../../tp_all_reduce_amd",
           "-Wl,-rpath,$ORIGIN/../../../oracle",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", BIN]
    print("+", " ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    return BIN


if __name__ == "__main__":
    build()
