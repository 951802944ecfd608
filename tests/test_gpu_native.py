"""The C ABI from C++ with no Python in the path (tests/host/native_check.cpp,
built by __graft_entry__.build()): device memory and a stream from the HIP
runtime, one call of each entry point, outputs checked against the C oracle."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "host"))
import native  # noqa: E402

pytestmark = pytest.mark.gpu


def test_native_cpp_caller():
    if not os.path.exists(native.BIN):
        pytest.skip("the native check is not built (__graft_entry__.build() builds it)")
    print(f"[native] {native.BIN}", flush=True)
    run = subprocess.run([native.BIN], capture_output=True, text=True, timeout=300)
    print(run.stdout)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "OK: 0 failures" in run.stdout
