"""include/arrms.h as a C99 header: a C program compiled with -pedantic -Werror
and linked against libarrms.so runs the host-side entry points (CPU only)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "tp_all_reduce_amd")


def test_c99_consumer(tmp_path):
    cc = shutil.which("gcc")
    lib = os.path.join(PKG, "libarrms.so")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(lib):
        pytest.skip("libarrms.so is not built")
    exe = str(tmp_path / "c_consumer")
    build = subprocess.run(
        [cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
         "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "host", "c_consumer.c"),
         "-L", PKG, "-larrms", f"-Wl,-rpath,{PKG}", "-o", exe],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("OK"), run.stdout
