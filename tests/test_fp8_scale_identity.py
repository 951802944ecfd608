"""The FP8 epilogue's scale amax / 448 without a division: the product with
RN(1/448) plus one FMA correction equals the IEEE quotient wherever the kernel
uses it (amax >= 2^-116), checked bit for bit on the CPU (tests/host/div448_check.c)
over the binades at the guard, a middle one and the top one.  The check over
every positive float was also run once; below the guard, where quotients are
subnormal, the form does differ, so the kernel divides there."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "div448_check.c")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    out = str(tmp_path_factory.mktemp("div448") / "div448_check")
    # no contraction: the products and FMAs are exactly the ones written
    subprocess.run([cc, "-std=c99", "-O2", "-ffp-contract=off", SRC, "-o", out, "-lm"],
                   check=True)
    return out


def run(exe, *ranges):
    r = subprocess.run([exe, *map(str, ranges)], capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout.strip()


def test_identity_where_the_kernel_uses_it(exe):
    rc, out = run(exe, -116, -112, -1, 1, 126, 128)
    assert rc == 0 and out.startswith("OK"), out
    assert int(out.split()[1]) == 8 * (1 << 23)


def test_identity_fails_below_the_guard(exe):
    """Quotients in the subnormal range: the guard is needed."""
    rc, out = run(exe, -149, -117)
    assert rc == 1 and out.startswith("MISMATCH"), out
