"""Host-side logic of bench.py, without a GPU: the algorithmic byte count, the
source hash that ties recorded counters to the kernel sources, and the refusal
of runs on more than one GPU."""
import os
import shutil
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from tp_all_reduce_amd import workloads  # noqa: E402
from tp_all_reduce_amd.workloads import WORKLOADS  # noqa: E402


def tensor_bytes(*ts):
    return sum(t.numel() * t.element_size() for t in ts)


def touched(wl, T):
    """Bytes of every tensor one fused call reads or writes once, counted from
    the tensors themselves: the partials, the residual and the weight read, the
    two 16-bit outputs written, and with the FP8 epilogue the codes and the
    fp32 scales."""
    inp = workloads.make_inputs(wl, T)
    norm_out = torch.empty_like(inp["residual"])
    residual_out = torch.empty_like(inp["residual"])
    n = tensor_bytes(*inp["partials"], inp["residual"], inp["weight"], norm_out, residual_out)
    if wl.group:
        codes = torch.empty(norm_out.shape, dtype=torch.uint8)
        scales = torch.empty((T, wl.H // wl.group), dtype=torch.float32)
        n += tensor_bytes(codes, scales)
    return n


def test_rms_bytes_match_the_tensors_a_call_touches():
    for name in ("c1", "c2", "c4"):
        wl = WORKLOADS[name]
        for T in wl.Ts:
            assert bench.rms_bytes(wl.W, T, wl.H, wl.group) == touched(wl, T), (name, T)
    c3 = WORKLOADS["c3"]
    assert bench.rms_bytes(c3.W, 1024, c3.H) == touched(c3, 1024)


def test_decode_sweep_bytes_per_launch():
    """The headline's bytes per launch: the mean over the sweep's calls."""
    wl = WORKLOADS["c2"]
    mean = sum(touched(wl, T) for T in wl.Ts) / len(wl.Ts)
    assert mean == 1441792.0
    assert sum(bench.rms_bytes(wl.W, T, wl.H) for T in wl.Ts) / len(wl.Ts) == mean


def test_rms_bytes_without_residual():
    wl = WORKLOADS["c2"]
    inp = workloads.make_inputs(wl, 8)
    out = torch.empty_like(inp["residual"])
    assert bench.rms_bytes(wl.W, 8, wl.H, residual=False) == tensor_bytes(
        *inp["partials"], inp["weight"], out, out)


def test_source_hash_ignores_comments_and_whitespace(tmp_path):
    src = os.path.join(ROOT, "tp_all_reduce_amd", "csrc")
    copy = tmp_path / "csrc"
    shutil.copytree(src, copy)
    base = bench.kernel_source_sha(str(copy))
    assert base == bench.kernel_source_sha(src)

    k = copy / "kernels.h"
    text = k.read_text()
    k.write_text("// a new comment line\n" + text.replace("{\n", "{  \n\n", 3) + "\n/* block */\n")
    assert bench.kernel_source_sha(str(copy)) == base

    (copy / "notes.txt").write_text("not a source file")
    assert bench.kernel_source_sha(str(copy)) == base


def test_source_hash_sees_code_changes(tmp_path):
    src = os.path.join(ROOT, "tp_all_reduce_amd", "csrc")
    copy = tmp_path / "csrc"
    shutil.copytree(src, copy)
    base = bench.kernel_source_sha(str(copy))

    k = copy / "kernels.h"
    text = k.read_text()
    assert "row16_sum(v)" in text
    k.write_text(text.replace("row16_sum(v)", "row16_sum(v + 0.0f)", 1))
    changed = bench.kernel_source_sha(str(copy))
    assert changed != base
    k.write_text(text)
    assert bench.kernel_source_sha(str(copy)) == base

    # every kernel unit counts, also one added later
    (copy / "extra.hip").write_text('#include "kernels.h"\n')
    assert bench.kernel_source_sha(str(copy)) != base
    os.remove(copy / "extra.hip")
    plan = copy / "plan.cpp"
    plan.write_text(plan.read_text() + "\nstatic int unused_marker = 1;\n")
    assert bench.kernel_source_sha(str(copy)) != base


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
