"""Host-side logic of bench.py, without a GPU: the algorithmic byte count, the
source hash that ties recorded counters to the kernel sources, the argument
checks and step plan (run before torch is imported, so that a bad argument
costs no GPU), and the refusal of runs on more than one GPU."""
import json
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


def run_bench(*argv):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                          capture_output=True, text=True, timeout=120)


def steps_of(graphs):
    """Steps covered by a {steps per graph: graphs} summary."""
    return sum(int(n) * k for n, k in graphs.items())


def test_short_invocation_is_accepted_before_any_gpu_work():
    """`bench.py --gpus 1 --steps 20 --warmup 5 --check-args` (a warm-up that
    is not a multiple of the steps per graph): the arguments pass, exactly 20
    steps are timed after exactly 5 warm-up steps, and torch has not been
    imported by then."""
    r = run_bench("--gpus", "1", "--steps", "20", "--warmup", "5", "--check-args")
    assert r.returncode == 0, r.stderr
    plan = json.loads(r.stdout)
    assert plan["timed_steps"] == 20 and steps_of(plan["timed_graphs"]) == 20
    assert plan["warmup_steps"] == 5 and steps_of(plan["warmup_graphs"]) == 5
    assert plan["torch_imported"] is False


def test_default_invocation_is_accepted():
    r = run_bench("--check-args")
    assert r.returncode == 0, r.stderr
    plan = json.loads(r.stdout)
    assert steps_of(plan["timed_graphs"]) == plan["timed_steps"] >= 1


def test_bad_arguments_fail_fast_without_torch():
    for argv, what in ((["--steps", "0"], "--steps"), (["--warmup", "-1"], "--warmup"),
                       (["--steps-per-graph", "0"], "--steps-per-graph")):
        r = run_bench(*argv)
        assert r.returncode == 2, (argv, r.stderr)
        assert what in r.stderr and r.stdout == ""


def test_step_pieces_cover_exactly_the_requested_steps():
    for count in range(0, 57):
        for per in (1, 3, 10, 64):
            p = bench.pieces(count, per)
            assert sum(p) == count
            assert all(1 <= n <= per for n in p)
            # whole graphs first, at most one remainder graph, at the end
            assert all(n == per for n in p[:-1])


def test_cold_rotation_exceeds_the_caches():
    """The cold figures rotate through more than 512 MiB of sets (at least
    three), in whole graphs when there are more sets than calls per graph."""
    for set_bytes in (81920, 1 << 20, 18_874_368, 27_596_800, 184_565_760, 600 << 20):
        for calls in (10, 100):
            n = bench.cold_sets(set_bytes, calls)
            assert n >= 3
            assert n * set_bytes > bench.COLD_BYTES or set_bytes > bench.COLD_BYTES
            if n > calls:
                assert n % calls == 0


def test_pool_sets_are_aligned_disjoint_and_replicated():
    """The cold rotation's sets: every tensor 4 KiB-aligned within one
    allocation, no two overlapping (within a set or across sets), and every set
    holding the values copied into the first."""
    shapes = [(8, 1024), (3, 7), (80, 4096), (1, 8)]
    sizes = [bench.Pool.span(s) for s in shapes]
    assert all(n % 4096 == 0 and n >= 2 * a * b for n, (a, b) in zip(sizes, shapes))
    assert bench.Pool.size_of(shapes) == sum(sizes)
    p = bench.Pool(torch, "cpu", shapes, 3, torch.bfloat16)
    vals = [torch.randn(s).to(torch.bfloat16) for s in shapes[:2]]
    sets = p.sets(vals)
    base = p.buf.data_ptr()
    spans = sorted((t.data_ptr(), t.data_ptr() + t.numel() * 2) for st in sets for t in st)
    assert all((a - base) % 4096 == 0 for a, _ in spans)
    assert all(spans[i][1] <= spans[i + 1][0] for i in range(len(spans) - 1))
    assert spans[-1][1] <= base + p.buf.numel() * 2
    for st in sets:
        assert [tuple(x.shape) for x in st] == shapes
        for x, v in zip(st, vals):
            assert torch.equal(x, v)
