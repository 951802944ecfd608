"""Benchmark of the fused W-way reduce + residual add + RMSNorm (libarrms).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--steps-per-graph G]
                    [--no-cpu-baseline] [--no-others] [--no-unfused] [--headline-only]
                    [--check-args] [--copy-calibration] [--only c1|c3|c4|c5]

Headline workload: the decode-window sweep, W=4 partial buffers of [T, 4096]
bf16 with Gemma RMSNorm, eps 1e-6, T in {1, 2, 4, 8, 16, 21, 22, 32, 64, 80},
row-resident kernel.  One step is one pass over the sweep: ten fused calls,
one per T; the inputs are resident in HBM before the timed region starts.
Steps are launched from HIP graphs that hold up to G steps each (default 20,
200 calls: a captured decode step holds every layer's epilogues, two per
layer, and each graph launch costs the device a few microseconds once per
graph; the line reports that cost as graph_launch_us).  Any K and W are
accepted: the warm-up and the timed steps are cut into graphs of G steps and
one graph of the remainder, all captured before the warm-up; exactly K steps
are timed with HIP events on the replaying stream, the start event queued
behind the last warm-up replay, and the device is synchronised before that
replay and after the timed steps.
value = microseconds per fused call (timed region / (10 K)).

Beside the headline, the same sweep is timed
  cold            input and output sets rotated through more than 512 MiB, so
                  no call finds its rows in the L2 caches or the 256 MB
                  Infinity Cache;
  dependent chain every call adds into one shared residual buffer in place
                  (its residual is the previous call's residual_out), as a
                  layer-by-layer decode step does: consecutive calls cannot
                  overlap;
and every other workload is timed the same way, warm (one set) and cold
(rotated through more than 512 MiB), next to the oracle's time on the host's
cores for the same inputs (median of three runs; one for the largest).

The roofline object covers the dominant kernel (the row-resident kernel, every
launch of the step): algorithmic bytes per launch, (W + 3) * T * H * 2 + H * 2
(W partials and the residual read, norm_out and residual_out written, the
weight read once) averaged over the sweep, divided by that kernel's average
launch time over the timed region (HIP events on the replaying stream).
`traffic`, and the rocprofv3 duration of the same kernel, are read from the
committed counter summary when it was taken on the current kernel sources,
else null.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = ("µs/call at T<=80 and effective HBM GB/s (% of MI355X peak) for W-way "
          "reduce+add-RMSNorm")
KERNEL_SRC = os.path.join(ROOT, "tp_all_reduce_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_row_kernel_c2_sweep.json")
COLD_BYTES = 512 << 20          # a rotation through more than this misses every cache
MAX_THREADS = 16                # host threads of the all-cores oracle timing


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def rms_bytes(W, T, H, group=0, residual=True):
    """Algorithmic HBM bytes of one fused call on 16-bit data: W partials and
    the residual read, residual_out and norm_out written, the weight read once;
    with the FP8 epilogue also the codes (1 byte per element) and the fp32
    group scales."""
    n = (W + (1 if residual else 0) + 2) * T * H * 2 + H * 2
    if group:
        n += T * H + 4 * T * (H // group)
    return n


def qk_bytes(W, T, q_size, kv_size):
    """Algorithmic bytes of one QK-norm call: the q and k columns of every
    shard read and written once, both weights read once (v is not touched)."""
    return 2 * W * T * (q_size + kv_size) * 2 + W * (q_size + kv_size) * 2


def kernel_source_sha(path: str = KERNEL_SRC) -> str:
    """Hash of the code of every source file of the library (the kernel units,
    their headers, the run unit and the plan code, in name order): comments and
    whitespace are dropped, so a comment edit does not void the recorded
    counters (the sources hold no string literal with a comment marker)."""
    parts = []
    for name in sorted(os.listdir(path)):
        if not name.endswith((".hip", ".h", ".cpp")):
            continue
        src = open(os.path.join(path, name), encoding="utf-8").read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        parts.append(name + ": " + " ".join(src.split()))
    return hashlib.sha256("\n".join(parts).encode()).hexdigest()[:16]


# ------------------------------------------------------------ arguments
def parser():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000, help="timed steps (any K >= 1)")
    ap.add_argument("--warmup", type=int, default=200, help="untimed steps before (any W >= 0)")
    ap.add_argument("--steps-per-graph", type=int, default=20,
                    help="steps held by one HIP graph (the last graph holds the remainder)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timings on the host")
    ap.add_argument("--no-others", "--no-large-t", dest="no_others", action="store_true",
                    help="skip the other workloads (c1, c3 T=1024/8192/16384, c4, c5)")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip timing the unfused PyTorch composition (profiled runs)")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline sweep (profiled runs): implies --no-others, "
                         "--no-unfused and --no-cpu-baseline and skips the secondary sweep "
                         "figures")
    ap.add_argument("--only", default=None, choices=["c1", "c3", "c4", "c5"],
                    help="time only this other workload after the headline (profiled runs)")
    ap.add_argument("--check-args", action="store_true",
                    help="validate the arguments, print the step plan and exit (no GPU)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (for counter calibration)")
    return ap


def validate(args):
    """Problems with the arguments (empty list: fine).  Checked before torch is
    imported or the GPU is touched."""
    bad = []
    if args.gpus < 1:
        bad.append(f"--gpus must be >= 1 (got {args.gpus})")
    if args.steps < 1:
        bad.append(f"--steps must be >= 1 (got {args.steps})")
    if args.warmup < 0:
        bad.append(f"--warmup must be >= 0 (got {args.warmup})")
    if args.steps_per_graph < 1:
        bad.append(f"--steps-per-graph must be >= 1 (got {args.steps_per_graph})")
    return bad


def pieces(count, per_graph):
    """Steps per graph replay for `count` steps: whole graphs of per_graph
    steps, then one graph of the remainder."""
    return [per_graph] * (count // per_graph) + ([count % per_graph] if count % per_graph else [])


def step_plan(args):
    spg = args.steps_per_graph
    return {"warmup_graphs": pieces(args.warmup, spg),
            "timed_graphs": pieces(args.steps, spg),
            "timed_steps": args.steps, "warmup_steps": args.warmup, "steps_per_graph": spg}


def parse(argv=None):
    args = parser().parse_args(argv)
    bad = validate(args)
    if bad:
        print("bench.py: " + "; ".join(bad), file=sys.stderr)
        sys.exit(2)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library is the single-GPU kernel of the "
              "fused all-reduce + RMSNorm epilogue (W partial buffers resident on one device); "
              "multi-GPU runs are not part of it. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.headline_only:
        args.no_others = args.no_unfused = args.no_cpu_baseline = True
    return args


# ------------------------------------------------------------ GPU timing
class Pool:
    """Rotating sets of 16-bit tensors in one device allocation: every set holds
    the same shapes at the same 4 KiB-aligned offsets, one set after another."""

    def __init__(self, torch, dev, shapes, n_sets, dtype):
        self.shapes = list(shapes)
        self.per_set = self.size_of(self.shapes)
        self.n_sets = n_sets
        self.buf = torch.empty(n_sets * self.per_set // 2, dtype=dtype, device=dev)
        self.offsets = []
        off = 0
        for sh in self.shapes:
            self.offsets.append(off)
            off += self.span(sh)

    @staticmethod
    def span(shape):
        return -(-math.prod(shape) * 2 // 4096) * 4096

    @classmethod
    def size_of(cls, shapes):
        return sum(cls.span(s) for s in shapes)

    def tensor(self, s, i):
        """Tensor i of set s."""
        a = (s * self.per_set + self.offsets[i]) // 2
        return self.buf[a: a + math.prod(self.shapes[i])].view(*self.shapes[i])

    def sets(self, values):
        """Copies `values` (one tensor per leading shape) into set 0, then set 0
        into every other set with one broadcast copy; returns every set's
        tensors."""
        for i, v in enumerate(values):
            self.tensor(0, i).copy_(v.reshape(self.shapes[i]))
        rows = self.buf.view(self.n_sets, self.per_set // 2)
        if self.n_sets > 1:
            rows[1:].copy_(rows[:1].expand(self.n_sets - 1, -1))
        return [[self.tensor(s, i) for i in range(len(self.shapes))] for s in range(self.n_sets)]


def capture(torch, launch, stream):
    """A HIP graph of launch() on `stream`, after one eager run of the same
    calls, and replayed once (a graph's first replay also uploads it: that
    cost belongs to the capture, not to the steps timed later)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        launch()
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            launch()
        g.replay()
    torch.cuda.synchronize()
    return g


def replay_timed(torch, stream, warm, timed):
    """Replays the graphs `warm` (untimed), then `timed`; returns the elapsed ms
    of the timed replays measured with HIP events on `stream`, the stream they
    are replayed on.  The device is synchronised before the last warm-up replay
    and after the timed ones.  That last warm-up replay is still running when
    the start event and the timed replays are queued, so the timed region opens
    on a queued kernel and does not include the host's launch of the first
    timed graph (with no warm-up graph it does)."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for g in warm[:-1]:
            g.replay()
        torch.cuda.synchronize()
        if warm:
            warm[-1].replay()
        start.record(stream)
        for g in timed:
            g.replay()
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end)


def graph_time(torch, launch, reps, warmup, calls_per_rep, stream):
    """us per call of `launch()` (which queues `calls_per_rep` calls on
    `stream`) replayed `reps` times from one graph."""
    g = capture(torch, launch, stream)
    ms = replay_timed(torch, stream, [g] * warmup, [g] * reps)
    return ms * 1000.0 / (reps * calls_per_rep)


def rotating_time(torch, stream, launch_set, n_sets, calls, rounds=3):
    """us per call of a rotation over `n_sets` input sets: graphs of `calls`
    consecutive calls (set i mod n_sets for call i) that together visit every
    set `calls / gcd` times; replayed once untimed, then `rounds` times."""
    n_graphs = n_sets // math.gcd(n_sets, calls)
    graphs = []
    for gi in range(n_graphs):
        first = gi * calls

        def launch(first=first):
            for i in range(calls):
                launch_set((first + i) % n_sets)
        graphs.append(capture(torch, launch, stream))
    ms = replay_timed(torch, stream, graphs, graphs * rounds)
    return ms * 1000.0 / (rounds * n_graphs * calls), n_graphs


def cold_sets(set_bytes, calls):
    """Sets of `set_bytes` that together hold more than 512 MiB (at least
    three); beyond `calls` sets, a multiple of `calls`, so that whole graphs of
    `calls` calls cover the rotation."""
    n = max(3, -(-COLD_BYTES // set_bytes))
    return n if n <= calls else -(-n // calls) * calls


# ------------------------------------------------------------ the headline
def sweep_cases(torch, arrms, workloads, wl, dev):
    cases = []
    for T in wl.Ts:
        inp = {k: ([x.to(dev) for x in v] if isinstance(v, list) else v.to(dev))
               for k, v in workloads.make_inputs(wl, T).items()}
        plan = arrms.cached_plan(wl.W, T, wl.H, arrms.BF16, arrms.FORCE_ROW)
        cases.append((T, inp, plan, torch.empty_like(inp["residual"]),
                      torch.empty_like(inp["residual"])))
    return cases


def headline(torch, arrms, wl, cases, stream, args):
    """Exactly `warmup` then `steps` steps of the sweep, from graphs captured
    beforehand; returns (elapsed ms of the timed steps, plan)."""
    def step():
        for T, inp, plan, norm, res in cases:
            arrms.ar_rms_run(plan, inp["partials"], inp["residual"], inp["weight"], wl.eps,
                             True, norm, res, stream=stream)

    plan = step_plan(args)
    graphs = {}
    for n in plan["warmup_graphs"] + plan["timed_graphs"]:
        if n not in graphs:
            def launch(n=n):
                for _ in range(n):
                    step()
            graphs[n] = capture(torch, launch, stream)
    ms = replay_timed(torch, stream, [graphs[n] for n in plan["warmup_graphs"]],
                      [graphs[n] for n in plan["timed_graphs"]])
    return ms, plan


def sweep_cold(torch, arrms, wl, cases, dev, stream, spg):
    """The sweep with its inputs and outputs rotated over sets that together
    hold more than 512 MiB (the values of every set are the sweep's own)."""
    shapes, values = [], []
    for T, inp, *_ in cases:
        shapes += [(T, wl.H)] * (wl.W + 3)
        values += inp["partials"] + [inp["residual"]]
        values += [None, None]          # norm_out, residual_out: not filled
    per_set = Pool.size_of(shapes)
    n_sets = cold_sets(per_set, spg)
    pool = Pool(torch, dev, shapes, n_sets, torch.bfloat16)
    for i, v in enumerate(values):
        if v is not None:
            pool.tensor(0, i).copy_(v)
    tensors = pool.sets([])
    sets = []
    for st in tensors:
        one, k = [], 0
        for T, inp, plan, norm, res in cases:
            ps = st[k: k + wl.W]
            one.append((plan, ps, st[k + wl.W], inp["weight"], st[k + wl.W + 1],
                        st[k + wl.W + 2]))
            k += wl.W + 3
        sets.append(one)
    torch.cuda.synchronize()

    def launch_set(s):
        for plan, ps, r, w, n, ro in sets[s]:
            arrms.ar_rms_run(plan, ps, r, w, wl.eps, True, n, ro, stream=stream)
    us_step, n_graphs = rotating_time(torch, stream, launch_set, n_sets, spg)
    del sets, pool
    torch.cuda.empty_cache()
    return {"us_per_call": round(us_step / len(cases), 4), "sets": n_sets,
            "bytes_rotated": per_set * n_sets, "graphs": n_graphs}


def sweep_chain(torch, arrms, workloads, wl, cases, dev, stream, spg, reps=50):
    """The sweep as a dependent chain: one residual buffer [80, H]; the call
    for T reads its first T rows and writes residual_out over them in place,
    so every call reads what the call before it wrote (row 0 at least)."""
    Tmax = max(wl.Ts)
    buf = workloads.make_inputs(wl, Tmax, device=dev, seed=7)["residual"]

    def launch():
        for _ in range(spg):
            for T, inp, plan, norm, res in cases:
                view = buf[:T]
                arrms.ar_rms_run(plan, inp["partials"], view, inp["weight"], wl.eps, True, norm,
                                 view, stream=stream)
    us = graph_time(torch, launch, reps, 5, spg * len(cases), stream)
    return round(us, 4)


def unfused_sweep(torch, cases, wl, spg, stream):
    """us per call of the decode sweep computed without the library (PyTorch
    ops on the same inputs, graph-replayed like the fused calls), and whether
    its norm_out agrees with the fused kernel's within bf16 noise."""
    F = torch.nn.functional
    ucases = []
    for T, inp, plan, norm, res in cases:
        w1 = (inp["weight"].float() + 1.0).to(torch.bfloat16)
        ucases.append((inp, w1, torch.empty_like(norm), torch.empty_like(norm), [None]))

    def steps():
        for _ in range(spg):
            for inp, w1, s, y, out in ucases:
                ps = inp["partials"]
                torch.add(ps[0], ps[1], out=s)
                for q in ps[2:]:
                    s.add_(q)
                torch.add(s, inp["residual"], out=y)
                out[0] = F.rms_norm(y, (wl.H,), w1, wl.eps)
    us = graph_time(torch, steps, 20, 2, len(cases) * spg, stream)
    torch.cuda.synchronize()
    agree = all(torch.allclose(out[0].float(), c[3].float(), rtol=0.05, atol=0.05)
                for (_, _, _, _, out), c in zip(ucases, cases))
    return {"us_per_call": round(us, 3), "norm_out_agrees": bool(agree),
            "what": "W-1 chained bf16 adds, residual add, torch rms_norm (Gemma weight 1+w)"}


# ------------------------------------------------------------ other workloads
def rms_case(torch, arrms, workloads, wl, T, dev):
    """Inputs of one reduce+norm workload, drawn on the device (the oracle
    reads host copies of the same bytes), with the plan and output tensors."""
    inp = workloads.make_inputs(wl, T, device=dev)
    plan = arrms.cached_plan(wl.W, T, wl.H, arrms.BF16)
    out = {"norm": torch.empty_like(inp["residual"]), "res": torch.empty_like(inp["residual"])}
    if wl.group:
        out["q"] = torch.empty((T, wl.H), dtype=torch.uint8, device=dev)
        out["sc"] = torch.empty((T, wl.H // wl.group), dtype=torch.float32, device=dev)
    return inp, plan, out


def rms_call(arrms, wl, plan, ps, r, w, out, stream):
    if wl.group:
        arrms.ar_rms_quant_run(plan, ps, r, w, wl.eps, wl.gemma, wl.group, out["norm"],
                               out["q"], out["sc"], out["res"], stream=stream)
    else:
        arrms.ar_rms_run(plan, ps, r, w, wl.eps, wl.gemma, out["norm"], out["res"],
                         stream=stream)


def time_rms(torch, arrms, wl, T, inp, plan, out, dev, stream):
    """us per call, warm (one set, graphs of 100 calls; 2 above 512 MiB) and
    cold (sets rotated through more than 512 MiB; below that size only)."""
    nbytes = rms_bytes(wl.W, T, wl.H, wl.group)
    big = nbytes > COLD_BYTES
    calls = 2 if big else 100

    def warm():
        for _ in range(calls):
            rms_call(arrms, wl, plan, inp["partials"], inp["residual"], inp["weight"], out,
                     stream)
    us = graph_time(torch, warm, 10 if big else 20, 2 if big else 5, calls, stream)
    r = {"us_per_call": round(us, 3), "bytes": nbytes,
         "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1),
         "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
         "kernel": "row" if plan.kernel == 0 else "split"}
    if big:
        r["cold"] = "one set larger than 512 MiB: every call is cold"
        return r
    # cold: partials, residual and every output rotate; the weight is shared
    shapes = [(T, wl.H)] * (wl.W + 3)
    if wl.group:
        shapes += [(T, wl.H // 2), (T, 2 * (wl.H // wl.group))]   # codes, scales
    n_sets = cold_sets(Pool.size_of(shapes), 100)
    pool = Pool(torch, dev, shapes, n_sets, torch.bfloat16)
    sets = []
    for st in pool.sets(inp["partials"] + [inp["residual"]]):
        o = {"norm": st[wl.W + 1], "res": st[wl.W + 2]}
        if wl.group:
            o["q"] = st[wl.W + 3].view(torch.uint8)
            o["sc"] = st[wl.W + 4].view(torch.float32)
        sets.append((st[:wl.W], st[wl.W], o))
    torch.cuda.synchronize()

    def launch_set(s):
        ps, rr, o = sets[s]
        rms_call(arrms, wl, plan, ps, rr, inp["weight"], o, stream)
    cold_us, _ = rotating_time(torch, stream, launch_set, n_sets, 100)
    del sets, pool
    torch.cuda.empty_cache()
    r.update({"cold_us_per_call": round(cold_us, 3),
              "cold_GB_s": round(nbytes / (cold_us * 1e-6) / 1e9, 1),
              "cold_frac_of_peak": round(nbytes / (cold_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
              "cold_sets": n_sets})
    return r


def time_qk(torch, arrms, workloads, wl, T, dev, stream):
    inp = workloads.make_qk_inputs(wl, T, device=dev)
    plan = arrms.cached_plan(wl.W, T, wl.H, arrms.BF16)
    qo = torch.empty((wl.W, T, wl.q_size), dtype=torch.bfloat16, device=dev)
    ko = torch.empty((wl.W, T, wl.kv_size), dtype=torch.bfloat16, device=dev)

    def call():
        for _ in range(100):
            arrms.ar_qknorm_run(plan, inp["shards"], wl.q_size, wl.kv_size, inp["q_weight"],
                                inp["k_weight"], wl.eps, qo, ko, stream=stream)
    us = graph_time(torch, call, 20, 5, 100, stream)
    nbytes = qk_bytes(wl.W, T, wl.q_size, wl.kv_size)
    r = {"us_per_call": round(us, 3), "bytes": nbytes,
         "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1),
         "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
         "kernel": "qknorm"}
    # cold: shards and outputs rotate through more than 512 MiB
    stride = wl.q_size + 2 * wl.kv_size
    shapes = [(T, stride)] * wl.W + [(wl.W, T, wl.q_size), (wl.W, T, wl.kv_size)]
    n_sets = cold_sets(Pool.size_of(shapes), 100)
    pool = Pool(torch, dev, shapes, n_sets, torch.bfloat16)
    sets = [(st[:wl.W], st[wl.W], st[wl.W + 1]) for st in pool.sets(inp["shards"])]
    torch.cuda.synchronize()

    def launch_set(s):
        sh, q, k = sets[s]
        arrms.ar_qknorm_run(plan, sh, wl.q_size, wl.kv_size, inp["q_weight"], inp["k_weight"],
                            wl.eps, q, k, stream=stream)
    cold_us, _ = rotating_time(torch, stream, launch_set, n_sets, 100)
    del sets, pool
    torch.cuda.empty_cache()
    r.update({"cold_us_per_call": round(cold_us, 3),
              "cold_frac_of_peak": round(nbytes / (cold_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
              "cold_sets": n_sets})
    return inp, (qo, ko), r


# ------------------------------------------------------------ the oracle on the host
def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    return max(1, min(len(os.sched_getaffinity(0)), MAX_THREADS))


def time_oracle(run_rows, T, runs):
    """Wall ms of run_rows(0, T) on one thread, and of the same rows split into
    one contiguous block per host thread run side by side (the oracle is
    unchanged; rows are independent and the ctypes call releases the
    interpreter lock): the median of `runs` runs each."""
    from concurrent.futures import ThreadPoolExecutor
    n = host_threads()
    one = []
    for _ in range(runs):
        t0 = time.perf_counter()
        run_rows(0, T)
        one.append((time.perf_counter() - t0) * 1e3)
    blocks = [(T * i // n, T * (i + 1) // n) for i in range(n)]
    blocks = [b for b in blocks if b[1] > b[0]]
    allc = []
    with ThreadPoolExecutor(n) as pool:
        for _ in range(runs):
            t0 = time.perf_counter()
            list(pool.map(lambda b: run_rows(*b), blocks))
            allc.append((time.perf_counter() - t0) * 1e3)
    return {"oracle_ms_1_thread": round(statistics.median(one), 3),
            "oracle_ms_all_cores": round(statistics.median(allc), 3),
            "threads": n, "runs": runs}


def oracle_rms(wl, host, out, check=True):
    """The oracle on one reduce+norm workload (`host`: the call's inputs,
    copied to the host here), after checking the GPU outputs of the same
    inputs against it (the bench's parity guard)."""
    import oracle
    from oracle import compare
    from tp_all_reduce_amd.workloads import bits

    P = [bits(p) for p in host["partials"]]
    R, w = bits(host["residual"]), bits(host["weight"])
    if check:
        if wl.group:
            _, c_o, s_o, r_o, exact = oracle.ar_rms_quant(P, R, w, wl.eps, wl.gemma, wl.group)
            assert compare.max_code_distance(out["q"].cpu().numpy(), c_o) <= 1
            assert compare.max_scale_relerr(out["sc"].cpu().numpy(), s_o) <= compare.SCALE_TOL
        else:
            _, r_o, exact = oracle.ar_rms(P, R, w, wl.eps, wl.gemma)
        assert compare.bits_equal(bits(out["res"]), r_o), f"{wl.name}: residual_out differs"
        assert compare.max_relerr(bits(out["norm"]), exact, oracle.BF16) <= \
            compare.TOL[oracle.BF16], f"{wl.name}: norm_out beyond tolerance"
        del exact

    def run_rows(lo, hi):
        ps = [p[lo:hi] for p in P]
        if wl.group:
            oracle.ar_rms_quant(ps, R[lo:hi], w, wl.eps, wl.gemma, wl.group, want_exact=False)
        else:
            oracle.ar_rms(ps, R[lo:hi], w, wl.eps, wl.gemma, want_exact=False)
    return run_rows


def oracle_qk(wl, host, outs):
    import oracle
    from oracle import compare
    from tp_all_reduce_amd.workloads import bits

    S = [bits(s) for s in host["shards"]]
    qw, kw = bits(host["q_weight"]), bits(host["k_weight"])
    _, _, qe, ke = oracle.qknorm(S, wl.q_size, wl.kv_size, qw, kw, wl.eps)
    assert compare.max_relerr(bits(outs[0]), qe, oracle.BF16) <= compare.TOL[oracle.BF16]
    assert compare.max_relerr(bits(outs[1]), ke, oracle.BF16) <= compare.TOL[oracle.BF16]

    def run_rows(lo, hi):
        oracle.qknorm([s[lo:hi] for s in S], wl.q_size, wl.kv_size, qw, kw, wl.eps,
                      want_exact=False)
    return run_rows


def oracle_sweep(wl, cases):
    """The oracle over the whole decode sweep (ten calls), after checking the
    GPU outputs of the timed run against it."""
    import oracle
    from oracle import compare
    from tp_all_reduce_amd.workloads import bits

    host = []
    for T, inp, plan, norm, res in cases:
        P = [bits(p) for p in inp["partials"]]
        R, w = bits(inp["residual"]), bits(inp["weight"])
        _, r_o, exact = oracle.ar_rms(P, R, w, wl.eps, True)
        assert compare.bits_equal(bits(res), r_o), f"sweep T={T}: residual_out differs"
        assert compare.max_relerr(bits(norm), exact, oracle.BF16) <= compare.TOL[oracle.BF16]
        host.append((P, R, w))

    def run_sweep(lo, hi):
        # rows [lo, hi) of every call of the sweep (a row range past a call's
        # end is empty for it)
        for P, R, w in host:
            T = R.shape[0]
            a, b = min(lo, T), min(hi, T)
            if b > a:
                oracle.ar_rms([p[a:b] for p in P], R[a:b], w, wl.eps, True, want_exact=False)
    return run_sweep


# ------------------------------------------------------------ main
def main():
    args = parse()
    if args.check_args:
        plan = step_plan(args)
        for k in ("warmup_graphs", "timed_graphs"):   # {steps per graph: graphs}
            plan[k] = {str(n): plan[k].count(n) for n in sorted(set(plan[k]), reverse=True)}
        print(json.dumps(dict(plan, torch_imported="torch" in sys.modules)), flush=True)
        return

    import torch
    from tp_all_reduce_amd import arrms, workloads
    from tp_all_reduce_amd.workloads import WORKLOADS

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    arrms.library()   # fails loudly if the HIP library is not built

    if args.copy_calibration:
        n = 256 * 1024 * 1024
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)
        return

    wl = WORKLOADS["c2"]
    Ts, H, W = wl.Ts, wl.H, wl.W
    spg = args.steps_per_graph
    log(f"[bench] building inputs: c2 W={W} H={H} T={list(Ts)}")
    cases = sweep_cases(torch, arrms, workloads, wl, dev)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()

    log(f"[bench] timing {args.steps} steps after {args.warmup} warm-up steps "
        f"(up to {spg} steps per graph replay)")
    ms_total, plan = headline(torch, arrms, wl, cases, stream, args)
    calls = args.steps * len(Ts)
    us_per_call = ms_total * 1000.0 / calls
    ms_per_step = ms_total / args.steps
    bytes_per_launch = sum(rms_bytes(W, T, H) for T in Ts) / len(Ts)
    achieved = bytes_per_launch / (us_per_call * 1e-6) / 1e9
    log(f"[bench] {us_per_call:.3f} us/call over {calls} calls, {achieved:.1f} GB/s algorithmic")

    traffic = rocprof_us = rocprof_median = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("kernel_source_sha") == kernel_source_sha():
            traffic = rec.get("traffic_bytes_per_launch")
            rocprof_us = rec.get("rocprof_mean_duration_us")
            rocprof_median = rec.get("rocprof_median_duration_us")
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5), "traffic": traffic,
                "kernel": "reduce_norm_kernel<Bf16, W=4, 1 pack/lane, row-resident, residual>",
                "bytes_per_launch": bytes_per_launch, "us_per_launch": round(us_per_call, 4),
                "launches_timed": calls,
                # the committed trace of the same headline: each dispatch alone on an
                # otherwise idle GPU, so µs-scale durations differ from back-to-back calls
                "rocprof_us_per_launch": rocprof_us,
                "rocprof_median_us_per_launch": rocprof_median,
                "rocprof_frac": (round(bytes_per_launch / (rocprof_us * 1e-6) / 1e9
                                       / HBM_PEAK_GBS, 5) if rocprof_us else None)}

    config = {"workload": "c2 decode sweep: W=4 partials [T,4096] bf16, Gemma RMSNorm, eps 1e-6, "
                          "T in {1,2,4,8,16,21,22,32,64,80}, row-resident kernel; one step = 10 "
                          "fused calls, graph-replayed",
              "io_dtype": "bf16", "W": W, "H": H, "T": list(Ts), "calls_per_step": len(Ts),
              "steps_per_graph": spg, "timed_graphs": len(plan["timed_graphs"]),
              # the default dispatch per T (the one-stage window predicate): the
              # sweep forces the row-resident kernel throughout; beyond the
              # window a default plan is a split plan, whose grid of one
              # workgroup per row runs the same row body at these sizes
              "default_plan_kernel": {str(T): ("row" if arrms.cached_plan(W, T, H, arrms.BF16).kernel
                                               == arrms.KERNEL_ROW else "split") for T in Ts}}

    if not args.headline_only:
        log("[bench] the sweep with rotated inputs (cold) and as a dependent chain")
        config["cold"] = sweep_cold(torch, arrms, wl, cases, dev, stream, spg)
        config["dependent_chain_us_per_call"] = sweep_chain(torch, arrms, workloads, wl, cases,
                                                            dev, stream, spg)
        log(f"[bench]   cold {config['cold']}, chain {config['dependent_chain_us_per_call']}")
        per_t = {}
        for case in cases:
            def one(case=case):
                T_, inp_, plan_, norm_, res_ = case
                for _ in range(100):
                    arrms.ar_rms_run(plan_, inp_["partials"], inp_["residual"], inp_["weight"],
                                     wl.eps, True, norm_, res_, stream=stream)
            per_t[str(case[0])] = round(graph_time(torch, one, 20, 2, 100, stream), 3)
        config["per_T_us_per_call"] = per_t
        log(f"[bench]   per-T us/call: {per_t}")
        # the cost of a graph launch on the device, from the sweep in graphs of
        # 10 and of 50 steps (100 and 500 calls): each replay adds it once
        def sweep_steps(n):
            def launch():
                for _ in range(n):
                    for T, inp, pl, norm, res in cases:
                        arrms.ar_rms_run(pl, inp["partials"], inp["residual"], inp["weight"],
                                         wl.eps, True, norm, res, stream=stream)
            return launch
        by_size = {str(10 * n): round(graph_time(torch, sweep_steps(n), reps, 3, 10 * n, stream), 4)
                   for n, reps in ((10, 100), (50, 20))}
        config["us_per_call_by_graph_calls"] = by_size
        config["graph_launch_us"] = round((by_size["100"] - by_size["500"])
                                          / (1 / 100 - 1 / 500), 2)
        log(f"[bench]   per call in graphs of 100 / 500 calls: {by_size}, "
            f"graph launch {config['graph_launch_us']} us")
        # launch floor on this machine: a one-element torch fill kernel replayed the
        # same way (what any single-kernel call costs before it does any work),
        # and torch's add of two [1, H] rows into a third
        tiny = torch.zeros(1, device=dev)
        a_row = torch.randn(1, H, device=dev).to(torch.bfloat16)
        b_row, c_row = torch.randn_like(a_row), torch.empty_like(a_row)

        def fill():
            for _ in range(100):
                tiny.fill_(1.0)

        def add_row():
            for _ in range(100):
                torch.add(a_row, b_row, out=c_row)
        config["launch_floor_us"] = round(graph_time(torch, fill, 20, 2, 100, stream), 3)
        config["one_row_add_kernel_us"] = round(graph_time(torch, add_row, 20, 2, 100, stream), 3)
        # plain stream launches (no graph): host-bound
        with torch.cuda.stream(stream):
            for _ in range(20):
                for T, inp, pl, norm, res in cases:
                    arrms.ar_rms_run(pl, inp["partials"], inp["residual"], inp["weight"],
                                     wl.eps, True, norm, res, stream=stream)
            stream.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(200):
                for T, inp, pl, norm, res in cases:
                    arrms.ar_rms_run(pl, inp["partials"], inp["residual"], inp["weight"],
                                     wl.eps, True, norm, res, stream=stream)
            e1.record(stream)
            e1.synchronize()
        config["us_per_call_stream_launch"] = round(e0.elapsed_time(e1) * 1000.0 / (200 * len(Ts)), 3)
        log(f"[bench]   floor {config['launch_floor_us']} us, row add "
            f"{config['one_row_add_kernel_us']} us, stream launches "
            f"{config['us_per_call_stream_launch']} us")

    unfused = None
    if not args.no_unfused:
        unfused = unfused_sweep(torch, cases, wl, spg, stream)
        log(f"[bench] unfused PyTorch composition (graph): {unfused}")

    cpu = cpu_all = None
    if not args.no_cpu_baseline:
        run_sweep = oracle_sweep(wl, cases)
        t = time_oracle(run_sweep, max(Ts), 3)
        per_call_1 = t["oracle_ms_1_thread"] * 1e3 / len(Ts)
        per_call_n = t["oracle_ms_all_cores"] * 1e3 / len(Ts)
        cpu = {"value": round(per_call_1, 2), "unit": "µs/call", "cores": 1, "kind": "oracle",
               "cpu": cpu_model(),
               "sample": "the full c2 sweep (10 calls, T=1..80, the timed run's own inputs), "
                         "median of 3 runs on one thread"}
        cpu_all = {"value": round(per_call_n, 2), "unit": "µs/call", "cores": t["threads"],
                   "kind": "oracle", "cpu": cpu_model(),
                   "sample": f"the same sweep, each call's rows split over {t['threads']} "
                             "threads, median of 3 runs"}
        log(f"[bench] cpu oracle: {cpu}; all cores: {cpu_all}")

    others = None
    if not args.no_others or args.only:
        others = other_workloads(torch, arrms, workloads, WORKLOADS, dev, stream, args)

    line = {
        "metric": METRIC, "value": round(us_per_call, 4), "unit": "µs/call", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": config,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_oracle_all_cores": cpu_all,
        "unfused_torch_same_gpu": unfused,
        "per_config": others,
        "host": {"cpu": cpu_model(), "threads_available": len(os.sched_getaffinity(0))},
    }
    print(json.dumps(line), flush=True)


def other_workloads(torch, arrms, workloads, WORKLOADS, dev, stream, args):
    """Every other workload: GPU us per call (warm and cold), bytes, fraction of
    peak, and the oracle's time on the host for the same inputs."""
    todo = [("c1", 8), ("c3", 1024), ("c3", 8192), ("c3", 16384), ("c4", 256), ("c5", 64)]
    if args.only:
        todo = [(n, T) for n, T in todo if n == args.only]
    out = {}
    for name, T in todo:
        wl = WORKLOADS[name]
        key = f"{name}_T{T}"
        log(f"[bench] {key}")
        if name == "c5":
            host, outs, r = time_qk(torch, arrms, workloads, wl, T, dev, stream)
            if not args.no_cpu_baseline:
                r.update(time_oracle(oracle_qk(wl, host, outs), T, 3))
        else:
            inp, plan, o = rms_case(torch, arrms, workloads, wl, T, dev)
            r = time_rms(torch, arrms, wl, T, inp, plan, o, dev, stream)
            if not args.no_cpu_baseline:
                # the outputs of the timed run's own set are checked first
                rms_call(arrms, wl, plan, inp["partials"], inp["residual"], inp["weight"], o,
                         stream)
                torch.cuda.synchronize()
                runs = 1 if T >= 16384 else 3
                r.update(time_oracle(oracle_rms(wl, inp, o), T, runs))
            del inp, o
            torch.cuda.empty_cache()
        out[key] = r
        log(f"[bench]   {r}")
    return out


if __name__ == "__main__":
    main()
