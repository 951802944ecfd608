"""Benchmark of the fused W-way reduce + residual add + RMSNorm (libarrms).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--full PATH] [--copy-calibration]

Workload of the headline line: the decode-window sweep, W=4 partial buffers of
[T, 4096] bf16 with Gemma RMSNorm, eps 1e-6, T in {1, 2, 4, 8, 16, 21, 22, 32,
64, 80}, row-resident kernel.  One step is one pass over the sweep: ten fused
calls, one per T; inputs are resident in HBM before the timed region starts.
Steps are launched from a HIP graph that holds --steps-per-graph of them (as a
captured decode step holds every layer's epilogue); the K timed steps are K /
steps-per-graph replays.  value = microseconds per fused call (step time / 10).
The config also reports the figure with one step per graph.

The roofline object covers the dominant kernel (the row-resident kernel, every
launch of the step): algorithmic bytes per launch, (W + 3) * T * H * 2 + H * 2
(W partials and the residual read, norm_out and residual_out written, the
weight read once) averaged over the sweep, divided by that kernel's average launch duration,
measured with HIP events on the stream the graph is replayed on.  `traffic` is
read from the committed rocprofv3 counter summary when it was taken on the
current kernel source, else null.

cpu_baseline: the oracle, single-threaded, on the same sweep, repeated for
about 10 s on the host.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = ("µs/call at T<=80 and effective HBM GB/s (% of MI355X peak) for W-way "
          "reduce+add-RMSNorm")
KERNEL_SRC = os.path.join(ROOT, "tp_all_reduce_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_row_kernel_c2_sweep.json")


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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--steps-per-graph", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-large-t", action="store_true",
                    help="skip the figures of the other workloads reported beside the headline "
                         "(prefill W=8 [8192, 8192], c1, c3 T=1024, c4, c5)")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip timing the unfused PyTorch composition (profiled runs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--full", default=None,
                    help="also time every workload (c1..c5) and write a JSON report here")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (for counter calibration)")
    ap.add_argument("--only", default=None, choices=["c1", "c2", "c3", "c4", "c5"],
                    help="with --full: time only this workload (profiling runs)")
    return ap.parse_args()


def to_dev(d, dev):
    return {k: ([x.to(dev) for x in v] if isinstance(v, list) else
                (None if v is None else v.to(dev))) for k, v in d.items()}


def graph_time(torch, launch, reps, warmup, calls_per_rep, stream):
    """Captures `launch()` (which queues `calls_per_rep` library calls on
    `stream`) in a HIP graph and returns (us per call, total elapsed ms) over
    `reps` replays timed with HIP events on the replaying stream."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        launch()                      # eager warm-up of the same calls
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            launch()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):   # replays and both events on the same stream
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(reps):
            g.replay()
        end.record(stream)
    end.synchronize()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    return ms * 1000.0 / (reps * calls_per_rep), ms


def unfused_sweep(torch, cases, wl, spg, stream):
    """us per call of the decode sweep computed without the library (PyTorch
    ops on the same inputs, graph-replayed like the fused calls), and whether
    its norm_out agrees with the fused kernel's within bf16 noise."""
    F = torch.nn.functional
    ucases = []
    for T, inp, plan, norm, res in cases:
        w1 = (inp["weight"].float() + 1.0).to(torch.bfloat16)
        ucases.append((inp, w1, torch.empty_like(norm), torch.empty_like(norm), [None]))

    def step():
        for inp, w1, s, y, out in ucases:
            ps = inp["partials"]
            torch.add(ps[0], ps[1], out=s)
            for q in ps[2:]:
                s.add_(q)
            torch.add(s, inp["residual"], out=y)
            out[0] = F.rms_norm(y, (wl.H,), w1, wl.eps)

    def steps():
        for _ in range(spg):
            step()
    us, _ = graph_time(torch, steps, 20, 2, len(cases) * spg, stream)
    torch.cuda.synchronize()
    agree = all(torch.allclose(out[0].float(), c[3].float(), rtol=0.05, atol=0.05)
                for (_, _, _, _, out), c in zip(ucases, cases))
    return {"us_per_call": round(us, 3), "norm_out_agrees": bool(agree),
            "what": "W-1 chained bf16 adds, residual add, torch rms_norm (Gemma weight 1+w)"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library is the single-GPU kernel of the "
              "fused all-reduce + RMSNorm epilogue (W partial buffers resident on one device); "
              "multi-GPU runs are not part of it. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

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
    Ts = wl.Ts
    log(f"[bench] building inputs: c2 W={wl.W} H={wl.H} T={list(Ts)}")
    cases = []
    for T in Ts:
        inp = to_dev(workloads.make_inputs(wl, T), dev)
        plan = arrms.cached_plan(wl.W, T, wl.H, arrms.BF16, arrms.FORCE_ROW)
        norm = torch.empty_like(inp["partials"][0])
        res = torch.empty_like(inp["residual"])
        cases.append((T, inp, plan, norm, res))
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()

    def step():
        for T, inp, plan, norm, res in cases:
            arrms.ar_rms_run(plan, inp["partials"], inp["residual"], inp["weight"], wl.eps,
                             True, norm, res, stream=stream)

    spg = max(1, args.steps_per_graph)
    if args.steps % spg or args.warmup % spg:
        sys.exit(f"--steps and --warmup must be multiples of --steps-per-graph ({spg})")

    def steps():
        for _ in range(spg):
            step()

    log(f"[bench] timing {args.steps} steps after {args.warmup} warm-up steps "
        f"({spg} steps per graph replay)")
    us_per_call, ms_total = graph_time(torch, steps, args.steps // spg, args.warmup // spg,
                                       len(Ts) * spg, stream)
    ms_per_step = ms_total / args.steps
    us_one_step_graph, _ = graph_time(torch, step, 500, 20, len(Ts), stream)
    log(f"[bench] one step per graph replay: {us_one_step_graph:.3f} us/call")
    H, W = wl.H, wl.W
    bytes_per_launch = sum(rms_bytes(W, T, H) for T in Ts) / len(Ts)
    achieved = bytes_per_launch / (us_per_call * 1e-6) / 1e9
    log(f"[bench] {us_per_call:.3f} us/call (graph), {achieved:.1f} GB/s algorithmic")

    # per-T detail (same graph method, one T at a time)
    per_t = {}
    for case in cases:
        T, inp, plan, norm, res = case

        def one(case=case):
            T_, inp_, plan_, norm_, res_ = case
            for _ in range(len(Ts) * spg):
                arrms.ar_rms_run(plan_, inp_["partials"], inp_["residual"], inp_["weight"],
                                 wl.eps, True, norm_, res_, stream=stream)
        us, _ = graph_time(torch, one, 20, 2, len(Ts) * spg, stream)
        per_t[str(T)] = round(us, 3)
    log(f"[bench] per-T us/call: {per_t}")

    # launch floor on this machine: a one-element torch fill kernel replayed the
    # same way (what any single-kernel call costs before it does any work)
    tiny = torch.zeros(1, device=dev)

    def fill():
        for _ in range(len(Ts) * spg):
            tiny.fill_(1.0)
    floor_us, _ = graph_time(torch, fill, 20, 2, len(Ts) * spg, stream)
    log(f"[bench] launch floor (1-element fill kernel, graph): {floor_us:.3f} us")

    # a minimal kernel that touches a row: torch's elementwise add of two
    # [1, H] rows into a third, replayed the same way
    a_row = torch.randn(1, wl.H, device=dev).to(torch.bfloat16)
    b_row = torch.randn(1, wl.H, device=dev).to(torch.bfloat16)
    c_row = torch.empty_like(a_row)

    def add_row():
        for _ in range(len(Ts) * spg):
            torch.add(a_row, b_row, out=c_row)
    add_us, _ = graph_time(torch, add_row, 20, 2, len(Ts) * spg, stream)
    log(f"[bench] one-row add kernel (graph): {add_us:.3f} us")

    # the unfused composition on the same GPU, by PyTorch ops alone: the W-way
    # sum in bf16 by chained adds (what a separate all-reduce hands over), then
    # the residual add (residual_out) and torch's rms_norm with the Gemma
    # weight 1 + w (formed before the timed region); replayed the same way
    unfused = None
    if not args.no_unfused:
        unfused = unfused_sweep(torch, cases, wl, spg, stream)
        log(f"[bench] unfused PyTorch composition (graph): {unfused}")

    # plain stream launches (no graph): host-bound, one ctypes call and one
    # hipLaunchKernel per fused call
    with torch.cuda.stream(stream):
        for _ in range(20):
            step()
        stream.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(200):
            step()
        ev1.record(stream)
        ev1.synchronize()
    eager_us = ev0.elapsed_time(ev1) * 1000.0 / (200 * len(Ts))
    log(f"[bench] plain stream launches: {eager_us:.3f} us/call")

    traffic = None
    rocprof_us = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("kernel_source_sha") == kernel_source_sha():
            traffic = rec.get("traffic_bytes_per_launch")
            rocprof_us = rec.get("rocprof_mean_duration_us")

    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5), "traffic": traffic,
                "kernel": "reduce_norm_kernel<Bf16, W=4, 1 pack/lane, no prefetch> (row-resident)",
                "bytes_per_launch": bytes_per_launch, "us_per_launch": round(us_per_call, 4),
                "rocprof_us_per_launch": rocprof_us}

    large_t = None
    if not args.no_large_t:
        c3 = WORKLOADS["c3"]
        log("[bench] prefill W=8 [8192, 8192] (split kernel)")
        large_t = dict(time_rms(torch, arrms, workloads, c3, 8192, dev, stream),
                       workload="W=8 partials [8192, 8192] bf16, eps 1e-5, split kernel")
        log(f"[bench]   {large_t}")

    # the other workloads, one line each (same graph method; bytes algorithmic)
    others = None
    if not args.no_large_t:
        others = {}
        for name, T in (("c1", 8), ("c3", 1024), ("c4", 256), ("c5", 64)):
            wl_o = WORKLOADS[name]
            r = (time_qk if name == "c5" else time_rms)(torch, arrms, workloads, wl_o, T, dev,
                                                         stream)
            others[f"{name}_T{T}"] = {"us_per_call": r["us_per_call"], "GB_s": r["GB_s"],
                                      "frac_of_peak": r["frac_of_peak"], "kernel": r["kernel"]}
        log(f"[bench] other workloads: {others}")

    cpu = None
    cpu_all = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cases, wl, args.cpu_seconds)
        log(f"[bench] cpu oracle: {cpu}")
        cpu_all = cpu_oracle_all_cores(cases, wl, args.cpu_seconds / 2)
        log(f"[bench] cpu oracle, all cores: {cpu_all}")

    secondary = {}
    if args.full:
        secondary = full_report(torch, arrms, workloads, WORKLOADS, dev, stream, args)
        with open(args.full, "w") as f:
            json.dump({"c2_sweep": {"us_per_call": us_per_call, "per_T": per_t},
                       "workloads": secondary}, f, indent=1)

    line = {
        "metric": METRIC, "value": round(us_per_call, 4), "unit": "µs/call", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "c2 decode sweep: W=4 partials [T,4096] bf16, Gemma RMSNorm, "
                               "eps 1e-6, T in {1,2,4,8,16,21,22,32,64,80}, row-resident kernel; "
                               "one step = 10 fused calls, graph-replayed",
                   "io_dtype": "bf16",
                   "W": W, "H": H, "T": list(Ts), "calls_per_step": len(Ts),
                   "per_T_us_per_call": per_t,
                   "launch_floor_us": round(floor_us, 3),
                   "one_row_add_kernel_us": round(add_us, 3),
                   "us_per_call_stream_launch": round(eager_us, 3),
                   "steps_per_graph": spg,
                   "us_per_call_one_step_per_graph": round(us_one_step_graph, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_oracle_all_cores": cpu_all,
        "unfused_torch_same_gpu": unfused,
        "large_t": large_t,
        "other_workloads": others,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(cases, wl, seconds):
    """The oracle as it stands, single-threaded, on the same sweep."""
    import oracle
    from oracle import compare
    from tp_all_reduce_amd.workloads import bits

    host = [([bits(p) for p in inp["partials"]], bits(inp["residual"]), bits(inp["weight"]),
             norm, res) for T, inp, plan, norm, res in cases]
    # the sample's GPU outputs must match the oracle (parity guard of the bench)
    for P, R, w, norm, res in host:
        n_o, r_o, exact = oracle.ar_rms(P, R, w, wl.eps, True)
        assert compare.bits_equal(bits(res), r_o)
        assert compare.max_relerr(bits(norm), exact, oracle.BF16) <= compare.TOL[oracle.BF16]
    reps = 0
    t0 = time.perf_counter()
    while True:
        for P, R, w, _, _ in host:
            oracle.ar_rms(P, R, w, wl.eps, True, want_exact=False)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    us = el * 1e6 / (reps * len(host))
    return {"value": round(us, 2), "unit": "µs/call", "cores": 1, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"the full c2 sweep (10 calls, T=1..80) repeated {reps} times "
                      f"({el:.1f} s, one thread)"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_oracle_all_cores(cases, wl, seconds, max_threads=16):
    """The same oracle on every host core the process may use (at most
    max_threads): each call's rows are split into one contiguous block per
    thread (rows are independent, so the numbers are those of one call), and
    the threads run the unchanged oracle side by side (the ctypes call releases
    the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    from tp_all_reduce_amd.workloads import bits

    n = max(1, min(len(os.sched_getaffinity(0)), max_threads))
    host = [([bits(p) for p in inp["partials"]], bits(inp["residual"]), bits(inp["weight"]))
            for T, inp, plan, norm, res in cases]
    work = [[] for _ in range(n)]
    for P, R, w in host:
        T = R.shape[0]
        for i in range(n):
            lo, hi = T * i // n, T * (i + 1) // n
            if hi > lo:
                work[i].append(([p[lo:hi] for p in P], R[lo:hi], w))

    def run(items):
        for P, R, w in items:
            oracle.ar_rms(P, R, w, wl.eps, True, want_exact=False)

    reps = 0
    with ThreadPoolExecutor(n) as pool:
        list(pool.map(run, work))                     # warm-up round
        t0 = time.perf_counter()
        while True:
            list(pool.map(run, work))
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    us = el * 1e6 / (reps * len(host))
    return {"value": round(us, 2), "unit": "µs/call", "cores": n, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"the full c2 sweep, each call's rows split over {n} threads, "
                      f"repeated {reps} times ({el:.1f} s)"}


def time_rms(torch, arrms, workloads, wl, T, dev, stream):
    """us per call of one reduce+norm (or +FP8) workload, graph-replayed; inputs
    rotate over three sets when they fit in 512 MiB (beyond the 256 MB Infinity
    Cache), else one set."""
    big = rms_bytes(wl.W, T, wl.H) > (1 << 29)
    sets = 1 if big else 3
    inps = [workloads.make_inputs(wl, T, device=dev, seed=workloads.seed_of(wl, T) + 100000 * s)
            for s in range(sets)]
    plan = arrms.cached_plan(wl.W, T, wl.H, arrms.BF16)
    norm = torch.empty_like(inps[0]["partials"][0])
    res = torch.empty_like(norm)
    quant = wl.group > 0
    if quant:
        q = torch.empty(norm.shape, dtype=torch.uint8, device=dev)
        sc = torch.empty((T, wl.H // wl.group), dtype=torch.float32, device=dev)
    n_calls = 2 if big else 100

    def call():
        for i in range(n_calls):
            inp = inps[i % len(inps)]
            if quant:
                arrms.ar_rms_quant_run(plan, inp["partials"], inp["residual"], inp["weight"],
                                       wl.eps, wl.gemma, wl.group, norm, q, sc, res,
                                       stream=stream)
            else:
                arrms.ar_rms_run(plan, inp["partials"], inp["residual"], inp["weight"], wl.eps,
                                 wl.gemma, norm, res, stream=stream)
    us, _ = graph_time(torch, call, 10 if big else 20, 2 if big else 5, n_calls, stream)
    nbytes = rms_bytes(wl.W, T, wl.H, wl.group)
    gbs = nbytes / (us * 1e-6) / 1e9
    out = {"us_per_call": round(us, 3), "bytes": nbytes, "GB_s": round(gbs, 1),
           "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
           "kernel": "row" if plan.kernel == 0 else "split"}
    del inps, call
    torch.cuda.empty_cache()
    return out


def time_qk(torch, arrms, workloads, wl, T, dev, stream):
    inp = to_dev(workloads.make_qk_inputs(wl, T), dev)
    plan = arrms.cached_plan(wl.W, T, wl.H, arrms.BF16)
    qo = torch.empty((wl.W, T, wl.q_size), dtype=torch.bfloat16, device=dev)
    ko = torch.empty((wl.W, T, wl.kv_size), dtype=torch.bfloat16, device=dev)

    def call():
        for _ in range(100):
            arrms.ar_qknorm_run(plan, inp["shards"], wl.q_size, wl.kv_size, inp["q_weight"],
                                inp["k_weight"], wl.eps, qo, ko, stream=stream)
    us, _ = graph_time(torch, call, 20, 5, 100, stream)
    nbytes = 2 * wl.W * T * (wl.q_size + wl.kv_size) * 2 + wl.W * (wl.q_size + wl.kv_size) * 2
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us_per_call": round(us, 3), "bytes": nbytes, "GB_s": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "kernel": "qknorm"}


def full_report(torch, arrms, workloads, WORKLOADS, dev, stream, args):
    """Times every workload with the graph method; bytes are algorithmic."""
    out = {}
    todo = [args.only] if args.only else ["c1", "c3", "c4", "c5"]
    for name in todo:
        wl = WORKLOADS[name]
        for T in wl.Ts:
            key = f"{name}_T{T}"
            log(f"[bench] {key}")
            if name == "c5":
                out[key] = time_qk(torch, arrms, workloads, wl, T, dev, stream)
            else:
                out[key] = time_rms(torch, arrms, workloads, wl, T, dev, stream)
            log(f"[bench]   {out[key]}")
    if not args.only:
        # beyond the pages' eight ranks: 16 partial buffers at the prefill row
        # length (the persistent body without row-ahead loads)
        w16 = workloads.Workload("w16", 9, W=16, H=8192, Ts=(4096,), eps=1e-5)
        log("[bench] w16_T4096")
        out["w16_T4096"] = time_rms(torch, arrms, workloads, w16, 4096, dev, stream)
        log(f"[bench]   {out['w16_T4096']}")
    return out


if __name__ == "__main__":
    main()
