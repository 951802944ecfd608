"""GPU parity of libarrms against the oracle, through the C ABI (via the ctypes
binding), on seeded synthetic inputs.

Small cases compare every output; the full-size workloads compare every row
that the oracle can afford (all of them up to a few million elements, else a
seeded sample of rows, rows being independent).  Acceptance (oracle/compare.py):
residual_out bit-exact; norm_out and q/k outputs within 4e-3 (bf16) / 1e-3
(fp16) relative to the oracle's fp64 value; FP8 codes within one step; FP8
scales within 1e-6."""
import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from tp_all_reduce_amd import arrms, workloads
from tp_all_reduce_amd.workloads import WORKLOADS, bits

pytestmark = pytest.mark.gpu

DEV = "cuda"
FMT = {torch.bfloat16: oracle.BF16, torch.float16: oracle.FP16}


def sample_rows(T, n=192, seed=0):
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    pick = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.unique(np.concatenate([[0, T - 1], pick]))


def host_rows(t, rows):
    idx = torch.as_tensor(rows, device=t.device, dtype=torch.long)
    return bits(t.reshape(-1, t.shape[-1]).index_select(0, idx))


def check_rms(inp, norm_out, residual_out, eps, gemma, rows=None, fmt=oracle.BF16,
              expect_residual=True):
    """Compares the GPU outputs with the oracle on `rows` (default: all)."""
    T = inp["partials"][0].reshape(-1, inp["partials"][0].shape[-1]).shape[0]
    rows = np.arange(T) if rows is None else rows
    P = [host_rows(p, rows) for p in inp["partials"]]
    R = None if inp["residual"] is None else host_rows(inp["residual"], rows)
    n, r, exact = oracle.ar_rms(P, R, bits(inp["weight"]), eps, gemma, fmt)
    err = compare.max_relerr(host_rows(norm_out, rows), exact, fmt)
    assert err <= compare.TOL[fmt], f"norm_out relerr {err}"
    if expect_residual:
        res_gpu = host_rows(residual_out, rows)
        assert compare.bits_equal(res_gpu, r), "residual_out differs from the oracle"
    return err


def run_rms(inp, eps, gemma, flags=0, residual_out="new"):
    return arrms.fused_allreduce_rms_norm(inp["partials"], inp["residual"], inp["weight"], eps,
                                          gemma, residual_out=residual_out, flags=flags)


def to_cuda(inp):
    return {k: ([x.to(DEV) for x in v] if isinstance(v, list) else v.to(DEV))
            for k, v in inp.items()}


def cuda_inputs(wl, T, dtype=torch.bfloat16, device_draw=False, **kw):
    if device_draw:
        return workloads.make_inputs(wl, T, dtype, device=DEV, **kw)
    return to_cuda(workloads.make_inputs(wl, T, dtype, device="cpu", **kw))


# ------------------------------------------------------------ the workloads
def test_c1_decode_w2():
    wl = WORKLOADS["c1"]
    inp = cuda_inputs(wl, 8)
    plan = arrms.cached_plan(wl.W, 8, wl.H, arrms.BF16)
    assert plan.kernel == arrms.KERNEL_ROW
    norm, res = run_rms(inp, wl.eps, wl.gemma)
    torch.cuda.synchronize()
    check_rms(inp, norm, res, wl.eps, wl.gemma)


@pytest.mark.parametrize("flags", [arrms.FORCE_ROW, 0, arrms.FORCE_SPLIT],
                         ids=["row", "default", "split"])
@pytest.mark.parametrize("T", WORKLOADS["c2"].Ts)
def test_c2_gemma_decode_sweep(T, flags):
    wl = WORKLOADS["c2"]
    inp = cuda_inputs(wl, T)
    norm, res = run_rms(inp, wl.eps, True, flags=flags)
    torch.cuda.synchronize()
    check_rms(inp, norm, res, wl.eps, True)


@pytest.mark.parametrize("T", WORKLOADS["c3"].Ts)
def test_c3_prefill_w8(T):
    wl = WORKLOADS["c3"]
    inp = cuda_inputs(wl, T, device_draw=True)
    plan = arrms.cached_plan(wl.W, T, wl.H, arrms.BF16)
    assert plan.kernel == arrms.KERNEL_SPLIT
    norm, res = run_rms(inp, wl.eps, wl.gemma)
    torch.cuda.synchronize()
    rows = np.arange(T) if T <= 1024 else sample_rows(T, 256, seed=T)
    check_rms(inp, norm, res, wl.eps, wl.gemma, rows=rows)


def check_quant(inp, eps, gemma, group, outs, rows=None, fmt=oracle.BF16):
    norm, q, scales, res = outs
    T = inp["partials"][0].shape[0]
    rows = np.arange(T) if rows is None else rows
    P = [host_rows(p, rows) for p in inp["partials"]]
    R = None if inp["residual"] is None else host_rows(inp["residual"], rows)
    n_o, c_o, s_o, r_o, exact = oracle.ar_rms_quant(P, R, bits(inp["weight"]), eps, gemma, group,
                                                    fmt)
    q_gpu = q.view(torch.uint8).reshape(T, -1)[torch.as_tensor(rows, device=q.device)].cpu().numpy()
    s_gpu = scales.reshape(T, -1)[torch.as_tensor(rows, device=q.device)].cpu().numpy()
    assert compare.max_code_distance(q_gpu, c_o) <= 1
    assert compare.max_scale_relerr(s_gpu, s_o) <= compare.SCALE_TOL
    if norm is not None:
        assert compare.max_relerr(host_rows(norm, rows), exact, fmt) <= compare.TOL[fmt]
    if res is not None:
        assert compare.bits_equal(host_rows(res, rows), r_o)
    return float(np.mean(q_gpu != c_o))


def test_c4_fp8_group_quant():
    wl = WORKLOADS["c4"]
    inp = cuda_inputs(wl, 256)
    outs = arrms.fused_allreduce_rms_norm_quant(inp["partials"], inp["residual"], inp["weight"],
                                                wl.eps, wl.group)
    torch.cuda.synchronize()
    mismatch = check_quant(inp, wl.eps, False, wl.group, outs)
    assert mismatch < 0.01      # almost every code identical; the rest one step away


def check_qk(inp, q_size, kv_size, eps, q_out, k_out, fmt=oracle.BF16):
    qo, ko, qe, ke = oracle.qknorm([bits(s) for s in inp["shards"]], q_size, kv_size,
                                   bits(inp["q_weight"]), bits(inp["k_weight"]), eps, fmt)
    eq = compare.max_relerr(bits(q_out), qe, fmt)
    ek = compare.max_relerr(bits(k_out), ke, fmt)
    assert eq <= compare.TOL[fmt] and ek <= compare.TOL[fmt], (eq, ek)


def test_c5_qk_norm():
    wl = WORKLOADS["c5"]
    inp = workloads.make_qk_inputs(wl, 64)
    inp = {k: ([x.to(DEV) for x in v] if isinstance(v, list) else v.to(DEV)) for k, v in inp.items()}
    q_out, k_out = arrms.fused_qk_norm(inp["shards"], inp["q_weight"], inp["k_weight"],
                                       wl.q_size, wl.kv_size, wl.eps)
    torch.cuda.synchronize()
    check_qk(inp, wl.q_size, wl.kv_size, wl.eps, q_out, k_out)


FP16_CASES = ([("c1", 8)] + [("c2", T) for T in WORKLOADS["c2"].Ts]
              + [("c3", T) for T in WORKLOADS["c3"].Ts] + [("c4", 256)])


@pytest.mark.parametrize("name,T", FP16_CASES, ids=[f"{n}_T{T}" for n, T in FP16_CASES])
def test_workloads_fp16(name, T):
    """Every reduce+norm workload again with fp16 activations and weight."""
    wl = WORKLOADS[name]
    inp = cuda_inputs(wl, T, torch.float16, device_draw=name == "c3")
    rows = np.arange(T) if T <= 1024 else sample_rows(T, 256, seed=T)
    if wl.group:
        outs = arrms.fused_allreduce_rms_norm_quant(inp["partials"], inp["residual"],
                                                    inp["weight"], wl.eps, wl.group, wl.gemma)
        torch.cuda.synchronize()
        assert check_quant(inp, wl.eps, wl.gemma, wl.group, outs, fmt=oracle.FP16) < 0.01
    else:
        flags = arrms.FORCE_ROW if name == "c2" else 0
        norm, res = run_rms(inp, wl.eps, wl.gemma, flags=flags)
        torch.cuda.synchronize()
        check_rms(inp, norm, res, wl.eps, wl.gemma, rows=rows, fmt=oracle.FP16)


def test_c5_qk_norm_fp16():
    wl = WORKLOADS["c5"]
    inp = to_cuda(workloads.make_qk_inputs(wl, 64, torch.float16))
    q_out, k_out = arrms.fused_qk_norm(inp["shards"], inp["q_weight"], inp["k_weight"],
                                       wl.q_size, wl.kv_size, wl.eps)
    torch.cuda.synchronize()
    check_qk(inp, wl.q_size, wl.kv_size, wl.eps, q_out, k_out, fmt=oracle.FP16)


# ------------------------------------------------- shapes: tiles and tails
GENERIC = workloads.Workload("generic", 9, W=1, H=8, Ts=(1,), eps=1e-6)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("W,T,H", [(1, 1, 8), (3, 5, 72), (2, 37, 1000), (8, 3, 8192),
                                   (5, 17, 2056), (7, 9, 4104), (4, 70, 16384), (2, 300, 1024),
                                   (6, 129, 3000)])
@pytest.mark.parametrize("flags", [0, arrms.FORCE_SPLIT], ids=["default", "split"])
def test_generic_shapes(W, T, H, dtype, flags):
    inp = cuda_inputs(GENERIC, T, dtype, W=W, H=H, seed=W * 7919 + T * 31 + H)
    norm, res = run_rms(inp, 1e-5, False, flags=flags)
    torch.cuda.synchronize()
    check_rms(inp, norm, res, 1e-5, False, fmt=FMT[dtype])


@pytest.mark.parametrize("W,T,H", [(2, 80, 8192), (1, 1, 8), (8, 13, 1096), (4, 31, 4096)])
def test_row_kernel_shapes(W, T, H):
    inp = cuda_inputs(GENERIC, T, W=W, H=H, seed=W + T + H)
    norm, res = run_rms(inp, 1e-6, True, flags=arrms.FORCE_ROW)
    torch.cuda.synchronize()
    check_rms(inp, norm, res, 1e-6, True)


@pytest.mark.parametrize("group", [8, 32, 64, 128, 256, 512])
@pytest.mark.parametrize("flags", [arrms.FORCE_ROW, arrms.FORCE_SPLIT], ids=["row", "split"])
def test_quant_group_sizes(group, flags):
    W, T, H = 3, 11, 4096
    inp = cuda_inputs(WORKLOADS["c4"], T, W=W, H=H, seed=group)
    outs = arrms.fused_allreduce_rms_norm_quant(inp["partials"], inp["residual"], inp["weight"],
                                                1e-6, group, flags=flags)
    torch.cuda.synchronize()
    check_quant(inp, 1e-6, False, group, outs)


def test_quant_fp16_gemma_codes_only():
    W, T, H = 2, 40, 2048
    inp = cuda_inputs(WORKLOADS["c4"], T, torch.float16, W=W, H=H, seed=5)
    outs = arrms.fused_allreduce_rms_norm_quant(inp["partials"], inp["residual"], inp["weight"],
                                                1e-6, 128, gemma=True, with_norm=False)
    torch.cuda.synchronize()
    assert outs[0] is None
    check_quant(inp, 1e-6, True, 128, outs, fmt=oracle.FP16)


# the last two shapes do not fit every shard on whole wavefronts in 1024 lanes
# and take the packed lane layout
@pytest.mark.parametrize("W,T,q,kv", [(1, 3, 256, 256), (2, 17, 512, 256), (8, 5, 1024, 256),
                                      (4, 130, 1536, 256), (3, 7, 2048, 512), (5, 9, 1024, 768),
                                      (8, 4, 2048, 512), (3, 9, 8192, 2304), (7, 6, 4096, 512)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
def test_qk_shapes(W, T, q, kv, dtype):
    inp = workloads.make_qk_inputs(WORKLOADS["c5"], T, dtype, W=W, q_size=q, kv_size=kv,
                                   seed=W * 13 + T)
    inp = {k: ([x.to(DEV) for x in v] if isinstance(v, list) else v.to(DEV)) for k, v in inp.items()}
    q_out, k_out = arrms.fused_qk_norm(inp["shards"], inp["q_weight"], inp["k_weight"], q, kv,
                                       1e-6)
    torch.cuda.synchronize()
    check_qk(inp, q, kv, 1e-6, q_out, k_out, FMT[dtype])


# ------------------------------------------------------------- edge cases
def test_zero_tokens_touch_nothing():
    x = torch.empty(0, 1024, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(1024, dtype=torch.bfloat16, device=DEV)
    norm, res = arrms.fused_allreduce_rms_norm([x, x], x, w, 1e-6)
    torch.cuda.synchronize()
    assert norm.shape == (0, 1024) and res.shape == (0, 1024)


def test_three_d_input_tokens_are_numel_over_h():
    wl = WORKLOADS["c2"]
    inp = cuda_inputs(wl, 82)
    inp3 = {"partials": [p.reshape(2, 41, wl.H) for p in inp["partials"]],
            "residual": inp["residual"].reshape(2, 41, wl.H), "weight": inp["weight"]}
    norm, res = run_rms(inp3, wl.eps, True)
    torch.cuda.synchronize()
    assert norm.shape == (2, 41, wl.H)
    # 82 tokens: outside the one-stage window, so the split kernel ran
    assert arrms.cached_plan(wl.W, 82, wl.H, arrms.BF16).kernel == arrms.KERNEL_SPLIT
    check_rms(inp, norm.reshape(82, -1), res.reshape(82, -1), wl.eps, True)


@pytest.mark.parametrize("flags", [arrms.FORCE_ROW, arrms.FORCE_SPLIT], ids=["row", "split"])
def test_no_residual_and_dead_residual(flags):
    wl = WORKLOADS["c2"]
    inp = cuda_inputs(wl, 16)
    # no residual term: residual_out (if requested) is the reduced sum itself
    no_res = dict(inp, residual=None)
    norm, red = run_rms(no_res, wl.eps, True, flags=flags)
    torch.cuda.synchronize()
    check_rms(no_res, norm, red, wl.eps, True)
    # dead residual output: only norm_out is written
    norm2, none = run_rms(inp, wl.eps, True, flags=flags, residual_out=None)
    torch.cuda.synchronize()
    assert none is None
    check_rms(inp, norm2, None, wl.eps, True, expect_residual=False)


@pytest.mark.parametrize("flags", [arrms.FORCE_ROW, arrms.FORCE_SPLIT], ids=["row", "split"])
def test_residual_in_place(flags):
    wl = WORKLOADS["c2"]
    inp = cuda_inputs(wl, 21)
    ref_inp = dict(inp, residual=inp["residual"].clone())
    norm, res = run_rms(inp, wl.eps, True, flags=flags, residual_out=inp["residual"])
    torch.cuda.synchronize()
    assert res.data_ptr() == inp["residual"].data_ptr()
    check_rms(ref_inp, norm, res, wl.eps, True)


def test_rounding_ties_and_subnormals_bit_exact():
    # fp32 sums landing exactly halfway between 16-bit neighbours, and sums in
    # the subnormal range, decided by the oracle's nearest-even rounding
    H, T = 1024, 4
    for dtype, mant in ((torch.bfloat16, 7), (torch.float16, 10)):
        rng = np.random.default_rng(7)
        e = rng.integers(-12, 12, (T, H)).astype(np.float64)
        if dtype == torch.float16:
            e = np.clip(e, -12, 12)
        m = rng.integers(1 << mant, 1 << (mant + 1), (T, H)).astype(np.float64)
        a = m * np.exp2(e - mant)                         # exactly representable
        half_ulp = np.exp2(e - mant - 1) * np.where(rng.random((T, H)) < 0.5, 1, -1)
        tiny = np.exp2(-130.0 if dtype == torch.bfloat16 else -20.0)
        a[0, :64] = tiny * (1 + np.arange(64) % 4)
        half_ulp[0, :64] = tiny / 2
        P0 = torch.tensor(a, dtype=torch.float64).to(dtype)
        P1 = torch.tensor(half_ulp, dtype=torch.float64).to(dtype)
        assert torch.equal(P0.double(), torch.tensor(a)) and torch.equal(P1.double(),
                                                                       torch.tensor(half_ulp))
        R = torch.zeros(T, H, dtype=dtype)
        w = torch.ones(H, dtype=dtype)
        inp = {"partials": [P0.to(DEV), P1.to(DEV)], "residual": R.to(DEV), "weight": w.to(DEV)}
        for flags in (arrms.FORCE_ROW, arrms.FORCE_SPLIT):
            norm, res = run_rms(inp, 1e-6, False, flags=flags)
            torch.cuda.synchronize()
            check_rms(inp, norm, res, 1e-6, False, fmt=FMT[dtype])


@pytest.mark.parametrize("dtype,big", [(torch.bfloat16, 1e15), (torch.float16, 1e3)],
                         ids=["bf16", "fp16"])
@pytest.mark.parametrize("flags", [arrms.FORCE_ROW, arrms.FORCE_SPLIT], ids=["row", "split"])
def test_special_values(dtype, big, flags):
    # eps = 0 on non-zero rows; an all-zero row with eps > 0; an inf in a row
    # (that row's residual_out keeps the inf, its norm is NaN at the inf and 0
    # elsewhere, exactly as the oracle's definition gives); large finite values
    # (scaled to stay finite in the format)
    W, T, H = 2, 6, 512
    inp = cuda_inputs(GENERIC, T, dtype, W=W, H=H, seed=99)
    inp["partials"][0][1].zero_()
    inp["partials"][1][1].zero_()
    inp["residual"][1].zero_()
    inp["partials"][0][2, 7] = float("inf")
    inp["partials"][1][3] *= big
    assert bool(torch.isfinite(inp["partials"][1][3]).all())
    for eps in (0.0, 1e-6):
        if eps == 0.0:
            sel = [0, 2, 3, 4, 5]      # the zero row has 0/0 with eps = 0
        else:
            sel = list(range(T))
        norm, res = run_rms(inp, eps, False, flags=flags)
        torch.cuda.synchronize()
        check_rms(inp, norm, res, eps, False, rows=np.array(sel), fmt=FMT[dtype])


@pytest.mark.parametrize("flags", [arrms.FORCE_ROW, arrms.FORCE_SPLIT], ids=["row", "split"])
def test_quant_special_values(flags):
    """FP8 epilogue on non-finite rows: a NaN weight element gives a NaN code in
    every row while the other groups keep their scales; a row with an inf (norm
    NaN there, 0 elsewhere), a row with a NaN input (norm NaN everywhere) and a
    zero row all get scale 0 and code 0, as the oracle's NaN-free amax gives."""
    W, T, H = 2, 6, 1024
    inp = cuda_inputs(GENERIC, T, W=W, H=H, seed=321)
    inp["weight"][5] = float("nan")
    inp["partials"][0][1, 7] = float("inf")
    inp["partials"][0][2, 9] = float("nan")
    for x in (inp["partials"][0], inp["partials"][1], inp["residual"]):
        x[3].zero_()
    outs = arrms.fused_allreduce_rms_norm_quant(inp["partials"], inp["residual"], inp["weight"],
                                                1e-6, 128, flags=flags)
    torch.cuda.synchronize()
    check_quant(inp, 1e-6, False, 128, outs)
    q = outs[1].view(torch.uint8).cpu().numpy()
    scales = outs[2].cpu().numpy()
    assert (q[[0, 4, 5], 5] & 0x7F == 0x7F).all()      # NaN codes
    assert (scales[[1, 2, 3]] == 0).all() and (q[[1, 2, 3]] == 0).all()
    assert (scales[[0, 4, 5]] > 0).all()


def test_deterministic_and_row_split_agree():
    wl = WORKLOADS["c2"]
    inp = cuda_inputs(wl, 64)
    a = run_rms(inp, wl.eps, True, flags=arrms.FORCE_ROW)
    b = run_rms(inp, wl.eps, True, flags=arrms.FORCE_ROW)
    s1 = run_rms(inp, wl.eps, True, flags=arrms.FORCE_SPLIT)
    s2 = run_rms(inp, wl.eps, True, flags=arrms.FORCE_SPLIT)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(s1[0].view(torch.int16), s2[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int16), s1[1].view(torch.int16))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("gemma", [False, True], ids=["standard", "gemma"])
def test_kernel_bodies_agree_bit_for_bit(gemma, dtype):
    """With one pack per lane every body adds and reduces in the same order, so
    a row's outputs do not depend on which body ran it: the row-ahead loop
    (5000 rows), the lean body (1500), the lean body of few rows per workgroup
    (700), the row body behind a split plan (200) and the row-resident plan
    (64) give the same bits for the rows they share, whatever their store
    policies.  Same for the FP8 epilogue: the row-ahead loop (2048 rows)
    against the row body (256)."""
    inp = cuda_inputs(GENERIC, 5000, dtype, W=8, H=8192, seed=4242, device_draw=True)
    full = run_rms(inp, 1e-5, gemma)
    outs = {}
    for n, flags in ((1500, 0), (700, 0), (200, 0), (64, arrms.FORCE_ROW)):
        part = {"partials": [p[:n] for p in inp["partials"]], "residual": inp["residual"][:n],
                "weight": inp["weight"]}
        outs[n] = run_rms(part, 1e-5, gemma, flags=flags)
    torch.cuda.synchronize()
    for n, (norm, res) in outs.items():
        assert torch.equal(norm.view(torch.int16), full[0][:n].view(torch.int16)), n
        assert torch.equal(res.view(torch.int16), full[1][:n].view(torch.int16)), n
    del inp, full, outs

    qinp = cuda_inputs(WORKLOADS["c4"], 2048, dtype, seed=4343, device_draw=True)
    qfull = arrms.fused_allreduce_rms_norm_quant(qinp["partials"], qinp["residual"],
                                                 qinp["weight"], 1e-6, 128, gemma=gemma)
    n = 256
    qpart = arrms.fused_allreduce_rms_norm_quant([p[:n] for p in qinp["partials"]],
                                                 qinp["residual"][:n], qinp["weight"], 1e-6,
                                                 128, gemma=gemma)
    torch.cuda.synchronize()
    code = arrms.BF16 if dtype == torch.bfloat16 else arrms.FP16
    assert arrms.cached_plan(4, 2048, 7168, code).kernel == arrms.KERNEL_SPLIT
    for a, b in zip(qpart, qfull):
        if a.dtype == torch.float8_e4m3fn:
            a, b = a.view(torch.uint8), b.view(torch.uint8)
        elif a.dtype == torch.float32:
            a, b = a.view(torch.int32), b.view(torch.int32)
        else:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b[:n])


def test_graph_capture_replays_match_eager():
    wl = WORKLOADS["c2"]
    inp = cuda_inputs(wl, 8)
    eager = run_rms(inp, wl.eps, True)
    qinp = cuda_inputs(WORKLOADS["c4"], 32)
    eager_q = arrms.fused_allreduce_rms_norm_quant(qinp["partials"], qinp["residual"],
                                                   qinp["weight"], 1e-6, 128)
    # a persistent split launch whose workgroups loop over rows, and QK-norm
    linp = cuda_inputs(GENERIC, 3000, W=8, H=4096, seed=5, device_draw=True)
    eager_l = run_rms(linp, 1e-5, False, flags=arrms.FORCE_SPLIT)
    wl5 = WORKLOADS["c5"]
    kinp = to_cuda(workloads.make_qk_inputs(wl5, 64))
    eager_k = arrms.fused_qk_norm(kinp["shards"], kinp["q_weight"], kinp["k_weight"],
                                  wl5.q_size, wl5.kv_size, wl5.eps)
    torch.cuda.synchronize()
    plan = arrms.cached_plan(wl.W, 8, wl.H, arrms.BF16)
    qplan = arrms.cached_plan(4, 32, 7168, arrms.BF16)
    lplan = arrms.cached_plan(8, 3000, 4096, arrms.BF16, arrms.FORCE_SPLIT)
    kplan = arrms.cached_plan(wl5.W, 64, wl5.H, arrms.BF16)
    norm = torch.empty_like(eager[0])
    res = torch.empty_like(eager[1])
    qn, qq, qs, qr = (torch.empty_like(t) for t in eager_q)
    ln, lr = (torch.empty_like(t) for t in eager_l)
    kq, kk = (torch.empty_like(t) for t in eager_k)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            arrms.ar_rms_run(plan, inp["partials"], inp["residual"], inp["weight"], wl.eps, True,
                             norm, res, stream=s)
            arrms.ar_rms_quant_run(qplan, qinp["partials"], qinp["residual"], qinp["weight"],
                                   1e-6, False, 128, qn, qq, qs, qr, stream=s)
            arrms.ar_rms_run(lplan, linp["partials"], linp["residual"], linp["weight"], 1e-5,
                             False, ln, lr, stream=s)
            arrms.ar_qknorm_run(kplan, kinp["shards"], wl5.q_size, wl5.kv_size,
                                kinp["q_weight"], kinp["k_weight"], wl5.eps, kq, kk, stream=s)
    for _ in range(3):
        for t in (norm, ln, kq, kk):
            t.fill_(0)
        qq.view(torch.uint8).fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(norm.view(torch.int16), eager[0].view(torch.int16))
        assert torch.equal(res.view(torch.int16), eager[1].view(torch.int16))
        assert torch.equal(qq.view(torch.uint8), eager_q[1].view(torch.uint8))
        assert torch.equal(qs, eager_q[2])
        assert torch.equal(ln.view(torch.int16), eager_l[0].view(torch.int16))
        assert torch.equal(lr.view(torch.int16), eager_l[1].view(torch.int16))
        assert torch.equal(kq.view(torch.int16), eager_k[0].view(torch.int16))
        assert torch.equal(kk.view(torch.int16), eager_k[1].view(torch.int16))
        _ = (inp["partials"][0].float() * 2).sum().item()   # eager work between replays


def test_errors_leave_outputs_untouched():
    x = torch.randn(8, 1024, device=DEV).to(torch.bfloat16)
    w = torch.ones(1024, dtype=torch.bfloat16, device=DEV)
    norm = torch.full_like(x, 7.0)
    res = torch.full_like(x, 7.0)
    plan = arrms.ar_rms_plan(2, 8, 1024)
    buf = torch.empty(8 * 1024 + 8, dtype=torch.bfloat16, device=DEV)
    misaligned = buf[1:1 + 8 * 1024].view(8, 1024)
    with pytest.raises(arrms.ArrmsError) as e:
        arrms.ar_rms_run(plan, [x, misaligned], x, w, 1e-6, False, norm, res)
    assert e.value.code == arrms.EINVAL
    with pytest.raises(arrms.ArrmsError) as e:
        arrms.ar_rms_run(plan, [x, x], x, w, float("nan"), False, norm, res)
    assert e.value.code == arrms.EINVAL
    with pytest.raises(ValueError):
        arrms.ar_rms_run(plan, [x, x[:4]], x, w, 1e-6, False, norm, res)
    # quant: unsupported group size, misaligned scales
    q = torch.full((8, 1024), 7, dtype=torch.uint8, device=DEV)
    sc = torch.full((8, 8), 7.0, device=DEV)
    with pytest.raises(arrms.ArrmsError) as e:
        arrms.ar_rms_quant_run(plan, [x, x], x, w, 1e-6, False, 96, norm, q, sc, res)
    assert e.value.code == arrms.ENOTSUP
    qbuf = torch.full((8 * 1024 + 1,), 7, dtype=torch.uint8, device=DEV)
    with pytest.raises(arrms.ArrmsError) as e:     # codes need 8-byte alignment
        arrms.ar_rms_quant_run(plan, [x, x], x, w, 1e-6, False, 128, norm, qbuf[1:], sc, res)
    assert e.value.code == arrms.EINVAL
    # QK: k size not a multiple of 256, negative eps
    qkv = torch.randn(8, 2048, device=DEV).to(torch.bfloat16)
    qplan = arrms.ar_rms_plan(2, 8, 2048)
    qw = torch.ones(2 * 1536, dtype=torch.bfloat16, device=DEV)
    kw = torch.ones(2 * 256, dtype=torch.bfloat16, device=DEV)
    qo = torch.full((2, 8, 1536), 7.0, dtype=torch.bfloat16, device=DEV)
    ko = torch.full((2, 8, 256), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(arrms.ArrmsError) as e:     # raw addresses: the library decides
        arrms.ar_qknorm_run(qplan, [qkv, qkv], 1792, 128, qw.data_ptr(), kw.data_ptr(), 1e-6,
                            qo.data_ptr(), ko.data_ptr())
    assert e.value.code == arrms.ENOTSUP
    with pytest.raises(arrms.ArrmsError) as e:
        arrms.ar_qknorm_run(qplan, [qkv, qkv], 1536, 256, qw, kw, -1.0, qo, ko)
    assert e.value.code == arrms.EINVAL
    torch.cuda.synchronize()
    assert bool((norm == 7.0).all()) and bool((res == 7.0).all())
    assert bool((q == 7).all()) and bool((sc == 7.0).all()) and bool((qbuf == 7).all())
    assert bool((qo == 7.0).all()) and bool((ko == 7.0).all())


# ------------------------------------- persistent loops (more rows than workgroups)
@pytest.mark.parametrize("W,T,H,quant", [(3, 20000, 1000, False), (2, 9000, 2048, True),
                                         (5, 700, 16384, False), (8, 600, 12288, True)])
def test_split_loops_over_rows(W, T, H, quant):
    """T beyond what the device holds at once, so workgroups loop over rows
    (with the next row prefetched; four packs per lane above 8192)."""
    inp = cuda_inputs(GENERIC, T, W=W, H=H, seed=T + H, device_draw=True)
    rows = sample_rows(T, 160, seed=W)
    if quant:
        outs = arrms.fused_allreduce_rms_norm_quant(inp["partials"], inp["residual"],
                                                    inp["weight"], 1e-6, 128,
                                                    flags=arrms.FORCE_SPLIT)
        torch.cuda.synchronize()
        check_quant(inp, 1e-6, False, 128, outs, rows=rows)
    else:
        norm, res = run_rms(inp, 1e-6, False, flags=arrms.FORCE_SPLIT)
        torch.cuda.synchronize()
        check_rms(inp, norm, res, 1e-6, False, rows=rows)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("W,T,H", [(9, 1, 8), (11, 5, 72), (12, 37, 1000), (16, 300, 8192),
                                   (16, 3000, 4096), (13, 2000, 1096)])
def test_more_than_eight_partials(W, T, H, dtype):
    """W = 9..16: the persistent body without prefetch; T = 2000 and 3000 loop."""
    inp = cuda_inputs(GENERIC, T, dtype, W=W, H=H, seed=W * 131 + T + H, device_draw=T > 1000)
    norm, res = run_rms(inp, 1e-5, False)
    torch.cuda.synchronize()
    rows = np.arange(T) if T <= 300 else sample_rows(T, 160, seed=W)
    check_rms(inp, norm, res, 1e-5, False, rows=rows, fmt=FMT[dtype])


@pytest.mark.parametrize("variant", ["quant", "quant_gemma_no_norm", "round", "no_residual",
                                     "dead_residual"])
def test_more_than_eight_partials_variants(variant):
    W, T, H = 16, 100, 7168
    inp = cuda_inputs(GENERIC, T, W=W, H=H, seed=len(variant))
    if variant.startswith("quant"):
        gemma = "gemma" in variant
        outs = arrms.fused_allreduce_rms_norm_quant(inp["partials"], inp["residual"],
                                                    inp["weight"], 1e-6, 128, gemma,
                                                    with_norm="no_norm" not in variant)
        torch.cuda.synchronize()
        assert check_quant(inp, 1e-6, gemma, 128, outs) < 0.01
    elif variant == "round":
        norm, res = arrms.fused_allreduce_rms_norm(inp["partials"], inp["residual"],
                                                   inp["weight"], 1e-6, round_reduced=True)
        torch.cuda.synchronize()
        P = [bits(p) for p in inp["partials"]]
        _, r, exact = oracle.ar_rms(P, bits(inp["residual"]), bits(inp["weight"]), 1e-6, False,
                                    round_reduced=True)
        assert compare.bits_equal(bits(res), r)
        assert compare.max_relerr(bits(norm), exact, oracle.BF16) <= compare.TOL[oracle.BF16]
    elif variant == "no_residual":
        inp["residual"] = None
        norm, res = run_rms(inp, 1e-6, False)
        torch.cuda.synchronize()
        check_rms(inp, norm, res, 1e-6, False)
    else:
        norm, res = run_rms(inp, 1e-6, False, residual_out=None)
        torch.cuda.synchronize()
        assert res is None
        check_rms(inp, norm, None, 1e-6, False, expect_residual=False)


@pytest.mark.parametrize("W,T,q,kv", [(2, 70000, 256, 256), (8, 66000, 2048, 512),
                                      (3, 66000, 8192, 2304)],
                         ids=["shard_aligned", "shard_aligned_4_per_lane", "packed"])
def test_qk_more_tokens_than_workgroups(W, T, q, kv):
    """Beyond 65536 tokens the QK workgroups loop over tokens, in both lane
    layouts (the second shape does not fit shards on whole wavefronts)."""
    inp = workloads.make_qk_inputs(WORKLOADS["c5"], T, W=W, q_size=q, kv_size=kv, seed=3,
                                   device=DEV)
    q_out, k_out = arrms.fused_qk_norm(inp["shards"], inp["q_weight"], inp["k_weight"], q, kv,
                                       1e-6)
    torch.cuda.synchronize()
    rows = sample_rows(T, 128, seed=5)
    idx = torch.as_tensor(rows, device=DEV)
    sub = {"shards": [s.index_select(0, idx) for s in inp["shards"]],
           "q_weight": inp["q_weight"], "k_weight": inp["k_weight"]}
    check_qk(sub, q, kv, 1e-6, q_out.index_select(1, idx).contiguous(),
             k_out.index_select(1, idx).contiguous())


@pytest.mark.parametrize("flags", [arrms.FORCE_ROW, arrms.FORCE_SPLIT], ids=["row", "split"])
def test_quant_tiny_and_zero_scales(flags):
    """Groups whose scale is subnormal (amax/448 below 2^-126, reciprocal beyond
    fp32), a group of zero weights (scale 0, codes 0), groups just above the
    kernel's 2^-116 guard for the division-free scale and far up the range, and
    ordinary groups."""
    W, T, H, G = 2, 9, 1024, 128
    inp = cuda_inputs(WORKLOADS["c4"], T, W=W, H=H, seed=11)
    w = inp["weight"].float()
    w[:G] = w[:G] * 1e-37          # tiny: normalised values ~1e-37
    w[G:2 * G] = 0.0               # zero group
    w[2 * G:3 * G] = w[2 * G:3 * G] * 3e-36
    w[3 * G:4 * G] = w[3 * G:4 * G] * 2.0 ** -114   # amax a few times 2^-114
    w[5 * G:6 * G] = w[5 * G:6 * G] * 1e36          # amax ~1e36
    inp["weight"] = w.to(torch.bfloat16)
    outs = arrms.fused_allreduce_rms_norm_quant(inp["partials"], inp["residual"], inp["weight"],
                                                1e-6, G, flags=flags)
    torch.cuda.synchronize()
    check_quant(inp, 1e-6, False, G, outs)
    scales = outs[2].cpu().numpy()
    assert np.all(scales[:, 1] == 0) and np.all(scales[:, 0] < 2.0 ** -126)
    assert np.all(outs[1].view(torch.uint8).cpu().numpy()[:, G:2 * G] == 0)
    # the division-free scale at both ends of its range
    assert np.all(scales[:, 3] >= 2.0 ** -116 / 448) and np.all(scales[:, 3] < 2.0 ** -116)
    assert np.all(scales[:, 5] > 1e32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("W", [4, 6, 8])
@pytest.mark.parametrize("form", ["residual", "gemma", "no_residual", "dead_residual",
                                  "round_reduced"])
def test_split_band_of_few_rows_per_workgroup(W, form, dtype):
    """Split plans of 512 to 8 x (resident workgroups) rows, where four to eight
    partials without the FP8 epilogue may run on twice the workgroups per CU
    without the row-ahead loads: every form of the call at rows of 8192 (one
    workgroup per CU otherwise) and 4096 elements, with at most two rows per
    workgroup (the body with the few-rows store policy: T = 700 and 1024 at 8192
    elements, 1100 at 4096) and with more (T = 1500 at 8192, 2500 at 4096)."""
    fmt = FMT[dtype]
    for H, T in ((8192, 700), (8192, 1024), (8192, 1500), (4096, 1100), (4096, 2500)):
        inp = cuda_inputs(WORKLOADS["c3"], T, dtype, W=W, H=H, seed=W * 100 + T,
                          device_draw=True)
        gemma = form == "gemma"
        if form == "no_residual":
            inp["residual"] = None
        norm, res = arrms.fused_allreduce_rms_norm(
            inp["partials"], inp["residual"], inp["weight"], 1e-5, gemma,
            residual_out=None if form == "dead_residual" else "new",
            round_reduced=form == "round_reduced")
        torch.cuda.synchronize()
        rows = sample_rows(T, 160, seed=T)
        P = [host_rows(p, rows) for p in inp["partials"]]
        R = None if inp["residual"] is None else host_rows(inp["residual"], rows)
        n, r, exact = oracle.ar_rms(P, R, bits(inp["weight"]), 1e-5, gemma, fmt,
                                    round_reduced=form == "round_reduced")
        assert compare.max_relerr(host_rows(norm, rows), exact, fmt) <= compare.TOL[fmt]
        if form == "dead_residual":
            assert res is None
        else:
            assert compare.bits_equal(host_rows(res, rows), r)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("flags,T", [(arrms.FORCE_ROW, 21), (arrms.FORCE_SPLIT, 21),
                                     (arrms.FORCE_SPLIT, 5000)], ids=["row", "split", "split_loop"])
def test_round_reduced_sum(flags, T, dtype):
    """ARRMS_ROUND_REDUCED: the W-way sum is rounded to 16 bits before the residual."""
    wl = WORKLOADS["c2"]
    fmt = FMT[dtype]
    inp = cuda_inputs(wl, T, dtype, seed=77 + T, device_draw=T > 1000)
    norm, res = arrms.fused_allreduce_rms_norm(inp["partials"], inp["residual"], inp["weight"],
                                               wl.eps, True, flags=flags, round_reduced=True)
    torch.cuda.synchronize()
    rows = sample_rows(T, 128, seed=1)
    P = [host_rows(p, rows) for p in inp["partials"]]
    R = host_rows(inp["residual"], rows)
    n, r, exact = oracle.ar_rms(P, R, bits(inp["weight"]), wl.eps, True, fmt, round_reduced=True)
    assert compare.bits_equal(host_rows(res, rows), r)
    assert compare.max_relerr(host_rows(norm, rows), exact, fmt) <= compare.TOL[fmt]
    # and it differs from the fp32-sum reading somewhere (the option is live)
    _, r_fp32, _ = oracle.ar_rms(P, R, bits(inp["weight"]), wl.eps, True, fmt)
    assert not compare.bits_equal(r, r_fp32)


def test_round_reduced_quant():
    wl = WORKLOADS["c4"]
    inp = cuda_inputs(wl, 256)
    outs = arrms.fused_allreduce_rms_norm_quant(inp["partials"], inp["residual"], inp["weight"],
                                                wl.eps, wl.group, round_reduced=True)
    torch.cuda.synchronize()
    norm, q, scales, res = outs
    P = [bits(p) for p in inp["partials"]]
    n_o, c_o, s_o, r_o, exact = oracle.ar_rms_quant(P, bits(inp["residual"]), bits(inp["weight"]),
                                                    wl.eps, False, wl.group, round_reduced=True)
    assert compare.bits_equal(bits(res), r_o)
    assert compare.max_relerr(bits(norm), exact, oracle.BF16) <= compare.TOL[oracle.BF16]
    assert compare.max_code_distance(q.view(torch.uint8).cpu().numpy(), c_o) <= 1
    assert compare.max_scale_relerr(scales.cpu().numpy(), s_o) <= compare.SCALE_TOL


@pytest.mark.parametrize("flags", [arrms.FORCE_ROW, arrms.FORCE_SPLIT], ids=["row", "split"])
def test_round_reduced_worked_case(flags):
    """P = {1, 2^-8}, R = 2^-9 in bf16: fp32 sum gives 1 + 2^-7, the rounded sum 1."""
    H = 1024
    one = torch.ones(2, H, dtype=torch.bfloat16, device=DEV)
    parts = [one, one * 2.0 ** -8]
    res = one * 2.0 ** -9
    w = torch.ones(H, dtype=torch.bfloat16, device=DEV)
    _, r_fused = arrms.fused_allreduce_rms_norm(parts, res, w, 1e-6, flags=flags)
    _, r_round = arrms.fused_allreduce_rms_norm(parts, res, w, 1e-6, flags=flags,
                                                round_reduced=True)
    torch.cuda.synchronize()
    assert torch.all(r_fused == 1.0 + 2.0 ** -7)
    assert torch.all(r_round == 1.0)


# ------------------------------------------- seeded random configurations
def random_config(seed):
    """One call's configuration drawn from everything the library accepts."""
    rng = np.random.default_rng(seed)
    dtype = [torch.bfloat16, torch.float16][rng.integers(2)]
    W = int(rng.integers(1, 17))
    max_packs = 1024 if W > 8 else 2048
    H = 8 * int(rng.integers(1, max_packs + 1))
    T = int(rng.choice([0, 1, 2, 3, 7, 31, 80, 81, 129, 300]))
    quant = bool(rng.random() < 0.4)
    group = 0
    if quant:
        choices = [g for g in (8, 16, 32, 64, 128, 256, 512) if H % g == 0]
        group = int(rng.choice(choices))
    kinds = ["default", "split"]
    if W <= 8 and T <= 80 and H <= 8192:
        kinds.append("row")
    kind = kinds[rng.integers(len(kinds))]
    return dict(dtype=dtype, W=W, H=H, T=T, group=group, kind=kind,
                gemma=bool(rng.random() < 0.5), residual=["yes", "none", "dead"][rng.integers(3)],
                round_reduced=bool(rng.random() < 0.3), with_norm=bool(rng.random() < 0.7))


@pytest.mark.parametrize("seed", range(40))
def test_random_configurations(seed):
    c = random_config(seed)
    print(f"[random] seed {seed}: {c}", flush=True)
    flags = {"default": 0, "split": arrms.FORCE_SPLIT, "row": arrms.FORCE_ROW}[c["kind"]]
    inp = cuda_inputs(GENERIC, c["T"], c["dtype"], W=c["W"], H=c["H"], seed=10_000 + seed)
    if c["residual"] == "none":
        inp["residual"] = None
    residual_out = None if c["residual"] == "dead" else "new"
    fmt = FMT[c["dtype"]]
    T, H = c["T"], c["H"]
    rows = np.arange(T)
    P = [host_rows(p, rows) for p in inp["partials"]]
    R = None if inp["residual"] is None else host_rows(inp["residual"], rows)
    if c["group"]:
        outs = arrms.fused_allreduce_rms_norm_quant(
            inp["partials"], inp["residual"], inp["weight"], 1e-6, c["group"], c["gemma"],
            with_norm=c["with_norm"], residual_out=residual_out, flags=flags,
            round_reduced=c["round_reduced"])
        torch.cuda.synchronize()
        norm, q, sc, res = outs
        _, c_o, s_o, r_o, exact = oracle.ar_rms_quant(P, R, bits(inp["weight"]), 1e-6, c["gemma"],
                                                      c["group"], fmt,
                                                      round_reduced=c["round_reduced"])
        assert compare.max_code_distance(q.view(torch.uint8).reshape(T, H).cpu().numpy(), c_o) <= 1
        assert compare.max_scale_relerr(sc.reshape(T, H // c["group"]).cpu().numpy(),
                                        s_o) <= compare.SCALE_TOL
    else:
        norm, res = arrms.fused_allreduce_rms_norm(
            inp["partials"], inp["residual"], inp["weight"], 1e-6, c["gemma"],
            residual_out=residual_out, flags=flags, round_reduced=c["round_reduced"])
        torch.cuda.synchronize()
        _, r_o, exact = oracle.ar_rms(P, R, bits(inp["weight"]), 1e-6, c["gemma"], fmt,
                                      round_reduced=c["round_reduced"])
    if norm is not None:
        assert compare.max_relerr(host_rows(norm, rows), exact, fmt) <= compare.TOL[fmt]
    if res is None:
        assert c["residual"] == "dead"
    else:
        assert compare.bits_equal(host_rows(res, rows), r_o)


@pytest.mark.parametrize("seed", range(20))
def test_random_qk_configurations(seed):
    """QK-norm over shapes drawn from the whole accepted domain (both lane
    layouts, one to four packs per lane)."""
    rng = np.random.default_rng(50_000 + seed)
    while True:
        W = int(rng.integers(1, 9))
        q = 256 * int(rng.integers(1, 33))
        kv = 256 * int(rng.integers(1, 17))
        if W * (q + kv) <= 32768:
            break
    T = int(rng.choice([1, 2, 5, 17, 64]))
    dtype = [torch.bfloat16, torch.float16][rng.integers(2)]
    print(f"[random qk] seed {seed}: W={W} T={T} q={q} kv={kv} {dtype}", flush=True)
    inp = to_cuda(workloads.make_qk_inputs(WORKLOADS["c5"], T, dtype, W=W, q_size=q, kv_size=kv,
                                           seed=60_000 + seed))
    q_out, k_out = arrms.fused_qk_norm(inp["shards"], inp["q_weight"], inp["k_weight"], q, kv,
                                       1e-6)
    torch.cuda.synchronize()
    check_qk(inp, q, kv, 1e-6, q_out, k_out, FMT[dtype])


def test_concurrent_callers_on_their_own_streams():
    """Four host threads, each with its own stream, shape and inputs, call the
    library concurrently (the ctypes calls release the interpreter lock): the
    row body, the row-ahead split, the split of few rows per workgroup and the
    FP8 epilogue.  Each also makes one invalid call and reads its own error
    message (the last error is per thread).  Every output matches the oracle."""
    import threading
    cases = [(2, 16, 1024, 0), (8, 4000, 8192, 0), (6, 1500, 8192, 0), (4, 256, 7168, 128)]
    inputs = [cuda_inputs(WORKLOADS["c4"], T, W=W, H=H, seed=900 + i, device_draw=True)
              for i, (W, T, H, G) in enumerate(cases)]
    torch.cuda.synchronize()
    results, errors = [None] * len(cases), []
    barrier = threading.Barrier(len(cases))

    def worker(i):
        try:
            W, T, H, G = cases[i]
            inp = inputs[i]
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                barrier.wait()
                for _ in range(20):
                    if G:
                        out = arrms.fused_allreduce_rms_norm_quant(
                            inp["partials"], inp["residual"], inp["weight"], 1e-6, G)
                    else:
                        out = arrms.fused_allreduce_rms_norm(inp["partials"], inp["residual"],
                                                             inp["weight"], 1e-6)
                    try:
                        arrms.fused_allreduce_rms_norm(inp["partials"], inp["residual"],
                                                       inp["weight"], float("nan"))
                        errors.append(f"thread {i}: NaN eps accepted")
                    except arrms.ArrmsError as e:
                        if e.code != arrms.EINVAL or "eps" not in e.message:
                            errors.append(f"thread {i}: wrong error {e}")
                stream.synchronize()
            results[i] = out
        except Exception as e:  # reported below, with the thread
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a caller thread did not finish"
    assert not errors, errors
    for (W, T, H, G), inp, out in zip(cases, inputs, results):
        rows = sample_rows(T, 96, seed=T)
        if G:
            sub = {"partials": [p.index_select(0, torch.as_tensor(rows, device=DEV))
                                for p in inp["partials"]],
                   "residual": inp["residual"].index_select(0, torch.as_tensor(rows, device=DEV)),
                   "weight": inp["weight"]}
            idx = torch.as_tensor(rows, device=DEV)
            norm, q, scales, res = out
            check_quant(sub, 1e-6, False, G, (norm.index_select(0, idx),
                                              q.view(torch.uint8).index_select(0, idx),
                                              scales.index_select(0, idx),
                                              res.index_select(0, idx)))
        else:
            check_rms(inp, out[0], out[1], 1e-6, False, rows=rows)
