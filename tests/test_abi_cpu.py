"""Host-side checks of libarrms that need no GPU: the library loads and exports
every entry point include/arrms.h declares, the dispatch predicate matches the
hand-derived cases and the oracle's independent predicate, plans choose the
documented kernels, and every validation error returns its status before any
launch (fake, never dereferenced addresses are used for pointer arguments)."""
import ctypes
import os
import re

import pytest

import oracle
from golden_cases import one_stage_cases
from tp_all_reduce_amd import arrms, workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "arrms.h")

A = 0x10000          # a fake 16-byte-aligned device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ar_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "ar_qknorm_run", "ar_rms_last_error", "ar_rms_one_stage", "ar_rms_plan",
        "ar_rms_plan_destroy", "ar_rms_plan_kernel", "ar_rms_quant_run", "ar_rms_run"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(arrms.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


# ------------------------------------------------------------- predicate
CASES = one_stage_cases()


@pytest.mark.parametrize("W,numel,hidden,dtype,fc,expected,note", CASES,
                         ids=[c[-1] or str(i) for i, c in enumerate(CASES)])
def test_one_stage_golden(W, numel, hidden, dtype, fc, expected, note):
    T = numel // hidden          # tokens over all leading dimensions
    assert arrms.ar_rms_one_stage(W, T, hidden, dtype, fc) == bool(expected)


def test_one_stage_agrees_with_oracle_on_a_sweep():
    for W in (1, 2, 3, 4, 5, 8, 9):
        for H in (8, 1000, 1024, 4096, 6144, 7168, 8192, 8200):
            for T in (0, 1, 10, 15, 16, 21, 22, 31, 32, 79, 80, 81, 200):
                for dt in (0, 1, 2):
                    for fc in (0, 1):
                        assert (arrms.ar_rms_one_stage(W, T, H, dt, fc)
                                == oracle.one_stage(W, T * H, H, dt, fc)), (W, H, T, dt, fc)


# ------------------------------------------------------------------ plans
def test_plan_dispatch_for_the_workloads():
    c1, c2, c3, c4 = (workloads.WORKLOADS[k] for k in ("c1", "c2", "c3", "c4"))
    assert arrms.ar_rms_plan(c1.W, 8, c1.H).kernel == arrms.KERNEL_ROW
    for T in c2.Ts:
        want = arrms.KERNEL_ROW if T <= 31 else arrms.KERNEL_SPLIT
        assert arrms.ar_rms_plan(c2.W, T, c2.H).kernel == want
        assert arrms.ar_rms_plan(c2.W, T, c2.H, flags=arrms.FORCE_ROW).kernel == arrms.KERNEL_ROW
        assert (arrms.ar_rms_plan(c2.W, T, c2.H, flags=arrms.FORCE_SPLIT).kernel
                == arrms.KERNEL_SPLIT)
    for T in c3.Ts:
        assert arrms.ar_rms_plan(c3.W, T, c3.H).kernel == arrms.KERNEL_SPLIT
    assert arrms.ar_rms_plan(c4.W, 256, c4.H).kernel == arrms.KERNEL_SPLIT


@pytest.mark.parametrize("args,code", [
    ((0, 8, 1024, 0, 0), arrms.EINVAL),          # W < 1
    ((2, -1, 1024, 0, 0), arrms.EINVAL),         # T < 0
    ((2, 8, 0, 0, 0), arrms.EINVAL),             # H <= 0
    ((2, 8, 1024, 2, 0), arrms.EINVAL),          # fp32 / unknown dtype
    ((2, 8, 1024, 0, 8), arrms.EINVAL),          # unknown flag bit
    ((2, 8, 1024, 0, 3), arrms.EINVAL),          # both FORCE flags
    ((17, 8, 1024, 0, 0), arrms.ENOTSUP),        # W > 16
    ((9, 8, 8200, 0, 0), arrms.ENOTSUP),         # W > 8 with rows beyond 8192
    ((9, 8, 1024, 0, 1), arrms.ENOTSUP),         # FORCE_ROW with W > 8
    ((2, 8, 1020, 0, 0), arrms.ENOTSUP),         # H % 8 != 0
    ((2, 8, 16392, 0, 0), arrms.ENOTSUP),        # H > 16384
    ((2, 81, 1024, 0, 1), arrms.ENOTSUP),        # FORCE_ROW beyond 80 tokens
    ((2, 8, 8200, 0, 1), arrms.ENOTSUP),         # FORCE_ROW beyond 1024 packs
])
def test_plan_errors(args, code):
    with pytest.raises(arrms.ArrmsError) as e:
        arrms.ar_rms_plan(*args)
    assert e.value.code == code and e.value.message


def test_more_than_eight_partials_plan_the_split_kernel():
    for W in (9, 12, 16):
        for flags in (0, arrms.FORCE_SPLIT):
            p = arrms.ar_rms_plan(W, 8, 8192, 0, flags)
            assert p.kernel == arrms.KERNEL_SPLIT
        assert not arrms.ar_rms_one_stage(W, 8, 1024)


def test_round_reduced_flag_accepted_with_any_kernel():
    for f in (0, arrms.FORCE_ROW, arrms.FORCE_SPLIT):
        p = arrms.ar_rms_plan(4, 8, 4096, 0, f | arrms.ROUND_REDUCED)
        assert p.kernel == (arrms.KERNEL_SPLIT if f == arrms.FORCE_SPLIT else arrms.KERNEL_ROW)


def test_plan_limits_accepted():
    assert arrms.ar_rms_plan(8, 80, 8192, 1, arrms.FORCE_ROW).kernel == arrms.KERNEL_ROW
    assert arrms.ar_rms_plan(1, 0, 8, 0).kernel == arrms.KERNEL_ROW
    assert arrms.ar_rms_plan(8, 1 << 20, 16384, 0).kernel == arrms.KERNEL_SPLIT


def test_null_plan_and_null_out():
    lib = arrms.library()
    assert lib.ar_rms_plan(2, 8, 1024, 0, 0, None) == arrms.EINVAL
    assert lib.ar_rms_plan_kernel(None) == arrms.EINVAL
    ptrs = (ctypes.c_void_p * 2)(A, A)
    assert lib.ar_rms_run(None, ptrs, A, A, 1e-6, 0, A, A, None) == arrms.EINVAL
    assert "plan" in arrms.ar_rms_last_error()
    lib.ar_rms_plan_destroy(None)       # ignored


# ------------------------------------------------------- run-time validation
def _run(plan, partials=(A, A), residual=A, weight=A, eps=1e-6, norm_out=A, residual_out=A):
    lib = arrms.library()
    arr = None if partials is None else (ctypes.c_void_p * len(partials))(*partials)
    return lib.ar_rms_run(plan.handle, arr, residual, weight, eps, 0, norm_out, residual_out,
                          None)


@pytest.mark.parametrize("kw,code", [
    (dict(partials=None), arrms.EINVAL),
    (dict(partials=(A, 0)), arrms.EINVAL),
    (dict(partials=(A, A + 8)), arrms.EINVAL),
    (dict(residual=A + 2), arrms.EINVAL),
    (dict(weight=0), arrms.EINVAL),
    (dict(weight=A + 4), arrms.EINVAL),
    (dict(norm_out=0), arrms.EINVAL),
    (dict(norm_out=A + 8), arrms.EINVAL),
    (dict(residual_out=A + 1), arrms.EINVAL),
    (dict(eps=float("nan")), arrms.EINVAL),
    (dict(eps=float("inf")), arrms.EINVAL),
    (dict(eps=-1e-6), arrms.EINVAL),
])
def test_run_rejects_bad_arguments(kw, code):
    plan = arrms.ar_rms_plan(2, 8, 1024)
    assert _run(plan, **kw) == code
    assert arrms.ar_rms_last_error()


def test_run_with_zero_tokens_is_ok_and_launches_nothing():
    plan = arrms.ar_rms_plan(2, 0, 1024)
    assert _run(plan) == arrms.OK
    assert _run(plan, residual=None, residual_out=None) == arrms.OK
    assert arrms.ar_rms_last_error() == ""


def _quant(plan, group, q_out=A, scales=A, norm_out=A):
    lib = arrms.library()
    arr = (ctypes.c_void_p * plan.W)(*([A] * plan.W))
    return lib.ar_rms_quant_run(plan.handle, arr, A, A, 1e-6, 0, group, norm_out, q_out, scales,
                                A, None)


@pytest.mark.parametrize("group,kw,code", [
    (96, {}, arrms.ENOTSUP),            # not a power of two
    (4, {}, arrms.ENOTSUP),             # below one pack
    (1024, {}, arrms.ENOTSUP),          # above 512
    (256, {}, arrms.ENOTSUP),           # 256 does not divide H = 7296
    (128, dict(q_out=0), arrms.EINVAL),
    (128, dict(q_out=A + 4), arrms.EINVAL),
    (128, dict(scales=0), arrms.EINVAL),
    (128, dict(scales=A + 2), arrms.EINVAL),
])
def test_quant_validation(group, kw, code):
    H = 7168 if group != 256 else 7296    # 7296 = 57 * 128, not a multiple of 256
    plan = arrms.ar_rms_plan(4, 0 if code == arrms.OK else 16, H)
    assert _quant(plan, group, **kw) == code


def test_quant_with_zero_tokens_ok():
    plan = arrms.ar_rms_plan(4, 0, 7168)
    assert _quant(plan, 128) == arrms.OK
    assert _quant(plan, 128, norm_out=None) == arrms.OK


def _qk(plan, q, kv, **kw):
    lib = arrms.library()
    arr = (ctypes.c_void_p * plan.W)(*([A] * plan.W))
    args = dict(q_weight=A, k_weight=A, eps=1e-6, q_out=A, k_out=A)
    args.update(kw)
    return lib.ar_qknorm_run(plan.handle, arr, q, kv, args["q_weight"], args["k_weight"],
                             args["eps"], args["q_out"], args["k_out"], None)


def test_qk_validation():
    plan = arrms.ar_rms_plan(4, 64, 2048)
    assert _qk(plan, 1536, 256, q_weight=0) == arrms.EINVAL
    assert _qk(plan, 1536, 256, k_out=A + 8) == arrms.EINVAL
    assert _qk(plan, 1536, 256, eps=-1.0) == arrms.EINVAL
    assert _qk(plan, 0, 1024) == arrms.EINVAL
    assert _qk(plan, 1792, 128) == arrms.ENOTSUP          # kv not a multiple of 256
    assert _qk(plan, 1024, 256) == arrms.ENOTSUP          # q + 2 kv != H
    big = arrms.ar_rms_plan(8, 64, 4096 + 2 * 1024)
    assert _qk(big, 4096, 1024) == arrms.ENOTSUP          # W (q + kv) > 32768
    many = arrms.ar_rms_plan(9, 64, 768)
    assert _qk(many, 256, 256) == arrms.ENOTSUP           # more than eight shards
    zero = arrms.ar_rms_plan(4, 0, 2048)
    assert _qk(zero, 1536, 256) == arrms.OK


def test_binding_refuses_cpu_tensors():
    import torch
    plan = arrms.ar_rms_plan(2, 2, 64)
    x = torch.zeros(2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        arrms.ar_rms_run(plan, [x, x], x, torch.zeros(64, dtype=torch.bfloat16), 1e-6, False,
                         x, x)


def test_zero_tokens_accept_null_activation_pointers():
    lib = arrms.library()
    plan = arrms.ar_rms_plan(2, 0, 1024)
    ptrs = (ctypes.c_void_p * 2)(None, None)
    assert lib.ar_rms_run(plan.handle, ptrs, None, A, 1e-6, 0, None, None, None) == arrms.OK
    qplan = arrms.ar_rms_plan(4, 0, 7168)
    qp = (ctypes.c_void_p * 4)(None, None, None, None)
    assert lib.ar_rms_quant_run(qplan.handle, qp, None, A, 1e-6, 0, 128, None, None, None, None,
                                None) == arrms.OK
    kplan = arrms.ar_rms_plan(4, 0, 2048)
    assert lib.ar_qknorm_run(kplan.handle, qp, 1536, 256, A, A, 1e-6, None, None,
                             None) == arrms.OK
    # with tokens present the same NULLs are errors
    plan8 = arrms.ar_rms_plan(2, 8, 1024)
    assert lib.ar_rms_run(plan8.handle, ptrs, None, A, 1e-6, 0, A, None, None) == arrms.EINVAL


def test_binding_device_and_stream_checks():
    import torch
    # raw addresses name no device; a stream of another device is refused
    assert arrms._device_of([A, A], A, None) is None

    class FakeStream:
        device = torch.device("cuda", 1)
        cuda_stream = 0
    with pytest.raises(ValueError):
        arrms._stream(FakeStream(), torch.device("cuda", 0))
    assert arrms._stream(FakeStream(), torch.device("cuda", 1)) == 0
    assert arrms._stream(1234) == 1234


def test_plan_cache_is_bounded_and_held_plans_stay_valid(monkeypatch):
    monkeypatch.setattr(arrms, "PLAN_CACHE_MAX", 4)
    monkeypatch.setattr(arrms, "_plans", arrms.OrderedDict())
    first = arrms.cached_plan(2, 1, 1024, arrms.BF16)
    assert arrms.cached_plan(2, 1, 1024, arrms.BF16) is first
    for T in range(2, 12):
        arrms.cached_plan(2, T, 1024, arrms.BF16)
    assert len(arrms._plans) == 4
    assert list(arrms._plans)[-1] == (2, 11, 1024, arrms.BF16, 0)
    # evicted from the cache, still usable through the caller's reference
    assert (2, 1, 1024, arrms.BF16, 0) not in arrms._plans
    assert first.kernel == arrms.KERNEL_ROW
    # a hit moves the entry to the most recent end
    arrms.cached_plan(2, 8, 1024, arrms.BF16)
    assert list(arrms._plans)[-1] == (2, 8, 1024, arrms.BF16, 0)


def test_fused_helpers_take_only_new_none_or_a_tensor_for_residual_out():
    import torch
    x = torch.zeros(2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="residual_out"):
        arrms._new_residual_out("alloc", x, x)
    assert arrms._new_residual_out(None, x, x) is None
    assert arrms._new_residual_out(x, x, x) is x
    y = arrms._new_residual_out("new", None, x)
    assert y.shape == x.shape and y.dtype == x.dtype
