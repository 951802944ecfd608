"""ctypes binding of libarrms (declared in include/arrms.h).

The functions named like the C entry points marshal their arguments (torch
tensors or raw device addresses) and raise ArrmsError on any non-OK status.
They also check every tensor against the plan (device, dtype, contiguity,
element count), because the C ABI receives bare pointers and cannot.  The
``fused_*`` helpers additionally allocate the outputs with torch, shaped like
the inputs, and derive the token count as numel // H for inputs of any rank
(vLLM PR #49673 page, "Implementation breakdown" item 1).

Every step of the computation runs in the HIP kernels of libarrms.so.  The
library is loaded on first use; if it has not been built the binding raises
instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
import threading
from collections import OrderedDict

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libarrms.so")

OK, EINVAL, ENOTSUP, EHIP, ENOMEM = 0, -1, -2, -3, -4
BF16, FP16 = 0, 1
FORCE_ROW, FORCE_SPLIT, ROUND_REDUCED = 1, 2, 4
KERNEL_ROW, KERNEL_SPLIT = 0, 1
_STATUS = {OK: "OK", EINVAL: "EINVAL", ENOTSUP: "ENOTSUP", EHIP: "EHIP", ENOMEM: "ENOMEM"}
_TORCH_DTYPE = {BF16: torch.bfloat16, FP16: torch.float16}
_CODE_OF = {torch.bfloat16: BF16, torch.float16: FP16}

_lib = None
_lock = threading.Lock()


class ArrmsError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"libarrms {_STATUS.get(code, code)}: {message}")
        self.code = code
        self.message = message


def library():
    """The loaded libarrms.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with __graft_entry__.build() or "
                    "python -m tp_all_reduce_amd.build (there is no fallback path)")
            lib = ctypes.CDLL(LIB_PATH)
            vp, i64, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32
            vpp = ctypes.POINTER(ctypes.c_void_p)
            lib.ar_rms_one_stage.argtypes = [ctypes.c_int, i64, i64, ctypes.c_int, ctypes.c_int]
            lib.ar_rms_one_stage.restype = ctypes.c_int
            lib.ar_rms_plan.argtypes = [ctypes.c_int, i64, i64, ctypes.c_int, u32, vpp]
            lib.ar_rms_plan.restype = ctypes.c_int
            lib.ar_rms_plan_destroy.argtypes = [vp]
            lib.ar_rms_plan_destroy.restype = None
            lib.ar_rms_plan_kernel.argtypes = [vp]
            lib.ar_rms_plan_kernel.restype = ctypes.c_int
            lib.ar_rms_run.argtypes = [vp, vpp, vp, vp, ctypes.c_float, ctypes.c_int, vp, vp, vp]
            lib.ar_rms_run.restype = ctypes.c_int
            lib.ar_rms_quant_run.argtypes = [vp, vpp, vp, vp, ctypes.c_float, ctypes.c_int,
                                             ctypes.c_int, vp, vp, vp, vp, vp]
            lib.ar_rms_quant_run.restype = ctypes.c_int
            lib.ar_qknorm_run.argtypes = [vp, vpp, ctypes.c_int, ctypes.c_int, vp, vp,
                                          ctypes.c_float, vp, vp, vp]
            lib.ar_qknorm_run.restype = ctypes.c_int
            lib.ar_rms_last_error.argtypes = []
            lib.ar_rms_last_error.restype = ctypes.c_char_p
            _lib = lib
        return _lib


def ar_rms_last_error() -> str:
    return library().ar_rms_last_error().decode()


def _check(rc: int):
    if rc != OK:
        raise ArrmsError(rc, ar_rms_last_error())


class Plan:
    """Owns an ar_rms_plan_t; immutable, shareable."""

    def __init__(self, W: int, T: int, H: int, dtype: int = BF16, flags: int = 0):
        h = ctypes.c_void_p()
        _check(library().ar_rms_plan(int(W), int(T), int(H), int(dtype), int(flags),
                                     ctypes.byref(h)))
        self.handle = h
        self.W, self.T, self.H, self.dtype, self.flags = int(W), int(T), int(H), int(dtype), int(flags)

    @property
    def kernel(self) -> int:
        return ar_rms_plan_kernel(self)

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.dtype]

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.ar_rms_plan_destroy(h)
            self.handle = None


# ---------------------------------------------------------------- C names
def ar_rms_one_stage(W: int, T: int, H: int, dtype: int = BF16, fully_connected: int = 1) -> bool:
    return bool(library().ar_rms_one_stage(int(W), int(T), int(H), int(dtype),
                                           int(fully_connected)))


def ar_rms_plan(W: int, T: int, H: int, dtype: int = BF16, flags: int = 0) -> Plan:
    return Plan(W, T, H, dtype, flags)


def ar_rms_plan_destroy(plan: Plan) -> None:
    if plan.handle:
        library().ar_rms_plan_destroy(plan.handle)
        plan.handle = None


def ar_rms_plan_kernel(plan: Plan) -> int:
    rc = library().ar_rms_plan_kernel(plan.handle)
    if rc < 0:
        _check(rc)
    return rc


def _addr(x, what, numel=None, dtype=None):
    """Device address of a tensor (checked) or a raw integer address."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{what}: expected a tensor or an address, got {type(x).__name__}")
    if not x.is_cuda:
        raise ValueError(f"{what}: must be a GPU tensor")
    if not x.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if dtype is not None and x.dtype != dtype:
        raise ValueError(f"{what}: dtype {x.dtype}, expected {dtype}")
    if numel is not None and x.numel() != numel:
        raise ValueError(f"{what}: {x.numel()} elements, expected {numel}")
    return x.data_ptr()


def _ptr_array(xs, what, numel, dtype):
    arr = (ctypes.c_void_p * len(xs))()
    for i, x in enumerate(xs):
        arr[i] = _addr(x, f"{what}[{i}]", numel, dtype)
    return arr


def _device_of(*args):
    """The one device of the tensor arguments (lists are flattened), or None if
    every argument is a raw address.  Tensors on different devices are refused:
    the kernel runs on one device and dereferences every pointer there."""
    dev = None
    for a in args:
        for x in (a if isinstance(a, (list, tuple)) else (a,)):
            if isinstance(x, torch.Tensor) and x.is_cuda:
                if dev is None:
                    dev = x.device
                elif x.device != dev:
                    raise ValueError(f"tensors on {dev} and {x.device}: all arguments of one "
                                     "call must be on the same device")
    return dev


def _stream(stream, device=None):
    """hipStream_t handle: the given stream, else torch's current stream of the
    arguments' device (of the current device for raw addresses)."""
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    if device is not None and stream.device != device:
        raise ValueError(f"stream on {stream.device}, tensors on {device}")
    return stream.cuda_stream


def ar_rms_run(plan: Plan, partials, residual, weight, eps: float, gemma: bool,
               norm_out, residual_out, stream=None) -> None:
    if len(partials) != plan.W:
        raise ValueError(f"expected {plan.W} partials, got {len(partials)}")
    n, dt = plan.T * plan.H, plan.torch_dtype
    _check(library().ar_rms_run(
        plan.handle, _ptr_array(partials, "partials", n, dt), _addr(residual, "residual", n, dt),
        _addr(weight, "weight", plan.H, dt), float(eps), int(bool(gemma)),
        _addr(norm_out, "norm_out", n, dt), _addr(residual_out, "residual_out", n, dt),
        _stream(stream, _device_of(partials, residual, weight, norm_out, residual_out))))


def ar_rms_quant_run(plan: Plan, partials, residual, weight, eps: float, gemma: bool,
                     group_size: int, norm_out, q_out, scales, residual_out,
                     stream=None) -> None:
    if len(partials) != plan.W:
        raise ValueError(f"expected {plan.W} partials, got {len(partials)}")
    n, dt = plan.T * plan.H, plan.torch_dtype
    if group_size <= 0 or plan.H % group_size:
        n_scales = None   # the library reports the unsupported group size
    else:
        n_scales = plan.T * (plan.H // group_size)
    if isinstance(q_out, torch.Tensor) and q_out.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise ValueError("q_out must be uint8 or float8_e4m3fn")
    _check(library().ar_rms_quant_run(
        plan.handle, _ptr_array(partials, "partials", n, dt), _addr(residual, "residual", n, dt),
        _addr(weight, "weight", plan.H, dt), float(eps), int(bool(gemma)), int(group_size),
        _addr(norm_out, "norm_out", n, dt), _addr(q_out, "q_out", n),
        _addr(scales, "scales", n_scales, torch.float32),
        _addr(residual_out, "residual_out", n, dt),
        _stream(stream, _device_of(partials, residual, weight, norm_out, q_out, scales,
                                   residual_out))))


def ar_qknorm_run(plan: Plan, qkv, q_size: int, kv_size: int, q_weight, k_weight, eps: float,
                  q_out, k_out, stream=None) -> None:
    if len(qkv) != plan.W:
        raise ValueError(f"expected {plan.W} shards, got {len(qkv)}")
    dt = plan.torch_dtype
    W, T = plan.W, plan.T
    _check(library().ar_qknorm_run(
        plan.handle, _ptr_array(qkv, "qkv", T * plan.H, dt), int(q_size), int(kv_size),
        _addr(q_weight, "q_weight", W * q_size, dt), _addr(k_weight, "k_weight", W * kv_size, dt),
        float(eps), _addr(q_out, "q_out", W * T * q_size, dt),
        _addr(k_out, "k_out", W * T * kv_size, dt),
        _stream(stream, _device_of(qkv, q_weight, k_weight, q_out, k_out))))


# ------------------------------------------------------ tensor-level helpers
PLAN_CACHE_MAX = 1024
_plans: OrderedDict = OrderedDict()
_plans_lock = threading.Lock()


def cached_plan(W: int, T: int, H: int, dtype: int, flags: int = 0) -> Plan:
    """Plans depend only on (W, T, H, dtype, flags), so they are shared.  The
    PLAN_CACHE_MAX most recently used are kept (a serving loop meets many
    token counts); a plan still held by a caller stays valid after it leaves
    the cache, since it is destroyed only with its last reference."""
    key = (int(W), int(T), int(H), int(dtype), int(flags))
    with _plans_lock:
        p = _plans.get(key)
        if p is not None:
            _plans.move_to_end(key)
            return p
    p = Plan(W, T, H, dtype, flags)
    with _plans_lock:
        p = _plans.setdefault(key, p)
        _plans.move_to_end(key)
        while len(_plans) > PLAN_CACHE_MAX:
            _plans.popitem(last=False)
    return p


def _new_residual_out(residual_out, residual, x):
    """residual_out as the fused_* helpers take it: "new" allocates it shaped
    like the residual (like the first partial without one); None or a tensor
    passes through."""
    if isinstance(residual_out, str):
        if residual_out != "new":
            raise ValueError(f'residual_out: "new", None or a tensor, got {residual_out!r}')
        return torch.empty_like(residual if residual is not None else x)
    return residual_out


def _tokens(x: torch.Tensor) -> tuple[int, int]:
    H = x.shape[-1]
    return x.numel() // H, H


def fused_allreduce_rms_norm(partials, residual, weight, eps: float, gemma: bool = False,
                             residual_out="new", flags: int = 0, stream=None,
                             round_reduced: bool = False):
    """Returns (norm_out, residual_out) shaped like the first partial and the
    residual.  residual_out="new" allocates it, None skips it (dead residual),
    a tensor receives it (may be `residual` itself).  round_reduced rounds the
    W-way sum to 16 bits before the residual add (the unfused path's numerics)."""
    flags |= ROUND_REDUCED if round_reduced else 0
    x = partials[0]
    T, H = _tokens(x)
    dtype = _CODE_OF[x.dtype]
    plan = cached_plan(len(partials), T, H, dtype, flags)
    norm_out = torch.empty_like(x)
    residual_out = _new_residual_out(residual_out, residual, x)
    ar_rms_run(plan, partials, residual, weight, eps, gemma, norm_out, residual_out, stream)
    return norm_out, residual_out


def fused_allreduce_rms_norm_quant(partials, residual, weight, eps: float, group_size: int = 128,
                                   gemma: bool = False, with_norm: bool = True,
                                   residual_out="new", flags: int = 0, stream=None,
                                   round_reduced: bool = False):
    """Returns (norm_out or None, q_out [.., H] float8_e4m3fn, scales
    [.., H // group_size] fp32, residual_out)."""
    flags |= ROUND_REDUCED if round_reduced else 0
    x = partials[0]
    T, H = _tokens(x)
    dtype = _CODE_OF[x.dtype]
    plan = cached_plan(len(partials), T, H, dtype, flags)
    norm_out = torch.empty_like(x) if with_norm else None
    q_out = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    scales = torch.empty((*x.shape[:-1], H // group_size if group_size > 0 else 0),
                         dtype=torch.float32, device=x.device)
    residual_out = _new_residual_out(residual_out, residual, x)
    ar_rms_quant_run(plan, partials, residual, weight, eps, gemma, group_size, norm_out, q_out,
                     scales, residual_out, stream)
    return norm_out, q_out, scales, residual_out


def fused_qk_norm(shards, q_weight, k_weight, q_size: int, kv_size: int, eps: float,
                  stream=None):
    """shards: W tensors [T, q_size + 2*kv_size].  Returns (q_out [W, T, q_size],
    k_out [W, T, kv_size])."""
    x = shards[0]
    T, H = _tokens(x)
    plan = cached_plan(len(shards), T, H, _CODE_OF[x.dtype], 0)
    W = len(shards)
    q_out = torch.empty((W, T, q_size), dtype=x.dtype, device=x.device)
    k_out = torch.empty((W, T, kv_size), dtype=x.dtype, device=x.device)
    ar_qknorm_run(plan, shards, q_size, kv_size, q_weight, k_weight, eps, q_out, k_out, stream)
    return q_out, k_out
