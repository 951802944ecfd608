"""Python access to the reference oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY.  The oracle is the plain CPU definition of the fused
W-way reduce + residual add + RMSNorm epilogue (and its FP8 per-group-quant and
QK-norm variants) that the GPU library is checked against.  Only the tests, the
smoke check and the CPU-baseline leg of the benchmark import this module; the
GPU library never does.  This module only marshals numpy arrays into the C
functions: every step of the arithmetic is in ``oracle.c``.

Arrays of 16-bit values are passed as their bit patterns (``numpy.uint16``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

BF16, FP16, FP32, E4M3 = 0, 1, 2, 3

_lib = None


def compile_c(src: str, out: str) -> str:
    """gcc -O2, IEEE arithmetic (no contraction, no fast-math), shared object."""
    tmp = out + ".tmp"
    subprocess.check_call([
        "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
        "-Wall", "-Wextra", "-fPIC", "-shared", src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so``."""
    if force or not os.path.exists(LIB):
        compile_c(SRC, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        # ORACLE_LIB lets the planted-mistake tests run the pins against a
        # deliberately broken copy of the oracle
        path = os.environ.get("ORACLE_LIB") or LIB
        if path == LIB and (not os.path.exists(LIB)
                            or os.path.getmtime(LIB) < os.path.getmtime(SRC)):
            build(force=True)
        _lib = open_library(path)
    return _lib


def open_library(path: str):
    lib = ctypes.CDLL(path)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    u16pp = ctypes.POINTER(u16p)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.oracle_decode.argtypes = [ctypes.c_int, ctypes.c_uint32]
    lib.oracle_decode.restype = ctypes.c_double
    lib.oracle_round.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.oracle_round.restype = ctypes.c_double
    lib.oracle_bits.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.oracle_bits.restype = ctypes.c_uint32
    lib.oracle_encode.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.oracle_encode.restype = ctypes.c_uint32
    lib.oracle_one_stage.argtypes = [ctypes.c_int, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.oracle_one_stage.restype = ctypes.c_int
    lib.oracle_ar_rms_ex.argtypes = [ctypes.c_int, i64, i64, ctypes.c_int, u16pp, u16p, u16p,
                                     ctypes.c_float, ctypes.c_int, ctypes.c_int, u16p, u16p, dp]
    lib.oracle_ar_rms_ex.restype = ctypes.c_int
    lib.oracle_ar_rms_quant_ex.argtypes = [ctypes.c_int, i64, i64, ctypes.c_int, u16pp, u16p,
                                           u16p, ctypes.c_float, ctypes.c_int, ctypes.c_int, i64,
                                           u16p, ctypes.POINTER(ctypes.c_uint8),
                                           ctypes.POINTER(ctypes.c_float), u16p, dp]
    lib.oracle_ar_rms_quant_ex.restype = ctypes.c_int
    lib.oracle_qknorm.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_int, u16pp,
                                  u16p, u16p, ctypes.c_float, u16p, u16p, dp, dp]
    lib.oracle_qknorm.restype = ctypes.c_int
    return lib


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bit patterns, got {a.dtype}")
    return a


def _ptr_array(arrays):
    u16p = ctypes.POINTER(ctypes.c_uint16)
    return (u16p * len(arrays))(*[_ptr(a, ctypes.c_uint16) for a in arrays])


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def decode(fmt: int, bits: int) -> float:
    return _load().oracle_decode(fmt, int(bits))


def round_to(fmt: int, x: float) -> float:
    return _load().oracle_round(fmt, float(x))


def encode(fmt: int, x: float) -> int:
    return _load().oracle_encode(fmt, float(x))


def decode_array(fmt: int, bits) -> np.ndarray:
    lib = _load()
    flat = np.asarray(bits).reshape(-1)
    out = np.fromiter((lib.oracle_decode(fmt, int(b)) for b in flat), dtype=np.float64,
                      count=flat.size)
    return out.reshape(np.shape(bits))


def encode_array(fmt: int, values) -> np.ndarray:
    lib = _load()
    flat = np.asarray(values, dtype=np.float64).reshape(-1)
    dt = np.uint8 if fmt == E4M3 else np.uint16
    out = np.fromiter((lib.oracle_encode(fmt, float(v)) for v in flat), dtype=dt,
                      count=flat.size)
    return out.reshape(np.shape(values))


# --------------------------------------------------------------------------
# the method
# --------------------------------------------------------------------------

def one_stage(W: int, numel: int, hidden: int, fmt: int, fully_connected: int = 1) -> bool:
    return bool(_load().oracle_one_stage(W, numel, hidden, fmt, fully_connected))


def ar_rms(partials, residual, weight, eps: float, gemma: bool, fmt: int = BF16,
           want_exact: bool = True, round_reduced: bool = False):
    """Returns (norm_out bits, residual_out bits, exact fp64 or None).

    partials: sequence of W uint16 arrays [T, H]; residual: [T, H] or None (no
    residual term; residual_out is then the reduced sum itself); weight: [H]."""
    partials = [_u16(p) for p in partials]
    W = len(partials)
    T, H = partials[0].shape
    residual = None if residual is None else _u16(residual)
    weight = _u16(weight)
    norm = np.empty((T, H), np.uint16)
    res_out = np.empty((T, H), np.uint16)
    exact = np.empty((T, H), np.float64) if want_exact else None
    rc = _load().oracle_ar_rms_ex(W, T, H, fmt, _ptr_array(partials),
                                  _ptr(residual, ctypes.c_uint16), _ptr(weight, ctypes.c_uint16),
                                  float(eps), int(bool(gemma)), int(bool(round_reduced)),
                                  _ptr(norm, ctypes.c_uint16), _ptr(res_out, ctypes.c_uint16),
                                  _ptr(exact, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_ar_rms rejected its arguments")
    return norm, res_out, exact


def ar_rms_quant(partials, residual, weight, eps: float, gemma: bool, group: int,
                 fmt: int = BF16, want_exact: bool = True, round_reduced: bool = False):
    """Returns (norm_out bits, codes u8, scales f32, residual_out bits, exact)."""
    partials = [_u16(p) for p in partials]
    W = len(partials)
    T, H = partials[0].shape
    residual = None if residual is None else _u16(residual)
    weight = _u16(weight)
    norm = np.empty((T, H), np.uint16)
    codes = np.empty((T, H), np.uint8)
    scales = np.empty((T, H // group if group > 0 else 0), np.float32)
    res_out = np.empty((T, H), np.uint16)
    exact = np.empty((T, H), np.float64) if want_exact else None
    rc = _load().oracle_ar_rms_quant_ex(W, T, H, fmt, _ptr_array(partials),
                                        _ptr(residual, ctypes.c_uint16),
                                        _ptr(weight, ctypes.c_uint16), float(eps),
                                        int(bool(gemma)), int(bool(round_reduced)), int(group),
                                        _ptr(norm, ctypes.c_uint16), _ptr(codes, ctypes.c_uint8),
                                        _ptr(scales, ctypes.c_float), _ptr(res_out, ctypes.c_uint16),
                                        _ptr(exact, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_ar_rms_quant rejected its arguments")
    return norm, codes, scales, res_out, exact


def qknorm(shards, q_size: int, kv_size: int, q_weight, k_weight, eps: float,
           fmt: int = BF16, want_exact: bool = True):
    """shards: W uint16 arrays [T, stride] laid out [q | k | v].

    Returns (q_out [W,T,q], k_out [W,T,kv], q_exact, k_exact)."""
    shards = [_u16(s) for s in shards]
    W = len(shards)
    T, stride = shards[0].shape
    q_weight = _u16(q_weight)
    k_weight = _u16(k_weight)
    q_out = np.empty((W, T, q_size), np.uint16)
    k_out = np.empty((W, T, kv_size), np.uint16)
    q_exact = np.empty((W, T, q_size), np.float64) if want_exact else None
    k_exact = np.empty((W, T, kv_size), np.float64) if want_exact else None
    rc = _load().oracle_qknorm(W, T, q_size, kv_size, stride, fmt, _ptr_array(shards),
                               _ptr(q_weight, ctypes.c_uint16), _ptr(k_weight, ctypes.c_uint16),
                               float(eps), _ptr(q_out, ctypes.c_uint16),
                               _ptr(k_out, ctypes.c_uint16), _ptr(q_exact, ctypes.c_double),
                               _ptr(k_exact, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle_qknorm rejected its arguments")
    return q_out, k_out, q_exact, k_exact
