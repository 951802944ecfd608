"""Acceptance rules for comparing the GPU library's outputs with the oracle.

TEST INFRASTRUCTURE ONLY (used by the tests, the smoke check and the
benchmark's parity guard).

  residual_out      bit-exact
  norm_out, q/k     max_i |gpu_i - exact_i| / max(|exact_i|, smallest normal)
                    <= 4e-3 (bf16) / 1e-3 (fp16), against the oracle's
                    unrounded fp64 value; a correctly rounded result is within
                    the unit roundoff 2^-8 (bf16) / 2^-11 (fp16), the kernel's
                    fp32 evaluation adds about 1e-7
  FP8 codes         within one E4M3 step: |ord(a) - ord(b)| <= 1 with
                    ord(c) = +-(c & 0x7F) by the sign bit
  FP8 scales        relative error <= 1e-6
NaNs must sit where the oracle has NaNs.
"""
from __future__ import annotations

import numpy as np
import torch

from . import BF16, FP16

TOL = {BF16: 4e-3, FP16: 1e-3}
MIN_NORMAL = {BF16: 2.0 ** -126, FP16: 2.0 ** -14}
SCALE_TOL = 1e-6


def values(bits, fmt: int) -> np.ndarray:
    dt = torch.bfloat16 if fmt == BF16 else torch.float16
    b = np.ascontiguousarray(bits).view(np.int16)
    return torch.from_numpy(b).view(dt).double().numpy()


def max_relerr(gpu_bits, exact, fmt: int) -> float:
    """Largest relative error of 16-bit outputs against fp64 values; inf if a
    NaN is missing or extra."""
    g = values(gpu_bits, fmt)
    e = np.asarray(exact, np.float64)
    if not np.array_equal(np.isnan(g), np.isnan(e)):
        return float("inf")
    ok = ~np.isnan(e)
    if not ok.any():
        return 0.0
    g, e = g[ok], e[ok]
    if not np.array_equal(np.isinf(g), np.isinf(e)) or np.any(g[np.isinf(g)] != e[np.isinf(e)]):
        return float("inf")
    fin = np.isfinite(e)
    if not fin.any():
        return 0.0
    den = np.maximum(np.abs(e[fin]), MIN_NORMAL[fmt])
    return float(np.max(np.abs(g[fin] - e[fin]) / den))


def e4m3_ord(codes) -> np.ndarray:
    c = np.asarray(codes, np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def e4m3_is_nan(codes) -> np.ndarray:
    """E4M3FN has two NaN patterns, S.1111.111, whatever the sign bit."""
    return (np.asarray(codes, np.int32) & 0x7F) == 0x7F


def max_code_distance(a, b) -> int:
    """Largest distance in steps between E4M3FN codes (sign-magnitude order,
    +0 and -0 equal).  The two NaN patterns are equal to each other; a NaN
    against a number is an unbounded mismatch."""
    a = np.asarray(a, np.uint8)
    b = np.asarray(b, np.uint8)
    if a.size == 0:
        return 0
    na, nb = e4m3_is_nan(a), e4m3_is_nan(b)
    if not np.array_equal(na, nb):
        return 1 << 30
    ok = ~na
    if not ok.any():
        return 0
    return int(np.max(np.abs(e4m3_ord(a[ok]) - e4m3_ord(b[ok]))))


def max_scale_relerr(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    den = np.where(b == 0, 1.0, np.abs(b))
    return float(np.max(np.abs(a - b) / den))


def bits_equal(a, b) -> bool:
    return np.array_equal(np.asarray(a, np.uint16), np.asarray(b, np.uint16))
