"""Pins of the acceptance rules in oracle/compare.py (CPU)."""
import numpy as np

import oracle
from oracle import compare


def test_code_distance_orders_sign_magnitude():
    assert compare.max_code_distance([0x7E], [0x7D]) == 1
    assert compare.max_code_distance([0x00], [0x80]) == 0          # +0 and -0
    assert compare.max_code_distance([0x01], [0x81]) == 2          # across zero
    assert compare.max_code_distance([0x70, 0x3A], [0x70, 0x3B]) == 1
    assert compare.max_code_distance([], []) == 0


def test_code_distance_nan_patterns():
    # S.1111.111 is NaN for either sign: the two patterns are the same value
    assert compare.max_code_distance([0x7F], [0xFF]) == 0
    assert compare.max_code_distance([0x7F, 0x10], [0xFF, 0x10]) == 0
    # a NaN against a number is never within tolerance
    assert compare.max_code_distance([0x7F], [0x7E]) > 1
    assert compare.max_code_distance([0x00], [0xFF]) > 1


def test_relerr_rules():
    bf = oracle.BF16
    one = oracle.encode(bf, 1.0)
    nxt = one + 1                                     # 1 + 2^-7
    assert compare.max_relerr(np.array([one], np.uint16), np.array([1.0]), bf) == 0.0
    assert abs(compare.max_relerr(np.array([nxt], np.uint16), np.array([1.0]), bf)
               - 2.0 ** -7) < 1e-12
    nan = oracle.encode(bf, float("nan"))
    assert compare.max_relerr(np.array([nan], np.uint16), np.array([np.nan]), bf) == 0.0
    assert compare.max_relerr(np.array([one], np.uint16), np.array([np.nan]), bf) == float("inf")
    assert compare.max_relerr(np.array([nan], np.uint16), np.array([1.0]), bf) == float("inf")
    inf = oracle.encode(bf, float("inf"))
    assert compare.max_relerr(np.array([inf], np.uint16), np.array([np.inf]), bf) == 0.0
    assert compare.max_relerr(np.array([inf], np.uint16), np.array([-np.inf]), bf) == float("inf")


def test_scale_relerr():
    assert compare.max_scale_relerr(np.float32([2.0]), np.float32([2.0])) == 0.0
    assert compare.max_scale_relerr(np.float32([0.0]), np.float32([0.0])) == 0.0
    e = compare.max_scale_relerr(np.float32([np.nextafter(np.float32(2), np.float32(3))]),
                                 np.float32([2.0]))
    assert 0 < e < 2e-7
