"""Pins of the oracle's number formats against library conversions and the
format definitions (bfloat16, IEEE binary16, OCP FP8 E4M3FN).

The oracle builds every codec from the definitions; these tests check it
against torch's and numpy's conversion routines (independent code), exhaustively
where the format is small."""
import numpy as np
import pytest
import torch

import oracle
from oracle import BF16, E4M3, FP16


def _same(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return np.all(both_nan | eq)


# ---------------------------------------------------------------- decoding
def test_bf16_decode_exhaustive_matches_torch():
    pats = np.arange(1 << 16, dtype=np.uint32)
    mine = oracle.decode_array(BF16, pats)
    ref = torch.from_numpy(pats.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    assert _same(mine, ref.double().numpy())


def test_fp16_decode_exhaustive_matches_numpy():
    pats = np.arange(1 << 16, dtype=np.uint32)
    mine = oracle.decode_array(FP16, pats)
    ref = pats.astype(np.uint16).view(np.float16).astype(np.float64)
    assert _same(mine, ref)


def test_e4m3_decode_exhaustive_matches_torch():
    pats = np.arange(256, dtype=np.uint32)
    mine = oracle.decode_array(E4M3, pats)
    ref = torch.from_numpy(pats.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    assert _same(mine, ref)
    # format facts: max 448 = 0x7E, min normal 2^-6 = 0x08, min subnormal 2^-9 = 0x01,
    # NaN only at S.1111.111
    assert mine[0x7E] == 448.0 and mine[0x08] == 2.0 ** -6 and mine[0x01] == 2.0 ** -9
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])
    assert np.isfinite(np.delete(mine, [0x7F, 0xFF])).all()


# ---------------------------------------------------------------- encoding
def _float32_probe_set(rng, n=20000):
    """float32 values over the whole range, plus exact midpoints between
    neighbouring bf16 values (ties) and values next to them."""
    mant = rng.uniform(1.0, 2.0, n)
    expo = rng.integers(-140, 128, n)
    x = (mant * np.exp2(expo.astype(np.float64))).astype(np.float32)
    x *= np.where(rng.random(n) < 0.5, -1, 1).astype(np.float32)
    # bf16 ties: a bf16 pattern plus half its ulp is 0x....8000 in fp32
    hi = rng.integers(0, 1 << 15, n).astype(np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    near = ((hi << 16) | rng.integers(0x7FF0, 0x8010, n).astype(np.uint32)).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895e38, 3.4e38, 1e-45, -1e-40,
                        1.17549435e-38, 65504.0, 65520.0, 65519.99], np.float32)
    out = np.concatenate([x, ties, near, special])
    return out[np.isfinite(out) | np.isinf(out)]


def test_bf16_encode_matches_torch_rne():
    rng = np.random.default_rng(1)
    x = _float32_probe_set(rng)
    mine = oracle.encode_array(BF16, x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_fp16_encode_matches_numpy_rne():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-28, 18, 20000))
    # exact ties between neighbouring fp16 values, including subnormal ones
    h = rng.integers(0, 0x7BFF, 4000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    x = np.concatenate([x, (lo + hi) / 2, -(lo + hi) / 2, [65504.0, 65519.0, 65520.0, 7e4]])
    mine = oracle.encode_array(FP16, x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(mine, ref)


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(3)
    x = (rng.uniform(-448, 448, 20000) * np.exp2(-rng.integers(0, 14, 20000))).astype(np.float32)
    # every midpoint between neighbouring codes (ties go to the even code)
    vals = oracle.decode_array(E4M3, np.arange(0, 0x7E + 1))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, np.float32([448.0, -448.0, 0.0])])
    mine = oracle.encode_array(E4M3, x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_roundtrip_identity_on_every_finite_pattern():
    for fmt, n in ((BF16, 1 << 16), (FP16, 1 << 16), (E4M3, 256)):
        pats = np.arange(n, dtype=np.uint32)
        vals = oracle.decode_array(fmt, pats)
        finite = np.isfinite(vals)
        back = oracle.encode_array(fmt, vals[finite]).astype(np.uint32)
        assert np.array_equal(back, pats[finite]), fmt


def test_e4m3_saturates_and_ties_to_even():
    enc = lambda v: oracle.encode(E4M3, v)
    assert enc(448.0) == 0x7E and enc(460.0) == 0x7E and enc(1e6) == 0x7E
    assert enc(-1e6) == 0xFE and enc(float("inf")) == 0x7E
    # 2^-10 is halfway between 0 and the smallest subnormal 2^-9: tie -> 0 (even)
    assert enc(2.0 ** -10) == 0x00
    # 3 * 2^-10 is halfway between 0x01 and 0x02: tie -> 0x02 (even)
    assert enc(3 * 2.0 ** -10) == 0x02
    # 1.0625 is halfway between 1.0 (0x38) and 1.125 (0x39): tie -> 0x38
    assert enc(1.0625) == 0x38 and enc(1.1875) == 0x3A


@pytest.mark.parametrize("x,code", [
    # normalised value / scale, with scale = 3.5/448 = 2^-7 exactly
    (3.5, 0x7E),                     # 448
    (1.0, 0x70),                     # 128 = 2^7 -> exponent field 14
    (0.010009765625, 0x3A),          # bf16(0.01) / 2^-7 = 1.28125 -> 1.25
    (-0.5, 0xE8),                    # -64
    (2.0 ** -12, 0x10),              # 2^-5 -> exponent field 2
    (2.0 ** -16, 0x01),              # 2^-9, the smallest subnormal
    (2.0 ** -17, 0x00),              # 2^-10: tie -> 0
    (3 * 2.0 ** -17, 0x02),          # 3*2^-10: tie -> 2
])
def test_e4m3_worked_values(x, code):
    scale = 3.5 / 448
    assert scale == 2.0 ** -7
    assert oracle.encode(E4M3, x / scale) == code
