"""Pins of the oracle's reduce + residual add + RMSNorm, FP8 group quant and
QK-norm against hand-worked examples, closed forms, invariants and library
routines (numpy IEEE float32 arithmetic, torch's float64 RMSNorm, torch's FP8
conversion), so that a dropped term, a wrong sign, index or operand in the
oracle fails at least one of them."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import BF16, E4M3, FP16
from tp_all_reduce_amd import workloads

BF16_U = 2.0 ** -8   # unit roundoff of bfloat16


def b16(values, dtype=torch.bfloat16):
    """bit patterns of exactly representable values"""
    t = torch.as_tensor(np.asarray(values, np.float64)).to(dtype)
    assert np.array_equal(t.double().numpy(), np.asarray(values, np.float64)), "not exact"
    return t.view(torch.int16).numpy().view(np.uint16)


def val(bits, fmt=BF16):
    dt = torch.bfloat16 if fmt == BF16 else torch.float16
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dt).double().numpy()


def rand_bits(rng, shape, std=1.0, mean=0.0, dtype=torch.bfloat16):
    x = torch.from_numpy(rng.standard_normal(shape) * std + mean).float().to(dtype)
    return x.view(torch.int16).numpy().view(np.uint16)


def fp32_sum(partials, residual, fmt=BF16):
    """rank-ordered float32 sum using numpy's IEEE float32 adds"""
    acc = val(partials[0], fmt).astype(np.float32)
    for p in partials[1:]:
        acc = (acc + val(p, fmt).astype(np.float32)).astype(np.float32)
    if residual is not None:
        acc = (acc + val(residual, fmt).astype(np.float32)).astype(np.float32)
    return acc


def torch_rms(y, w, eps):
    """torch's own RMSNorm in float64 (a library routine, not the oracle's code)"""
    y = torch.from_numpy(np.asarray(y, np.float64))
    w = torch.from_numpy(np.asarray(w, np.float64))
    return F.rms_norm(y, (y.shape[-1],), w, eps).numpy()


# ------------------------------------------------------------- worked examples
def test_worked_3_4():
    # y = [3, 4] from W=2 partials + residual; rstd = 1/sqrt(12.5 + 1e-6)
    P = [b16([[1.0, 2.0]]), b16([[1.5, 1.0]])]
    R = b16([[0.5, 1.0]])
    norm, res, exact = oracle.ar_rms(P, R, b16([1.0, 1.0]), 1e-6, False)
    assert np.array_equal(val(res), [[3.0, 4.0]])
    e = float(np.float32(1e-6))
    assert np.allclose(exact, [[3 / np.sqrt(12.5 + e), 4 / np.sqrt(12.5 + e)]],
                       rtol=1e-15, atol=0)
    # bf16: 0.8485 lies in [0.5,1) with spacing 2^-8; 1.1314 in [1,2), spacing 2^-7
    assert np.array_equal(val(norm), [[0.84765625, 1.1328125]])


def test_worked_weights_and_gemma():
    P = [b16([[1.0, -1.0]])]
    R = b16([[0.0, 0.0]])
    norm, _, _ = oracle.ar_rms(P, R, b16([2.0, 0.5]), 1e-6, False)
    assert np.array_equal(val(norm), [[2.0, -0.5]])
    # Gemma scales by (1 + w): w = [1, -0.5] gives the same weights 2 and 0.5
    norm_g, _, exact_g = oracle.ar_rms(P, R, b16([1.0, -0.5]), 1e-6, True)
    assert np.array_equal(val(norm_g), [[2.0, -0.5]])
    r = 1 / np.sqrt(1 + float(np.float32(1e-6)))
    assert np.allclose(exact_g, [[2 * r, -0.5 * r]], rtol=1e-15, atol=0)


def test_sum_is_fp32_then_one_rounding():
    # W=2, P0 = 1, P1 = 2^-8, R = 2^-9: the fp32 sum 1 + 3*2^-9 rounds once to
    # 1 + 2^-7; rounding the reduced sum to bf16 first would give 1.0.
    P = [b16([[1.0]]), b16([[2.0 ** -8]])]
    _, res, _ = oracle.ar_rms(P, b16([[2.0 ** -9]]), b16([1.0]), 1e-6, False)
    assert val(res)[0, 0] == 1.0078125


def test_rank_order_is_fixed():
    # 2^24 + 1 ties to 2^24 in fp32, so the ordered sum of {2^24, 1, -2^24} is 0;
    # the order (0, 2, 1) would give 1.
    P = [b16([[2.0 ** 24]]), b16([[1.0]]), b16([[-(2.0 ** 24)]])]
    _, res, _ = oracle.ar_rms(P, b16([[0.0]]), b16([1.0]), 1e-6, False)
    assert val(res)[0, 0] == 0.0
    _, res2, _ = oracle.ar_rms([P[0], P[2], P[1]], b16([[0.0]]), b16([1.0]), 1e-6, False)
    assert val(res2)[0, 0] == 1.0


# ------------------------------------------------------ library-routine pins
@pytest.mark.parametrize("W,T,H,fmt", [(1, 3, 64, BF16), (2, 4, 40, BF16), (4, 5, 128, BF16),
                                       (8, 2, 256, BF16), (3, 3, 96, FP16)])
def test_residual_out_matches_numpy_fp32_sum(W, T, H, fmt):
    rng = np.random.default_rng(10 + W)
    dt = torch.bfloat16 if fmt == BF16 else torch.float16
    P = [rand_bits(rng, (T, H), dtype=dt) for _ in range(W)]
    R = rand_bits(rng, (T, H), dtype=dt)
    _, res, _ = oracle.ar_rms(P, R, rand_bits(rng, (H,), 0.1, 1.0, dt), 1e-6, False, fmt)
    acc = fp32_sum(P, R, fmt)
    ref = torch.from_numpy(acc).to(dt).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(res, ref)


@pytest.mark.parametrize("W,gemma", [(1, False), (2, True), (4, False), (8, True)])
def test_norm_matches_torch_rms_norm_float64(W, gemma):
    rng = np.random.default_rng(20 + W)
    T, H = 6, 192
    P = [rand_bits(rng, (T, H)) for _ in range(W)]
    R = rand_bits(rng, (T, H))
    w = rand_bits(rng, (H,), 0.1, 0.0 if gemma else 1.0)
    eps = 1e-5
    norm, _, exact = oracle.ar_rms(P, R, w, eps, gemma)
    acc = fp32_sum(P, R).astype(np.float64)
    w_eff = val(w) + 1.0 if gemma else val(w)
    ref = torch_rms(acc, w_eff, float(np.float32(eps)))
    np.testing.assert_allclose(exact, ref, rtol=1e-13, atol=1e-300)
    # the 16-bit output is the correctly rounded exact value
    assert np.max(np.abs(val(norm) - exact) / np.maximum(np.abs(exact), 2.0 ** -126)) <= BF16_U


def test_no_residual_equals_zero_residual():
    rng = np.random.default_rng(30)
    P = [rand_bits(rng, (3, 64)) for _ in range(3)]
    w = rand_bits(rng, (64,), 0.1, 1.0)
    a = oracle.ar_rms(P, None, w, 1e-6, False)
    b = oracle.ar_rms(P, np.zeros((3, 64), np.uint16), w, 1e-6, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])
    # without a residual, residual_out is the rank-ordered fp32 sum alone
    assert np.array_equal(val(a[1]), val(b[1]))
    ref = torch.from_numpy(fp32_sum(P, None)).to(torch.bfloat16)
    assert np.array_equal(a[1], ref.view(torch.int16).numpy().view(np.uint16))


# ------------------------------------------------------------- closed forms
@pytest.mark.parametrize("c", [1.0, -1.0])
def test_constant_row_gives_sign_times_weight(c):
    # y = c everywhere: out = w*c/sqrt(c^2 + eps) = sign(c)*w*(1 - 5e-7), which
    # rounds back to w in bf16 (the perturbation is far below half an ulp)
    rng = np.random.default_rng(40)
    H = 256
    w = rand_bits(rng, (H,), 0.1, 1.0)
    P = [b16(np.full((1, H), c / 2)), b16(np.full((1, H), c / 2))]
    norm, res, _ = oracle.ar_rms(P, b16(np.zeros((1, H))), w, 1e-6, False)
    assert np.array_equal(val(norm)[0], c * val(w))


def test_constant_row_at_eps_gives_w_over_sqrt2():
    # c = 2^-10, eps = 2^-20 = c^2: out = w * c / sqrt(2 c^2) = w / sqrt(2)
    H = 64
    rng = np.random.default_rng(41)
    w = rand_bits(rng, (H,), 0.1, 1.0)
    P = [b16(np.full((2, H), 2.0 ** -10))]
    _, _, exact = oracle.ar_rms(P, b16(np.zeros((2, H))), w, 2.0 ** -20, False)
    np.testing.assert_allclose(exact, np.broadcast_to(val(w) / np.sqrt(2), (2, H)), rtol=1e-15)


def test_zero_row_gives_zero():
    H = 64
    w = b16(np.arange(-H // 2, H // 2) / 16.0)
    norm, res, exact = oracle.ar_rms([b16(np.zeros((1, H))), b16(np.zeros((1, H)))],
                                     b16(np.zeros((1, H))), w, 1e-6, False)
    assert np.all(exact == 0) and np.all(val(norm) == 0) and np.all(val(res) == 0)


# --------------------------------------------------------------- invariants
def test_power_of_two_scaling_invariance():
    # eps = 0: scaling every input by 2^k scales residual_out by 2^k exactly and
    # leaves norm_out bit-identical
    rng = np.random.default_rng(50)
    T, H, W = 4, 128, 4
    P = [rand_bits(rng, (T, H)) for _ in range(W)]
    R = rand_bits(rng, (T, H))
    w = rand_bits(rng, (H,), 0.1, 1.0)
    n0, r0, _ = oracle.ar_rms(P, R, w, 0.0, False)
    for k in (-7, 5, 20):
        s = 2.0 ** k
        Ps = [b16(val(p) * s) for p in P]
        n1, r1, _ = oracle.ar_rms(Ps, b16(val(R) * s), w, 0.0, False)
        assert np.array_equal(val(r1), val(r0) * s)
        assert np.array_equal(n1, n0)


def test_sign_symmetry_bit_exact():
    rng = np.random.default_rng(51)
    T, H, W = 3, 96, 3
    P = [rand_bits(rng, (T, H)) for _ in range(W)]
    R = rand_bits(rng, (T, H))
    w = rand_bits(rng, (H,), 0.1, 1.0)
    n0, r0, _ = oracle.ar_rms(P, R, w, 1e-6, True)
    n1, r1, _ = oracle.ar_rms([p ^ np.uint16(0x8000) for p in P], R ^ np.uint16(0x8000), w,
                              1e-6, True)
    assert np.array_equal(val(n1), -val(n0)) and np.array_equal(val(r1), -val(r0))


def test_rank_permutation_within_tolerance():
    rng = np.random.default_rng(52)
    T, H, W = 8, 256, 8
    P = [rand_bits(rng, (T, H)) for _ in range(W)]
    R = rand_bits(rng, (T, H))
    w = rand_bits(rng, (H,), 0.1, 1.0)
    n0, r0, e0 = oracle.ar_rms(P, R, w, 1e-6, False)
    perm = rng.permutation(W)
    n1, r1, e1 = oracle.ar_rms([P[i] for i in perm], R, w, 1e-6, False)
    assert np.max(np.abs(val(n1) - e0) / np.maximum(np.abs(e0), 2.0 ** -126)) <= 4e-3
    # residual_out differs by at most one bf16 ulp of the reassociated sum
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(val(r0)), 2.0 ** -126))) - 7)
    assert np.all(np.abs(val(r1) - val(r0)) <= ulp * 1.0000001)


def test_tokens_of_3d_input_are_numel_over_h():
    # [B, S, H] is processed as B*S independent token rows
    rng = np.random.default_rng(53)
    B, S, H, W = 2, 3, 64, 2
    P = [rand_bits(rng, (B, S, H)) for _ in range(W)]
    R = rand_bits(rng, (B, S, H))
    w = rand_bits(rng, (H,), 0.1, 1.0)
    flat = oracle.ar_rms([p.reshape(B * S, H) for p in P], R.reshape(B * S, H), w, 1e-6, False)
    for b in range(B):
        per = oracle.ar_rms([p[b] for p in P], R[b], w, 1e-6, False)
        assert np.array_equal(per[0], flat[0][b * S:(b + 1) * S])
        assert np.array_equal(per[1], flat[1][b * S:(b + 1) * S])


# ------------------------------------------------------------ FP8 group quant
def test_quant_matches_torch_fp8_conversion():
    rng = np.random.default_rng(60)
    T, H, W, G = 4, 512, 4, 128
    P = [rand_bits(rng, (T, H), 2.0) for _ in range(W)]
    R = rand_bits(rng, (T, H))
    w = rand_bits(rng, (H,), 0.1, 1.0)
    norm, codes, scales, res, exact = oracle.ar_rms_quant(P, R, w, 1e-6, False, G)
    n2, r2, e2 = oracle.ar_rms(P, R, w, 1e-6, False)
    assert np.array_equal(norm, n2) and np.array_equal(res, r2) and np.array_equal(exact, e2)
    grp = exact.reshape(T, H // G, G)
    amax = np.abs(grp).max(axis=-1)
    np.testing.assert_array_equal(scales, (amax / 448.0).astype(np.float32))
    x32 = grp.astype(np.float32)
    v = (x32 / scales[..., None]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes.reshape(T, H // G, G), ref)
    # every group reaches the top code 0x7E in magnitude
    assert np.all((codes.reshape(T, H // G, G) & 0x7F).max(axis=-1) == 0x7E)
    # dequantised values are within 2^-4 relative for normal codes
    deq = oracle.decode_array(E4M3, codes.astype(np.uint32)).reshape(T, H // G, G)
    deq = deq * scales[..., None]
    normal = (codes.reshape(T, H // G, G) & 0x78) != 0
    rel = np.abs(deq - grp)[normal] / np.abs(grp)[normal]
    assert rel.max() <= 2.0 ** -4


def test_quant_zero_group_gives_zero_scale_and_codes():
    H, G = 256, 128
    P = [b16(np.zeros((1, H)))]
    _, codes, scales, _, _ = oracle.ar_rms_quant(P, b16(np.zeros((1, H))), b16(np.ones(H)),
                                                 1e-6, False, G)
    assert np.all(scales == 0) and np.all(codes == 0)


# ----------------------------------------------------------------- QK-norm
def test_qk_worked_example():
    # two shards with one q element each: q = [3 | 4] -> [3, 4]/sqrt(12.5 + eps)
    shards = [b16([[3.0, 1.0, 7.0]]), b16([[4.0, -1.0, 9.0]])]
    q, k, qe, ke = oracle.qknorm(shards, 1, 1, b16([1.0, 1.0]), b16([1.0, 2.0]), 1e-6)
    assert np.array_equal(val(q).reshape(-1), [0.84765625, 1.1328125])
    e = float(np.float32(1e-6))   # eps reaches the method as an fp32 value
    np.testing.assert_allclose(ke.reshape(-1), [1 / np.sqrt(1 + e), -2 / np.sqrt(1 + e)],
                               rtol=1e-15)


@pytest.mark.parametrize("W,q,kv", [(1, 64, 32), (4, 128, 32), (3, 256, 128)])
def test_qk_matches_rms_norm_of_concatenated_heads(W, q, kv):
    rng = np.random.default_rng(70 + W)
    T = 5
    shards = [rand_bits(rng, (T, q + 2 * kv)) for _ in range(W)]
    qw = rand_bits(rng, (W * q,), 0.1, 1.0)
    kw = rand_bits(rng, (W * kv,), 0.1, 1.0)
    eps = 1e-6
    qo, ko, qe, ke = oracle.qknorm(shards, q, kv, qw, kw, eps)
    xs = [val(s) for s in shards]
    qcat = np.concatenate([x[:, :q] for x in xs], axis=1)
    kcat = np.concatenate([x[:, q:q + kv] for x in xs], axis=1)
    e32 = float(np.float32(eps))
    qref = torch_rms(qcat, val(qw), e32)
    kref = torch_rms(kcat, val(kw), e32)
    for r in range(W):
        np.testing.assert_allclose(qe[r], qref[:, r * q:(r + 1) * q], rtol=1e-13)
        np.testing.assert_allclose(ke[r], kref[:, r * kv:(r + 1) * kv], rtol=1e-13)
    # v columns are not read
    shards2 = [s.copy() for s in shards]
    for s in shards2:
        s[:, q + kv:] = 0
    qo2, ko2, _, _ = oracle.qknorm(shards2, q, kv, qw, kw, eps)
    assert np.array_equal(qo, qo2) and np.array_equal(ko, ko2)


def test_workload_generator_is_seeded_and_shaped():
    wl = workloads.WORKLOADS["c2"]
    a = workloads.make_inputs(wl, 4)
    b = workloads.make_inputs(wl, 4)
    assert len(a["partials"]) == 4 and a["partials"][0].shape == (4, 4096)
    assert all(torch.equal(x, y) for x, y in zip(a["partials"], b["partials"]))
    # the partials' spread matches N(0, 0.5)
    s = torch.cat([p.float().reshape(-1) for p in a["partials"]]).std().item()
    assert abs(s - 0.5) < 0.02
    qk = workloads.make_qk_inputs(workloads.WORKLOADS["c5"], 64)
    assert qk["shards"][0].shape == (64, 2048) and qk["q_weight"].shape == (6144,)


# ------------------------------------- reduced sum rounded first (unfused numerics)
def test_round_reduced_worked_case():
    # P = {1, 2^-8}, R = 2^-9: the 16-bit all-reduce gives bf16(1 + 2^-8) = 1.0 (tie to
    # even); adding 2^-9 then rounds back to 1.0 (without rounding first: 1.0078125)
    P = [b16([[1.0]]), b16([[2.0 ** -8]])]
    _, res, _ = oracle.ar_rms(P, b16([[2.0 ** -9]]), b16([1.0]), 1e-6, False, round_reduced=True)
    assert val(res)[0, 0] == 1.0


@pytest.mark.parametrize("W,fmt", [(2, BF16), (4, BF16), (8, BF16), (3, FP16)])
def test_round_reduced_matches_library_rounding(W, fmt):
    rng = np.random.default_rng(90 + W)
    T, H = 5, 160
    dt = torch.bfloat16 if fmt == BF16 else torch.float16
    P = [rand_bits(rng, (T, H), dtype=dt) for _ in range(W)]
    R = rand_bits(rng, (T, H), dtype=dt)
    w = rand_bits(rng, (H,), 0.1, 1.0, dt)
    norm, res, exact = oracle.ar_rms(P, R, w, 1e-5, False, fmt, round_reduced=True)
    s = fp32_sum(P, None, fmt)
    reduced = torch.from_numpy(s).to(dt).float().numpy()          # the 16-bit all-reduce
    acc = (reduced + val(R, fmt).astype(np.float32)).astype(np.float32)
    ref = torch.from_numpy(acc).to(dt).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(res, ref)
    np.testing.assert_allclose(exact, torch_rms(acc.astype(np.float64), val(w, fmt),
                                                float(np.float32(1e-5))), rtol=1e-13)
    # the quant variant carries the same reading
    n2, _, _, r2, e2 = oracle.ar_rms_quant(P, R, w, 1e-5, False, 32, fmt, round_reduced=True)
    assert np.array_equal(r2, res) and np.array_equal(e2, exact)
