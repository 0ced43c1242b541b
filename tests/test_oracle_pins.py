"""Pins for the CPU oracle.

Each test ties the oracle to something other than itself: values worked by
hand (tests/golden/*.json, each citing its page), exact rational arithmetic
(fractions.Fraction), closed forms, invariants, and library routines (numpy's
float16 conversion, numpy integer matmul and stable argsort, math.erf,
scipy's softmax).  A plausible slip in the oracle -- a swapped nibble, a
wrong group index, a transposed operand, a dropped bias, half-away rounding
instead of half-even, a divide instead of a multiply, double rounding --
fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle
import qgemm_inputs as qi

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bits16(a):
    return np.asarray(a, np.float16).view(np.uint16)


def unpack_numpy(Wb, K, N):
    """Natural int4 decode by numpy arithmetic shifts (independent of the oracle):
    even column = low nibble, odd column = high nibble, two's complement."""
    b = Wb.reshape(K, N // 2)
    lo = (b.astype(np.uint8) << 4).view(np.int8) >> 4
    hi = b.view(np.int8) >> 4
    q = np.empty((K, N), np.int8)
    q[:, 0::2] = lo
    q[:, 1::2] = hi
    return q


def pack_numpy(q):
    """Pack int8 values in [-8, 7] [K][N] into natural bytes (test-side helper)."""
    u = (q.astype(np.int16) & 15).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


# ------------------------------------------------------------------ binary16

def test_f16_to_f64_exhaustive():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    got = oracle.f16_to_f64(h.view(np.float16))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f64_to_f16_against_numpy():
    r = qi.rng(1)
    finite = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    finite = finite[np.isfinite(finite)].astype(np.float64)
    finite = np.unique(finite)
    mids = (finite[:-1] + finite[1:]) / 2  # exact ties between neighbours
    quarter = finite[:-1] + (finite[1:] - finite[:-1]) / 4
    rand = np.concatenate([
        r.standard_normal(200000),
        r.standard_normal(20000) * 1e-6,   # subnormal range
        r.standard_normal(20000) * 3e4,    # near overflow
        np.array([65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -25, 2.0 ** -26, 0.0, -0.0]),
    ])
    x = np.concatenate([finite, mids, quarter, rand])
    got = bits16(oracle.f64_to_f16(x))
    ref = bits16(x.astype(np.float16))
    assert np.array_equal(got, ref)


def test_f64_to_f16_rounds_once():
    # Just above the midpoint between 1 and 1 + 2^-10: one rounding goes up;
    # rounding to fp32 first would land on the midpoint and then go down.
    x = 1.0 + 2.0 ** -11 + 2.0 ** -40
    assert float(oracle.f64_to_f16([x])[0]) == 1.0 + 2.0 ** -10
    assert float(oracle.f64_to_f16([1.0 + 2.0 ** -11])[0]) == 1.0  # tie -> even


# ------------------------------------------------------------------ int4

def test_int4_decode_exhaustive():
    b = np.arange(256, dtype=np.uint8).reshape(256, 1)
    for i in range(256):
        got = oracle.int4_unpack(b[i], 1, 2)[0]
        assert list(got) == list(unpack_numpy(b[i], 1, 2)[0])


def test_int4_hand_bytes():
    g = golden("w4a16_hand_4x4.json")
    packed = np.array([int(h, 16) for h in g["packed_hex"].split()], np.uint8)
    assert oracle.int4_unpack(packed, 4, 4).tolist() == g["Q"]
    assert pack_numpy(np.array(g["Q"], np.int8)).ravel().tolist() == packed.tolist()


# ------------------------------------------------------------------ W4A16

def test_w4a16_hand_4x4():
    g = golden("w4a16_hand_4x4.json")
    packed = np.array([int(h, 16) for h in g["packed_hex"].split()], np.uint8).reshape(4, 2)
    A = np.array(g["A"], np.float16)
    S = np.array(g["S"], np.float16)
    Y = oracle.w4a16(A, packed, S, g["G"])
    assert Y.astype(np.float64).tolist() == g["Y"]


def exact_w4a16(A, q, S, G):
    M, K = A.shape
    N = q.shape[1]
    out = np.empty((M, N), object)
    for m in range(M):
        for n in range(N):
            out[m, n] = sum(Fraction(float(A[m, k])) * int(q[k, n]) * Fraction(float(S[k // G, n]))
                            for k in range(K))
    return out


@pytest.mark.parametrize("seed", range(6))
def test_w4a16_brute_force_tiny(seed):
    r = qi.rng(50 + seed)
    M = int(r.integers(1, 5))
    N = 2 * int(r.integers(1, 3))
    G = int(r.choice([1, 2, 4]))
    K = G * int(r.integers(1, 9 // G + 1))
    A, Wb, S = qi.w4a16_problem(M, K, N, G, 60 + seed)
    q = unpack_numpy(Wb, K, N)
    ex = exact_w4a16(A, q, S, G)
    Y, Y64 = oracle.w4a16(A, Wb, S, G, want_f64=True)
    ref64 = np.array([[float(v) for v in row] for row in ex])
    assert np.allclose(Y64, ref64, rtol=1e-14, atol=0)
    assert np.array_equal(bits16(Y), bits16(ref64.astype(np.float16)))


def test_w4a16_all_16_nibbles_brute_force():
    # every nibble value in every column parity, K spanning two groups
    K, N, G, M = 32, 4, 16, 3
    q = np.array([[((k * 5 + n * 3) % 16) - 8 for n in range(N)] for k in range(K)], np.int8)
    assert set(np.unique(q)) == set(range(-8, 8))
    A = qi.activations(M, K, 71)
    S = qi.w4a16_weights(K, N, G, 72)[1]
    Y, Y64 = oracle.w4a16(A, pack_numpy(q), S, G, want_f64=True)
    ex = exact_w4a16(A, q, S, G)
    ref64 = np.array([[float(v) for v in row] for row in ex])
    assert np.allclose(Y64, ref64, rtol=1e-14, atol=0)
    assert np.array_equal(bits16(Y), bits16(ref64.astype(np.float16)))


def test_w4a16_equal_scales_is_integer_matmul():
    M, K, N, G = 8, 256, 64, 64
    A, Wb, _ = qi.w4a16_problem(M, K, N, G, 80)
    s = np.float16(0.0137)
    S = np.full((K // G, N), s, np.float16)
    Y = oracle.w4a16(A, Wb, S, G)
    # A is a multiple of 2^-24, so A * 2^24 is integral: an exact int64 matmul
    Ai = (A.astype(np.float64) * 2.0 ** 24).astype(np.int64)
    P = Ai @ unpack_numpy(Wb, K, N).astype(np.int64)
    ref = np.array([[float(Fraction(int(v), 2 ** 24) * Fraction(float(s))) for v in row] for row in P])
    assert np.array_equal(bits16(Y), bits16(ref.astype(np.float16)))


def test_w4a16_group_isolation():
    M, K, N, G = 4, 512, 32, 128
    A, Wb, S = qi.w4a16_problem(M, K, N, G, 81)
    A2 = np.zeros_like(A)
    A2[:, 256:384] = A[:, 256:384]  # only group 2 active
    S2 = S.copy()
    S2[[0, 1, 3]] = np.float16(0.5)  # change every other group's scales
    Y1 = oracle.w4a16(A2, Wb, S, G)
    Y2 = oracle.w4a16(A2, Wb, S2, G)
    assert np.array_equal(bits16(Y1), bits16(Y2))
    S3 = S.copy()
    S3[2] = np.float16(0.5)
    assert not np.array_equal(bits16(oracle.w4a16(A2, Wb, S3, G)), bits16(Y1))


def test_w4a16_k_split_additivity_and_linearity():
    M, K, N, G = 3, 512, 64, 128
    A, Wb, S = qi.w4a16_problem(M, K, N, G, 82)
    _, Y = oracle.w4a16(A, Wb, S, G, want_f64=True)
    _, Y1 = oracle.w4a16(A[:, :256], Wb[:256], S[:2], G, want_f64=True)
    _, Y2 = oracle.w4a16(A[:, 256:], Wb[256:], S[2:], G, want_f64=True)
    assert np.allclose(Y, Y1 + Y2, rtol=1e-12, atol=1e-12)
    _, Yd = oracle.w4a16((A.astype(np.float32) * 2).astype(np.float16), Wb, S, G, want_f64=True)
    assert np.array_equal(Yd, 2 * Y)
    # transposing the roles of rows and columns changes the answer (orientation check)
    A4 = qi.activations(4, 4, 83)
    g = golden("w4a16_hand_4x4.json")
    packed = np.array([int(h, 16) for h in g["packed_hex"].split()], np.uint8).reshape(4, 2)
    qT = np.array(g["Q"], np.int8).T.copy()
    S = np.array(g["S"], np.float16)
    assert not np.array_equal(bits16(oracle.w4a16(A4, packed, S, 2)),
                              bits16(oracle.w4a16(A4, pack_numpy(qT), S, 2)))


def test_w4a16_zero_weights():
    A, _, S = qi.w4a16_problem(2, 256, 32, 128, 84)
    Y = oracle.w4a16(A, np.zeros((256, 16), np.uint8), S, 128)
    assert not np.any(Y.astype(np.float32))


def test_w4a16_sampled_matches_full():
    M, K, N, G = 16, 512, 512, 128
    A, Wb, S = qi.w4a16_problem(M, K, N, G, 100)
    Y = oracle.w4a16(A, Wb, S, G)
    ms, ns = qi.sample_positions(M, N, 300, 5)
    y = oracle.w4a16_at(A, Wb, S, G, ms, ns)
    assert np.array_equal(bits16(y), bits16(Y[ms, ns]))


def test_w4a16_output_scale_statistics():
    # y = sum_k a_k w_k with a ~ N(0,1), w = q s: std(y) = sqrt(K E[q^2] E[s^2])
    M, K, N, G = 8, 4096, 1024, 128
    A, Wb, S = qi.w4a16_problem(M, K, N, G, 85)
    Y = oracle.w4a16(A, Wb, S, G).astype(np.float64)
    eq2 = sum(v * v for v in range(-8, 8)) / 16
    es2 = (0.005 ** 2 + 0.005 * 0.02 + 0.02 ** 2) / 3
    assert abs(Y.std() / math.sqrt(K * eq2 * es2) - 1) < 0.05


# ------------------------------------------------------------------ fragment layout

def test_prepack_layout_is_a_bijection():
    K, N = 256, 256
    idx = np.array([[oracle.frag_nibble_index(K, k, n) for n in range(N)] for k in range(K)])
    assert np.array_equal(np.sort(idx.ravel()), np.arange(K * N))


def test_prepack_layout_hand_positions():
    K = 256
    cases = {  # (k, n) -> nibble index, worked from the layout definition
        (0, 0): 0, (2, 0): 1, (4, 0): 2, (6, 0): 3, (1, 0): 4, (7, 0): 7,
        (32, 0): 8, (8, 0): 512, (0, 1): 32, (0, 16): 2048,
        (128, 0): 16384, (0, 128): 32768, (255, 255): 32768 + 8192 * 2 + 7 * 2048 + 2 * ((15 + 48) * 16 + 12) + 7,
    }
    for (k, n), want in cases.items():
        assert oracle.frag_nibble_index(K, k, n) == want, (k, n)


def test_prepack_offset_binary_values():
    K, N = 128, 128
    assert not oracle.w4a16_prepack(np.full((K, N // 2), 0x88, np.uint8), K, N).any()
    assert (oracle.w4a16_prepack(np.full((K, N // 2), 0x77, np.uint8), K, N) == 0xFF).all()
    assert (oracle.w4a16_prepack(np.zeros((K, N // 2), np.uint8), K, N) == 0x88).all()


def test_prepack_moves_every_nibble():
    K, N = 256, 384
    Wb = qi.w4a16_weights(K, N, 128, 86)[0]
    F = oracle.w4a16_prepack(Wb, K, N)
    q = unpack_numpy(Wb, K, N)
    nib = np.empty(K * N, np.int64)
    nib[0::2] = F & 15
    nib[1::2] = F >> 4
    for k in range(0, K, 7):
        for n in range(0, N, 5):
            assert nib[oracle.frag_nibble_index(K, k, n)] == q[k, n] + 8


@pytest.mark.parametrize("K,N", [(200, 136), (8, 8), (136, 264), (1000, 24)])
def test_prepack_ragged_is_the_zero_padded_layout(K, N):
    """K and N that are not multiples of 128 (GEMM plugin page, class summary: scales
    [ceil(K/G), N], fragment rows ceil(N/128) * ceil(K/64) * 8) pad to whole tiles: the
    bytes equal those of the matrix extended with weight-0 rows and columns to the next
    multiples of 128, and the padding holds weight 0."""
    Wb = qi.w4a16_weights(K, N, 32, 87 + K + N)[0]
    Kp, Np = -(-K // 128) * 128, -(-N // 128) * 128
    Wp = np.zeros((Kp, Np // 2), np.uint8)  # nibble 0 = weight 0 (two's complement)
    Wp[:K, :N // 2] = Wb
    F = oracle.w4a16_prepack(Wb, K, N)
    assert F.size == Kp * Np // 2
    assert np.array_equal(F, oracle.w4a16_prepack(Wp, Kp, Np))
    idx = np.array([[oracle.frag_nibble_index(K, k, n) for n in range(N)] for k in range(K)]).ravel()
    assert np.unique(idx).size == K * N and idx.max() < Kp * Np
    nib = np.empty(Kp * Np, np.int64)
    nib[0::2] = F & 15
    nib[1::2] = F >> 4
    pad = np.ones(Kp * Np, bool)
    pad[idx] = False
    assert np.all(nib[pad] == 8)
    q = unpack_numpy(Wb, K, N)
    assert np.array_equal(nib[idx], (q.ravel() + 8))


@pytest.mark.parametrize("K,G", [(40, 32), (72, 64), (136, 128), (24, 32)])
def test_w4a16_partial_last_group_exact(K, G):
    """K not a multiple of G: scales have ceil(K/G) rows and the last group covers the
    remaining K % G rows (exact rationals, one fp16 rounding)."""
    M, N = 3, 8
    A, Wb, S = qi.w4a16_problem(M, K, N, G, 88 + K)
    assert S.shape == (-(-K // G), N)
    q = unpack_numpy(Wb, K, N)
    ex = exact_w4a16(A, q, S, G)
    Y, Y64 = oracle.w4a16(A, Wb, S, G, want_f64=True)
    ref64 = np.array([[float(v) for v in row] for row in ex])
    assert np.allclose(Y64, ref64, rtol=1e-14, atol=0)
    assert np.array_equal(bits16(Y), bits16(ref64.astype(np.float16)))
    # the last group's scales act on exactly the last K - (ceil(K/G) - 1) G rows
    S2 = S.copy()
    S2[-1] = np.float16(0.0)
    _, Y64b = oracle.w4a16(A, Wb, S2, G, want_f64=True)
    k0 = (S.shape[0] - 1) * G
    Ab = A.copy()
    Ab[:, k0:] = np.float16(0.0)
    _, Y64c = oracle.w4a16(Ab, Wb, S, G, want_f64=True)
    assert np.allclose(Y64b, Y64c, rtol=1e-14, atol=1e-300)


# ------------------------------------------------------------------ int8 quant / dequant

def test_quant_hand_rows():
    g = golden("quant_hand.json")
    for row in g["rows"]:
        x = np.array([row["x"]], np.float16)
        Q, S = oracle.quant_sym_int8(x)
        assert Q[0].tolist() == row["q"]
        s_ref = Fraction(row["s_fraction"]) if "s_fraction" in row else Fraction(row["s"])
        assert Fraction(float(S[0])) == s_ref


def test_dequant_hand():
    g = golden("quant_hand.json")["dequant"]
    X = oracle.dequant_sym_int8(np.array([g["q"]], np.int8), np.array([g["s"]], np.float32))
    assert X[0].astype(np.float64).tolist() == g["x"]


def test_dequant_rounds_in_fp32_then_fp16():
    g = golden("quant_hand.json")["dequant_two_roundings"]
    s = Fraction(g["s_fraction"])
    s32 = np.float32(float(s))
    assert Fraction(float(s32)) == s
    X = oracle.dequant_sym_int8(np.array([g["q"]], np.int8), np.array([s32], np.float32))
    assert X[0].astype(np.float64).tolist() == g["x"]


def round_half_even(fr):
    fl = math.floor(fr)
    d = fr - fl
    if d > Fraction(1, 2) or (d == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def round_to_f32(fr):
    """IEEE binary32 round-to-nearest-even of an exact rational (normal range only)."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e <= 127
    ulp = Fraction(2) ** (e - 23)
    return sign * round_half_even(a / ulp) * ulp


def quant_multiply_form(xs):
    """Codes and scale of one row by the multiply form, in exact rationals: m = fl32(127/amax),
    q = clamp(rne(fl32(x*m)), -127, 127), s = fl32(amax/127) (interview page, answer step 1)."""
    xs = [Fraction(float(v)) for v in xs]
    amax = max(abs(v) for v in xs)
    if amax == 0:
        return [0] * len(xs), Fraction(0)
    m = round_to_f32(Fraction(127) / amax)
    q = [max(-127, min(127, round_half_even(round_to_f32(v * m)))) for v in xs]
    return q, round_to_f32(amax / 127)


def test_round_to_f32_matches_hardware_float32():
    r = qi.rng(89)
    for v in np.concatenate([r.standard_normal(300), r.uniform(-1e4, 1e4, 300)]):
        a, b = np.float32(v), np.float32(r.uniform(0.5, 2.0))
        assert Fraction(float(a * b)) == round_to_f32(Fraction(float(a)) * Fraction(float(b)))
        assert Fraction(float(a / b)) == round_to_f32(Fraction(float(a)) / Fraction(float(b)))


def test_quant_against_exact_rationals():
    X = qi.kv_problem(1, 64, 128, 90).reshape(64, 128)
    X[3, 5] = np.float16(0.0)
    X[7, :] = np.float16(0.0)
    Q, S = oracle.quant_sym_int8(X)
    for r in range(X.shape[0]):
        q, s = quant_multiply_form(X[r])
        assert Q[r].tolist() == q
        assert Fraction(float(S[r])) == s


def test_quant_kv_block_multiply_form_not_division():
    """The full [32, 2048, 128] KV block of the workload: the elements where the multiply form
    and division by the stored scale give different codes (a few hundred of 8.4 M) carry the
    multiply form's codes, derived exactly for each of them."""
    X = qi.kv_problem(32, 2048, 128, 103).reshape(-1, 128)
    Q, S = oracle.quant_sym_int8(X)
    x32 = X.astype(np.float32)
    amax = np.abs(x32).max(axis=1, keepdims=True)
    m = np.float32(127.0) / amax
    s = amax / np.float32(127.0)
    by_mul = np.clip(np.rint(x32 * m), -127, 127)
    by_div = np.clip(np.rint(x32 / s), -127, 127)
    rows, cols = np.nonzero(by_mul != by_div)
    assert len(rows) > 300
    picks = list(zip(rows.tolist(), cols.tolist()))
    r = qi.rng(88)
    picks += list(zip(r.integers(0, X.shape[0], 300).tolist(), r.integers(0, 128, 300).tolist()))
    for (i, c) in picks:
        xs = [Fraction(float(v)) for v in X[i]]
        a = max(abs(v) for v in xs)
        mm = round_to_f32(Fraction(127) / a)
        qe = max(-127, min(127, round_half_even(round_to_f32(xs[c] * mm))))
        assert int(Q[i, c]) == qe
    assert np.array_equal(Q[rows, cols], by_mul[rows, cols].astype(np.int8))
    assert not np.any(Q[rows, cols] == by_div[rows, cols].astype(np.int8))


def test_quant_error_bounds_and_statistics():
    X = qi.kv_problem(4, 2048, 128, 91).reshape(-1, 128)
    Q, S = oracle.quant_sym_int8(X)
    x = X.astype(np.float64)
    s = S.astype(np.float64)[:, None]
    err = np.abs(x - Q.astype(np.float64) * s)
    assert np.all(err <= s * (0.5 + 2.0 ** -14))
    mse_ratio = np.mean(err ** 2) / np.mean(s ** 2 / 12)
    assert 0.95 < mse_ratio < 1.05
    # the KV demo's own acceptance bar: round-trip MSE below 1e-4
    Xh = oracle.dequant_sym_int8(Q, S).astype(np.float64)
    assert np.mean((x - Xh) ** 2) < 1e-4
    ulp = np.spacing(np.abs(Xh).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(x - Xh) <= s * (0.5 + 2.0 ** -14) + ulp / 2)
    # extremes map to +-127 exactly, never -128
    amax_idx = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(Q[np.arange(len(Q)), amax_idx]) == 127)
    assert Q.min() >= -127


def test_dequant_unit_scale_identity():
    q = np.arange(-127, 128, dtype=np.int8).reshape(1, -1)
    X = oracle.dequant_sym_int8(q, np.ones(1, np.float32))
    assert X.astype(np.int32).tolist() == q.astype(np.int32).tolist()


# ------------------------------------------------------------------ W8A8

def test_w8a8_acc_hand():
    g = golden("w8a8_hand_4x4.json")
    acc = oracle.w8a8_acc(np.array(g["qa"], np.int8), np.array(g["qw"], np.int8))
    assert acc.tolist() == g["acc"]


def test_w8a8_acc_closed_forms_and_numpy():
    K = 4096
    a = np.full((2, K), 127, np.int8)
    w = np.stack([np.full(K, 127, np.int8), np.full(K, -127, np.int8)])
    assert oracle.w8a8_acc(a, w).tolist() == [[K * 16129, -K * 16129]] * 2
    r = qi.rng(92)
    A = r.integers(-127, 128, size=(33, 300), dtype=np.int8)
    W = r.integers(-127, 128, size=(17, 300), dtype=np.int8)
    assert np.array_equal(oracle.w8a8_acc(A, W), A.astype(np.int64) @ W.astype(np.int64).T)


def test_w8a8_epilogue_hand():
    g = golden("w8a8_hand_4x4.json")
    qa = np.array(g["qa"], np.int8)
    qw = np.array(g["qw"], np.int8)
    sa = np.array(g["sa"], np.float32)
    sw = np.array(g["sw"], np.float32)
    bias = np.array(g["bias"], np.float16)
    Y = oracle.w8a8_epilogue(qa, qw, sa, sw, bias, 1.0, oracle.EPI_BIAS)
    assert Y.tolist() == g["bias_only_mult1"]
    Y4 = oracle.w8a8_epilogue(qa, qw, sa, sw, bias, 4.0, oracle.EPI_BIAS)
    for r, row in g["bias_only_mult4_rows"].items():
        assert Y4[int(r)].tolist() == row
    Yg = oracle.w8a8_epilogue(qa, qw, sa, sw, bias, 1.0, oracle.EPI_BIAS | oracle.EPI_GELU)
    assert Yg.tolist() == g["bias_gelu_mult1"]
    # without the bias flag the bias is ignored: row 3 (acc = 0) is all zero
    Yn = oracle.w8a8_epilogue(qa, qw, sa, sw, bias, 1.0, 0)
    assert Yn[3].tolist() == [0, 0, 0, 0] and Yn[0].tolist() == [10, 2, -6, 48]
    # saturation on both sides at +-127 (never -128)
    Y16 = oracle.w8a8_epilogue(qa, qw, sa, sw, bias, 16.0, oracle.EPI_BIAS)
    assert Y16[0].tolist() == g["bias_only_mult16_row0"]


def test_w8a8_epilogue_scale_order():
    c = golden("w8a8_hand_4x4.json")["scale_order"]
    sw = np.float32(float(Fraction(c["sw_fraction"])))
    assert Fraction(float(sw)) == Fraction(c["sw_fraction"])
    Y = oracle.w8a8_epilogue(np.array(c["qa"], np.int8), np.array(c["qw"], np.int8),
                             np.array(c["sa"], np.float32), np.array([sw], np.float32), None,
                             c["out_mult"], c["flags"])
    assert Y.tolist() == c["q"]


def gelu_exact(y):
    return 0.5 * y * (1.0 + math.erf(y / math.sqrt(2.0)))


def test_gelu28_against_erf():
    ys = np.concatenate([np.linspace(-10, 10, 40001), [-300.0, -60.0, 60.0, 300.0, 1e-30, -1e-30]])
    ys = ys.astype(np.float32)
    g = oracle.gelu28(ys).astype(np.float64)
    ref = np.array([gelu_exact(float(y)) for y in ys])
    # A&S 7.1.28 bounds |erf error| by 3e-7; evaluating it in fp32 adds rounding
    # that the 16th power amplifies (about 16 x 1.5e-7).  |g error| = |y|/2 * |erf error|.
    assert np.all(np.abs(g - ref) <= 0.5 * (3e-7 + 2.7e-6) * np.abs(ys.astype(np.float64)) + 1e-37)
    mid = np.abs(ys) > 2.0  # p^16 is large there: A&S error plus the rounding of g itself
    assert np.all(np.abs(g - ref)[mid] <= 0.5 * 6e-7 * np.abs(ys[mid].astype(np.float64)) + 1e-37)
    assert oracle.gelu28(np.float32(0.0)) == 0.0
    assert oracle.gelu28(np.float32(6.0)) == 6.0
    big = np.float32(64.5)
    assert oracle.gelu28(big) == big
    assert oracle.gelu28(np.float32(-6.0)) == 0.0


# Abramowitz & Stegun 7.1.28 coefficients as published (decimal) and 1/sqrt(2) to eight places
AS_COEFFS = ["0.0705230784", "0.0422820123", "0.0092705272", "0.0001520143", "0.0002765672", "0.0000430638"]


def gelu28_exact_steps(y):
    """The fixed fp32 sequence of the GELU reading, evaluated step by step in exact rationals with
    one binary32 rounding per operation (fma rounds once)."""
    a1, a2, a3, a4, a5, a6 = (round_to_f32(Fraction(c)) for c in AS_COEFFS)
    y = Fraction(float(y))
    u = round_to_f32(y * round_to_f32(Fraction("0.70710678")))
    a = abs(u)
    p = round_to_f32(a * a6 + a5)
    for c in (a4, a3, a2, a1, Fraction(1)):
        p = round_to_f32(a * p + c)
    for _ in range(4):
        p = round_to_f32(p * p)
    e = round_to_f32(1 - round_to_f32(1 / p))
    if u < 0:
        e = -e
    return round_to_f32(round_to_f32(y / 2) * round_to_f32(1 + e))


def test_gelu28_bits_against_exact_step_evaluation():
    ys = np.concatenate([np.linspace(-5.5, 5.5, 301), qi.rng(85).standard_normal(300) * 2.0])
    ys = ys.astype(np.float32)
    g = oracle.gelu28(ys)
    for y, v in zip(ys, g):
        assert Fraction(float(v)) == gelu28_exact_steps(y), float(y)


def test_w8a8_epilogue_matches_acc_path():
    M, N, K = 16, 24, 64
    X, Wf, bias, om = qi.w8a8_problem(M, N, K, 93)
    qa, sa = oracle.quant_sym_int8(X)
    qw, sw = oracle.quant_sym_int8(Wf)
    Y, acc = oracle.w8a8_epilogue(qa, qw, sa, sw, bias, om, 3, want_acc=True)
    assert np.array_equal(acc, qa.astype(np.int64) @ qw.astype(np.int64).T)
    ms, ns = qi.sample_positions(M, N, 50, 6)
    y, a2 = oracle.w8a8_epilogue_at(qa, qw, sa, sw, bias, om, 3, ms, ns)
    assert np.array_equal(y, Y[ms, ns]) and np.array_equal(a2, acc[ms, ns])
    # dequantized int8 GEMM approximates the fp GEMM (rescale step is right)
    yq = acc * sa[:, None].astype(np.float64) * sw[None, :].astype(np.float64)
    yf = X.astype(np.float64) @ Wf.astype(np.float64).T
    assert np.abs(yq - yf).max() < 0.05 * np.abs(yf).max()


# ------------------------------------------------------------------ MoE

def test_moe_route_hand():
    g = golden("moe_route_hand.json")
    ids, w = oracle.moe_route(np.array(g["logits"], np.float16), g["topK"])
    assert ids.tolist() == g["ids"]
    assert np.allclose(w, np.array(g["w"]), rtol=1e-12, atol=0)
    off, pairs = oracle.moe_permute(ids, g["E"])
    assert off.tolist() == g["offsets"] and pairs.tolist() == g["pairs"]


def test_moe_route_against_numpy():
    logits = qi.moe_problem(256, 8, 8, 8, 8, 94)[1]
    logits[5] = logits[5, 0]  # an all-tie row
    ids, w = oracle.moe_route(logits, 2)
    l = logits.astype(np.float64)
    ref = np.argsort(-l, axis=1, kind="stable")[:, :2]
    assert np.array_equal(ids, ref)
    sel = np.take_along_axis(l, ref, axis=1)
    assert np.allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-13, atol=0)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
    off, pairs = oracle.moe_permute(ids, 8)
    flat = ids.ravel()
    assert np.array_equal(pairs, np.argsort(flat, kind="stable"))
    assert np.array_equal(np.diff(off), np.bincount(flat, minlength=8))


SMALL_MOE = dict(T=6, H=256, I=256, E=4, topK=2, G=128)


def small_moe(seed):
    c = SMALL_MOE
    return qi.moe_problem(c["T"], c["H"], c["I"], c["E"], c["G"], seed)


def act_reference(z, activation):
    """Gate activations from library routines: SiLU = z * expit(z), GELU = z * Phi(z) with
    Phi from scipy's erf, the tanh approximation of GELU, ReLU."""
    if activation == oracle.MOE_GELU_ERF:
        return 0.5 * z * (1.0 + scipy.special.erf(z / math.sqrt(2.0)))
    if activation == oracle.MOE_GELU_TANH:
        return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))
    if activation == oracle.MOE_RELU:
        return np.maximum(z, 0.0)
    return z * scipy.special.expit(z)


def test_moe_activation_values():
    # textbook values at z = 1: SiLU = 1/(1 + 1/e), GELU = Phi(1) (standard normal CDF),
    # the tanh form of GELU, ReLU
    assert abs(oracle.moe_act(1.0, oracle.MOE_SILU) - 0.7310585786300049) < 1e-15
    assert abs(oracle.moe_act(1.0, oracle.MOE_GELU_ERF) - 0.8413447460685429) < 1e-15
    assert abs(oracle.moe_act(1.0, oracle.MOE_GELU_TANH) - 0.8411919906082768) < 1e-15
    assert oracle.moe_act(-1.0, oracle.MOE_RELU) == 0.0 and oracle.moe_act(2.5, oracle.MOE_RELU) == 2.5
    for a in range(4):
        assert oracle.moe_act(0.0, a) == 0.0
    zs = np.concatenate([np.linspace(-12, 12, 601), qi.rng(84).standard_normal(200) * 4])
    for a in range(4):
        got = np.array([oracle.moe_act(z, a) for z in zs])
        assert np.allclose(got, act_reference(zs, a), rtol=1e-13, atol=1e-15), a


@pytest.mark.parametrize("activation", [0, 1, 2, 3])
def test_moe_identical_experts_is_dense_swiglu(activation):
    c = SMALL_MOE
    X, logits, Wg, Wu, Wd, Sg, Su, Sd = small_moe(95)
    for arr in (Wg, Wu, Wd, Sg, Su, Sd):
        arr[1:] = arr[0]
    Y, ids, w = oracle.moe(X, logits, Wg, Wu, Wd, Sg, Su, Sd, c["topK"], c["G"], activation=activation)
    _, g = oracle.w4a16(X, Wg[0], Sg[0], c["G"], want_f64=True)
    _, u = oracle.w4a16(X, Wu[0], Su[0], c["G"], want_f64=True)
    h = (act_reference(g, activation) * u).astype(np.float16)
    _, o = oracle.w4a16(h, Wd[0], Sd[0], c["G"], want_f64=True)
    ref = o.astype(np.float16)
    diff = np.abs(Y.astype(np.float64) - ref.astype(np.float64))
    assert np.all(diff <= np.spacing(np.abs(ref)).astype(np.float64))


def test_moe_distinct_experts_each_weighted_by_its_own_gate():
    """Four tokens, four different experts, top-2 with unequal gate weights: the layer output is
    w[t,0]*o_e0 + w[t,1]*o_e1, each o_e built from W4A16 oracle pieces (gate and up products,
    SiLU, fp16 h, down product) and each weight from the two-logit softmax 1/(1 + e^-(l0 - l1))
    (MoE plugin page, constructor: numExperts, topK)."""
    T, H, I, E, topK, G = 4, 256, 256, 4, 2, 128
    X, _, Wg, Wu, Wd, Sg, Su, Sd = qi.moe_problem(T, H, I, E, G, 87)
    logits = np.array([[2.0, 0.5, -1.0, -3.0],
                       [-1.0, 0.25, 3.0, 1.0],
                       [1.0, -2.0, -0.5, 2.5],
                       [0.5, 1.75, -3.0, 0.75]], np.float16)
    ids_hand = [[0, 1], [2, 3], [3, 0], [1, 3]]
    w_hand = []
    for t, (a, b) in enumerate(ids_hand):
        w0 = 1.0 / (1.0 + math.exp(-(float(logits[t, a]) - float(logits[t, b]))))
        w_hand.append([w0, 1.0 - w0])
    Y, ids, w, Y64 = oracle.moe(X, logits, Wg, Wu, Wd, Sg, Su, Sd, topK, G, want_f64=True)
    assert ids.tolist() == ids_hand
    assert np.allclose(w, np.array(w_hand), rtol=1e-12, atol=0)
    o = []
    for e in range(E):
        _, g = oracle.w4a16(X, Wg[e], Sg[e], G, want_f64=True)
        _, u = oracle.w4a16(X, Wu[e], Su[e], G, want_f64=True)
        h = (g / (1.0 + np.exp(-g)) * u).astype(np.float16)
        o.append(oracle.w4a16(h, Wd[e], Sd[e], G, want_f64=True)[1])
    ref = np.stack([w_hand[t][0] * o[ids_hand[t][0]][t] + w_hand[t][1] * o[ids_hand[t][1]][t]
                    for t in range(T)])
    swapped = np.stack([w_hand[t][1] * o[ids_hand[t][0]][t] + w_hand[t][0] * o[ids_hand[t][1]][t]
                        for t in range(T)])
    tol = 1e-6 * np.abs(ref).max()
    assert np.abs(swapped - ref).max() > 1000 * tol  # the weights really are unequal
    assert np.all(np.abs(Y64 - ref) <= tol)
    assert np.array_equal(bits16(Y), bits16(Y64.astype(np.float16)))


def test_moe_token_permutation_and_expert_removal():
    c = SMALL_MOE
    X, logits, Wg, Wu, Wd, Sg, Su, Sd = small_moe(96)
    Y, ids, w = oracle.moe(X, logits, Wg, Wu, Wd, Sg, Su, Sd, c["topK"], c["G"])
    perm = qi.rng(97).permutation(c["T"])
    Yp, idsp, _ = oracle.moe(X[perm], logits[perm], Wg, Wu, Wd, Sg, Su, Sd, c["topK"], c["G"])
    assert np.array_equal(bits16(Yp), bits16(Y[perm])) and np.array_equal(idsp, ids[perm])
    # relabelling experts relabels ids and leaves the output unchanged
    rel = np.array([2, 0, 3, 1])
    inv = np.argsort(rel)
    Yr, idsr, _ = oracle.moe(X, logits[:, rel], Wg[rel], Wu[rel], Wd[rel], Sg[rel], Su[rel], Sd[rel],
                             c["topK"], c["G"])
    assert np.array_equal(bits16(Yr), bits16(Y)) and np.array_equal(rel[idsr], ids)
    assert np.array_equal(idsr, inv[ids])
    # zero the down projection of the top-1 expert of token 0: only the other remains
    e0 = ids[0, 0]
    Sd0 = Sd.copy()
    Sd0[e0] = np.float16(0.0)
    _, _, _, Y64 = oracle.moe(X, logits, Wg, Wu, Wd, Sg, Su, Sd0, c["topK"], c["G"], tokens=[0],
                              want_f64=True)
    _, _, _, Yfull = oracle.moe(X, logits, Wg, Wu, Wd, Sg, Su, Sd, c["topK"], c["G"], tokens=[0],
                                want_f64=True)
    e1 = ids[0, 1]
    keep = np.ones(c["E"], bool)
    keep[e1] = False
    Sd1 = Sd.copy()
    Sd1[keep] = np.float16(0.0)
    _, _, _, Yonly1 = oracle.moe(X, logits, Wg, Wu, Wd, Sg, Su, Sd1, c["topK"], c["G"], tokens=[0],
                                 want_f64=True)
    assert np.allclose(Y64[0], Yonly1[0], rtol=0, atol=0)
    assert not np.allclose(Yfull[0], Y64[0])


def test_moe_sampled_tokens_match_full():
    c = SMALL_MOE
    X, logits, Wg, Wu, Wd, Sg, Su, Sd = small_moe(98)
    Y, _, _ = oracle.moe(X, logits, Wg, Wu, Wd, Sg, Su, Sd, c["topK"], c["G"])
    Ys, _, _ = oracle.moe(X, logits, Wg, Wu, Wd, Sg, Su, Sd, c["topK"], c["G"], tokens=[4, 1])
    assert np.array_equal(bits16(Ys[[4, 1]]), bits16(Y[[4, 1]]))
