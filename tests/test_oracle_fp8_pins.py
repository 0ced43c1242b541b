"""Pins for the oracle's FP8 E4M3 functions (the FP8 article's E4M3 GEMM and
FP8 KV cache, per-tensor or per-row scaling).

Independent references: the OCP E4M3 values in tests/golden/e4m3_spec.json,
torch's own float8_e4m3fn conversion (an implementation unrelated to the
oracle's), a brute-force nearest-code search, exact rational arithmetic and
numpy's float64 matmul on exactly representable products.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import qgemm_inputs as qi

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
CODES = np.arange(256, dtype=np.uint8)
FINITE = np.array([c for c in range(256) if c & 0x7f != 0x7f], np.uint8)


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_spec_values():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_spec.json")))
    dec = oracle.e4m3_to_f64(CODES)
    for v in g["values"]:
        c = int(v["code"], 16)
        assert dec[c] == v["value"] and np.signbit(dec[c]) == np.signbit(v["value"]), v
        assert int(oracle.f64_to_e4m3(np.array([v["value"]]))[0]) == c, v
    for c in g["nan_codes"]:
        assert np.isnan(dec[int(c, 16)])
    assert np.isnan(dec).sum() == 2


def test_e4m3_decode_against_torch():
    ours, ref = oracle.e4m3_to_f64(CODES), torch_decode(CODES)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_monotone_and_round_trip():
    v = oracle.e4m3_to_f64(np.arange(0x7f, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)
    assert np.array_equal(oracle.f64_to_e4m3(oracle.e4m3_to_f64(FINITE)), FINITE)


def test_e4m3_encode_against_torch_and_ties():
    r = np.random.default_rng(11)
    mags = np.concatenate([r.uniform(0, 448, 20000), np.exp(r.uniform(np.log(1e-4), np.log(448), 20000)),
                           r.uniform(0, 2 ** -6, 2000)])
    x = mags * r.choice([-1.0, 1.0], mags.size)
    pos = oracle.e4m3_to_f64(np.arange(0x7f, dtype=np.uint8))
    mid = (0.5 * (pos[:-1] + pos[1:])).astype(np.float32)    # exact ties between neighbours
    # fp32 inputs, as the quantizer encodes (torch converts wider inputs to fp32 first)
    x = np.concatenate([x.astype(np.float32), mid, -mid, np.nextafter(mid, np.float32(0)),
                        np.nextafter(mid, np.float32(1e9)), pos.astype(np.float32)])
    x = x[np.abs(x) <= 448]
    assert np.array_equal(oracle.f64_to_e4m3(x.astype(np.float64)),
                          torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    # ties went to the even code (mantissa bit 0 clear)
    t = oracle.f64_to_e4m3(mid.astype(np.float64))
    assert np.all(t & 1 == 0)


def test_e4m3_saturates():
    assert oracle.f64_to_e4m3(np.array([448.0, 449.0, 464.0, 1e4, -1e9])).tolist() == [0x7e, 0x7e, 0x7e, 0x7e, 0xfe]


def nearest_code(t):
    """Brute force over every finite code: nearest value, ties to the even code."""
    vals = oracle.e4m3_to_f64(FINITE)
    d = np.abs(vals - t)
    best = np.flatnonzero(d == d.min())
    best = [int(FINITE[i]) for i in best]
    even = [c for c in best if c & 1 == 0]
    return (even or best)[0], d.min()


def test_quant_fp8_hand_rows():
    Q, S = oracle.quant_fp8(np.array([[448, 1, -448, 0], [2, 1, 0, -0.5]], np.float16))
    assert Q[0].tolist() == [0x7e, 0x38, 0xfe, 0x00] and S[0] == 1.0
    # row 2: amax 2, m = 224: t = 448, 224, 0, -112
    assert Q[1].tolist() == [0x7e, 0x76, 0x00, 0xee] and S[1] == np.float32(2) / np.float32(448)
    Qz, Sz = oracle.quant_fp8(np.zeros((2, 5), np.float16))
    assert not Qz.any() and not Sz.any()
    # per tensor: one amax (8) for both rows, m = 56
    Qt, St = oracle.quant_fp8(np.array([[1, 2], [4, -8]], np.float16), per_row=False)
    assert St.tolist() == [np.float32(8) / np.float32(448)]
    assert oracle.e4m3_to_f64(Qt).tolist() == [[56.0, 112.0], [224.0, -448.0]]


@pytest.mark.parametrize("per_row", [True, False])
def test_quant_fp8_nearest_code_by_brute_force(per_row):
    X = qi.kv_problem(1, 6, 128, 33).reshape(6, 128)
    Q, S = oracle.quant_fp8(X, per_row=per_row)
    for r in range(X.shape[0]):
        s = S[r if per_row else 0]
        amax = np.float32(np.abs(X[r] if per_row else X).astype(np.float32).max())
        assert s == amax / np.float32(448)
        m = np.float32(448) / amax
        for c in range(0, 128, 7):
            t = min(max(np.float32(X[r, c]) * m, np.float32(-448)), np.float32(448))
            code, _ = nearest_code(float(t))
            assert Q[r, c] == code


def test_dequant_fp8_hand_and_bound():
    X = oracle.dequant_fp8(np.array([[0x38, 0x7e, 0x01, 0xb8]], np.uint8), np.array([0.5], np.float32))
    assert X.astype(np.float64).tolist() == [[0.5, 224.0, 2.0 ** -10, -0.5]]
    # round trip: |x - x^| <= half an E4M3 step at |x| (relative 2^-4 in the normal range) + fp16 rounding
    X = np.random.default_rng(5).uniform(-0.5, 0.5, (64, 128)).astype(np.float16)
    Q, S = oracle.quant_fp8(X)
    Xh = oracle.dequant_fp8(Q, S).astype(np.float64)
    x = X.astype(np.float64)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, S[:, None].astype(np.float64) * 2.0 ** -10) * 1.001 + 2.0 ** -11 * np.abs(x)
    assert np.all(np.abs(Xh - x) <= bound + 1e-7)


def test_dequant_fp8_rounds_in_fp32_then_fp16():
    """Code 0x3D is 1.625 (exponent field 7, mantissa 101). With s = 5164741 * 2^-23 the exact
    product is 67141633 * 2^-26 = 1.000488296..., 8392704.125 fp32 spacings of 2^-23: fl32 gives
    exactly 1 + 2^-11, halfway between the fp16 values 1 and 1 + 2^-10, and the fp16 conversion
    (ties to even) gives 1.0, where one rounding of the exact product would give 1 + 2^-10.
    Same for the negative code 0xBD."""
    s = np.float32(5164741 * 2.0 ** -23)
    assert Fraction(float(s)) == Fraction(5164741, 2 ** 23)
    X = oracle.dequant_fp8(np.array([[0x3D, 0xBD, 0x38]], np.uint8), np.array([s], np.float32))
    assert X.astype(np.float64).tolist() == [[1.0, -1.0, float(np.float16(float(s)))]]


def test_fp8_gemm_hand():
    enc = lambda v: oracle.f64_to_e4m3(np.array(v, np.float64))
    A = enc([[1, 2], [-0.5, 448]])
    W = enc([[1, 1], [0.25, -3]])                  # rows = output columns
    sa = np.array([1, 0.5], np.float32)
    sw = np.array([2, 1], np.float32)
    Y, Y64 = oracle.fp8_gemm(A, W, sa, sw, want_f64=True)
    acc = [[Fraction(3), Fraction(-23, 4)], [Fraction(895, 2), Fraction(-10753, 8)]]
    want = [[float(acc[m][n] * Fraction(float(sa[m])) * Fraction(float(sw[n]))) for n in range(2)] for m in range(2)]
    assert Y64.tolist() == want
    assert Y.tolist() == np.array(want).astype(np.float16).tolist()


def test_fp8_gemm_against_numpy_and_closed_form():
    r = np.random.default_rng(21)
    M, N, K = 7, 9, 320
    A = r.choice(FINITE, (M, K)).astype(np.uint8)
    W = r.choice(FINITE, (N, K)).astype(np.uint8)
    sa = r.uniform(0.001, 0.01, M).astype(np.float32)
    sw = r.uniform(0.001, 0.01, N).astype(np.float32)
    _, Y64 = oracle.fp8_gemm(A, W, sa, sw, want_f64=True)
    acc = torch_decode(A) @ torch_decode(W).T          # exact: every product and partial sum is
    want = acc * sa.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    assert np.array_equal(Y64, want)
    ms, ns = np.array([0, 6, 3], np.int32), np.array([8, 0, 4], np.int32)
    Yf = oracle.fp8_gemm(A, W, sa, sw)
    assert np.array_equal(oracle.fp8_gemm_at(A, W, sa, sw, ms, ns), Yf[ms, ns])
    # closed form: A = 1.5 everywhere, W = -2 everywhere -> acc = -3 K
    A1 = np.full((2, K), 0x3c, np.uint8)
    W1 = np.full((3, K), 0xc0, np.uint8)
    _, Y1 = oracle.fp8_gemm(A1, W1, np.ones(1, np.float32), np.ones(1, np.float32), want_f64=True)
    assert np.all(Y1 == -3.0 * K)
    # per-tensor scale (one value) equals that value broadcast per row / column
    Yt = oracle.fp8_gemm(A, W, sa[:1], sw[:1])
    Yb = oracle.fp8_gemm(A, W, np.full(M, sa[0], np.float32), np.full(N, sw[0], np.float32))
    assert np.array_equal(Yt, Yb)
