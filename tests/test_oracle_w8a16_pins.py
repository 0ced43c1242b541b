"""Pins for the oracle's weight-only int8 GEMM (W8A16) and its int8 fragment layout.

The pages name weight-only int8 (int8 weights, fp16 activations) among the
INT8 configurations they compare (FP8 vs INT8 in TensorRT-LLM, itzkxy.com)
without fixing the scale granularity; the oracle takes fp16 scales per
(K-group, column), with G == K meaning one scale per column.  The pins tie
it to a hand-worked example with a round-half-even tie, exact rational
sums, numpy's integer matmul and the layout's written definition.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import qgemm_inputs as qi

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bits16(a):
    return np.asarray(a, np.float16).view(np.uint16)


def exact(A, W, S, G):
    M, K = A.shape
    N = W.shape[1]
    out = np.empty((M, N), object)
    for m in range(M):
        for n in range(N):
            out[m, n] = sum(Fraction(float(A[m, k])) * int(W[k, n]) * Fraction(float(S[k // G, n]))
                            for k in range(K))
    return out


def test_w8a16_hand():
    with open(os.path.join(GOLDEN, "w8a16_hand_2x4.json")) as f:
        g = json.load(f)
    A = np.array(g["A"], np.float16)
    W = np.array(g["W"], np.int8)
    for case in g["cases"]:
        S = np.array(case["S"], np.float16)
        Y, Y64 = oracle.w8a16(A, W, S, case["G"], want_f64=True)
        assert Y64.tolist() == case["exact"]
        assert Y.astype(np.float64).tolist() == case["Y"]


@pytest.mark.parametrize("seed", range(6))
def test_w8a16_brute_force_tiny(seed):
    r = qi.rng(300 + seed)
    M = int(r.integers(1, 5))
    N = int(r.integers(1, 4))
    G = int(r.choice([1, 2, 4]))
    K = G * int(r.integers(1, 9 // G + 1))
    if seed % 3 == 0:
        G = K  # one scale per column
    A, W, S = qi.w8a16_problem(M, K, N, G, 310 + seed)
    ref64 = np.array([[float(v) for v in row] for row in exact(A, W, S, G)])
    Y, Y64 = oracle.w8a16(A, W, S, G, want_f64=True)
    assert np.allclose(Y64, ref64, rtol=1e-14, atol=0)
    assert np.array_equal(bits16(Y), bits16(ref64.astype(np.float16)))


def test_w8a16_all_256_values_brute_force():
    K, N, G, M = 64, 8, 32, 2
    W = np.array([[((k * 37 + n * 11) % 256) - 128 for n in range(N)] for k in range(K)], np.int8)
    assert set(np.unique(W.astype(np.int32))) == set(range(-128, 128))
    A = qi.activations(M, K, 320)
    S = qi.w8a16_problem(1, K, N, G, 321)[2]
    Y, Y64 = oracle.w8a16(A, W, S, G, want_f64=True)
    ref64 = np.array([[float(v) for v in row] for row in exact(A, W, S, G)])
    assert np.allclose(Y64, ref64, rtol=1e-14, atol=0)
    assert np.array_equal(bits16(Y), bits16(ref64.astype(np.float16)))


def test_w8a16_per_column_is_scaled_integer_matmul():
    # G == K: y = s_n * sum_k a_k w_kn; A * 2^24 is integral, so the sum is an exact int64 matmul
    M, K, N = 6, 512, 96
    A, W, S = qi.w8a16_problem(M, K, N, K, 330)
    Y = oracle.w8a16(A, W, S, K)
    P = (A.astype(np.float64) * 2.0 ** 24).astype(np.int64) @ W.astype(np.int64)
    ref = np.array([[float(Fraction(int(P[m, n]), 2 ** 24) * Fraction(float(S[0, n]))) for n in range(N)]
                    for m in range(M)])
    assert np.array_equal(bits16(Y), bits16(ref.astype(np.float16)))


def test_w8a16_group_isolation_and_orientation():
    M, K, N, G = 3, 512, 32, 128
    A, W, S = qi.w8a16_problem(M, K, N, G, 331)
    A2 = np.zeros_like(A)
    A2[:, 128:256] = A[:, 128:256]  # only group 1 active
    S2 = S.copy()
    S2[[0, 2, 3]] = np.float16(0.25)
    assert np.array_equal(bits16(oracle.w8a16(A2, W, S, G)), bits16(oracle.w8a16(A2, W, S2, G)))
    S3 = S.copy()
    S3[1] = np.float16(0.25)
    assert not np.array_equal(bits16(oracle.w8a16(A2, W, S3, G)), bits16(oracle.w8a16(A2, W, S, G)))
    # a transposed weight matrix gives a different answer
    Wsq = W[:32, :32].copy()
    Asq = A[:, :32].copy()
    Ssq = S[:1, :32].copy()
    assert not np.array_equal(bits16(oracle.w8a16(Asq, Wsq, Ssq, 32)),
                              bits16(oracle.w8a16(Asq, Wsq.T.copy(), Ssq, 32)))


def test_w8a16_linearity_and_k_split():
    M, K, N, G = 3, 512, 64, 128
    A, W, S = qi.w8a16_problem(M, K, N, G, 332)
    _, Y = oracle.w8a16(A, W, S, G, want_f64=True)
    _, Y1 = oracle.w8a16(A[:, :256], W[:256], S[:2], G, want_f64=True)
    _, Y2 = oracle.w8a16(A[:, 256:], W[256:], S[2:], G, want_f64=True)
    assert np.allclose(Y, Y1 + Y2, rtol=1e-12, atol=1e-12)
    _, Yn = oracle.w8a16(A, (-W.astype(np.int16)).clip(-128, 127).astype(np.int8), S, G, want_f64=True)
    mask = (W != -128).all(axis=0)  # columns without -128 negate exactly
    assert np.array_equal(Yn[:, mask], -Y[:, mask])


def test_w8a16_sampled_matches_full():
    M, K, N, G = 16, 512, 384, 64
    A, W, S = qi.w8a16_problem(M, K, N, G, 333)
    Y = oracle.w8a16(A, W, S, G)
    ms, ns = qi.sample_positions(M, N, 300, 6)
    assert np.array_equal(bits16(oracle.w8a16_at(A, W, S, G, ms, ns)), bits16(Y[ms, ns]))


def test_w8a16_output_scale_statistics():
    # a ~ N(0,1), w uniform over [-128, 127], s ~ U[a, b]: std(y) = sqrt(K E[w^2] E[s^2])
    M, K, N, G = 8, 4096, 512, 128
    A, W, S = qi.w8a16_problem(M, K, N, G, 334)
    Y = oracle.w8a16(A, W, S, G).astype(np.float64)
    ew2 = sum(v * v for v in range(-128, 128)) / 256
    a, b = 0.0005, 0.002
    es2 = (a * a + a * b + b * b) / 3
    assert abs(Y.std() / math.sqrt(K * ew2 * es2) - 1) < 0.05


# ------------------------------------------------------------------ int8 fragment layout

def test_frag8_layout_is_a_bijection():
    K, N = 256, 256
    idx = np.array([[oracle.frag8_byte_index(K, k, n) for n in range(N)] for k in range(K)])
    assert np.array_equal(np.sort(idx.ravel()), np.arange(K * N))


def test_frag8_layout_hand_positions():
    K = 256
    cases = {  # (k, n) -> byte, worked from the layout definition
        (0, 0): 0, (1, 0): 1, (7, 0): 7, (8, 0): 256, (32, 0): 8, (64, 0): 1024, (96, 0): 1032,
        (0, 1): 16, (0, 16): 2048, (128, 0): 16384, (0, 128): 32768, (255, 255): 65535,
    }
    for (k, n), want in cases.items():
        assert oracle.frag8_byte_index(K, k, n) == want, (k, n)


def test_frag8_matches_int4_block_and_k_order():
    # byte (block b, half, lane position p, kk, j) holds the k and column of the int4
    # layout's nibble at (block b, p, kk, j): same block ordinal, same lane position
    K, N = 256, 256
    for k in range(0, K, 3):
        for n in range(0, N, 7):
            i8 = oracle.frag8_byte_index(K, k, n)
            i4 = oracle.frag_nibble_index(K, k, n)
            assert i8 // 2048 == i4 // 2048
            p8 = (i8 % 1024) // 16
            kk8 = 2 * ((i8 % 2048) // 1024) + (i8 % 16) // 8
            p4 = (i4 // 2 % 1024) // 16
            kk4 = (i4 // 2 % 16) // 4
            assert (p8, kk8) == (p4, kk4), (k, n)


def test_frag8_offset_binary_values():
    K, N = 128, 128
    assert not oracle.w8a16_prepack(np.full((K, N), -128, np.int8), K, N).any()
    assert (oracle.w8a16_prepack(np.full((K, N), 127, np.int8), K, N) == 0xFF).all()
    assert (oracle.w8a16_prepack(np.zeros((K, N), np.int8), K, N) == 0x80).all()


@pytest.mark.parametrize("K,N", [(200, 136), (8, 8), (1000, 24)])
def test_frag8_ragged_is_the_zero_padded_layout(K, N):
    """Ragged K and N pad to whole 128 x 128 tiles with weight 0 (offset-binary 128): the bytes
    equal the layout of the matrix extended with zero rows and columns."""
    W = qi.w8a16_problem(1, K, N, 32, 336 + K)[1]
    Kp, Np = -(-K // 128) * 128, -(-N // 128) * 128
    Wp = np.zeros((Kp, Np), np.int8)
    Wp[:K, :N] = W
    F = oracle.w8a16_prepack(W, K, N)
    assert F.size == Kp * Np
    assert np.array_equal(F, oracle.w8a16_prepack(Wp, Kp, Np))
    idx = np.array([[oracle.frag8_byte_index(K, k, n) for n in range(N)] for k in range(K)]).ravel()
    assert np.unique(idx).size == K * N
    pad = np.ones(F.size, bool)
    pad[idx] = False
    assert np.all(F[pad] == 128)


@pytest.mark.parametrize("K,G", [(40, 32), (200, 64), (72, 72)])
def test_w8a16_partial_last_group_exact(K, G):
    M, N = 2, 5
    A, W, S = qi.w8a16_problem(M, K, N, G, 337 + K)
    assert S.shape == (-(-K // G), N)
    ref64 = np.array([[float(v) for v in row] for row in exact(A, W, S, G)])
    Y, Y64 = oracle.w8a16(A, W, S, G, want_f64=True)
    assert np.allclose(Y64, ref64, rtol=1e-14, atol=0)
    assert np.array_equal(bits16(Y), bits16(ref64.astype(np.float16)))


def test_frag8_moves_every_byte():
    K, N = 256, 384
    W = qi.w8a16_problem(1, K, N, 128, 335)[1]
    F = oracle.w8a16_prepack(W, K, N)
    k = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    idx = np.vectorize(lambda a, b: oracle.frag8_byte_index(K, a, b))(k, n)
    assert np.array_equal(F[idx].astype(np.int32) - 128, W.astype(np.int32))
