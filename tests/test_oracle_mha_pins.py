"""Pins for the oracle's INT8 multi-head attention chain.

The interview page (INT8 cross-modal MHA TensorRT plugin, answer steps 2-3)
gives the chain -- int8 QK^T to int32 logits, an online fp32 softmax to int8
probabilities scaled by scale_q * scale_k, int8 P.V, requantization with an
fp16 bias -- but not the probability encoding; the oracle takes
P = rne(127 p) (scale 1/127, the page's +-127 code range).  The pins tie it
to a hand-worked case (a rounding tie included), numpy's integer matmul,
scipy's softmax, closed forms and invariances of attention.
"""
import json
import os

import numpy as np
import pytest
import scipy.special

import oracle
import qgemm_inputs as qi

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def hand_cases():
    with open(os.path.join(GOLDEN, "mha_int8_hand.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("idx", [0, 1])
def test_mha_hand(idx):
    c = hand_cases()[idx]
    Q = np.array(c["Q"], np.int8)[None, :, None, :]
    K = np.array(c["K"], np.int8)[None, :, None, :]
    V = np.array(c["V"], np.int8)[None, :, None, :]
    bias = np.array(c["bias"], np.float16)
    S, P, _ = oracle.mha_int8_probs(Q, K, c["alpha"])
    assert S[0].tolist() == c["S"]
    assert P[0].tolist() == c["P"]
    A = P[0].astype(np.int64) @ V[0, :, 0, :].astype(np.int64)
    assert A.tolist() == c["A"]
    for om, want in c["O"].items():
        O = oracle.mha_int8_out(P, V, bias, c["pv_scale"], float(om), c["flags"], Q.shape[1])
        assert O[0, :, 0, :].tolist() == want, om


def logits32(S, alpha):
    return (S.astype(np.float32) * np.float32(alpha)).astype(np.float32)


@pytest.mark.parametrize("shape", [(2, 9, 13, 3, 8), (1, 33, 70, 2, 64), (1, 5, 1, 2, 16)])
def test_mha_scores_and_probs_against_numpy_scipy(shape):
    B, Lq, Lk, H, D = shape
    Q, K, V, bias, alpha, pv, om = qi.mha_problem(B, Lq, Lk, H, D, 700 + Lq)
    S, P, R = oracle.mha_int8_probs(Q, K, alpha)
    S_np = np.einsum("bihc,bjhc->bhij", Q.astype(np.int64), K.astype(np.int64)).reshape(B * H, Lq, Lk)
    assert np.array_equal(S, S_np)
    ref = 127.0 * scipy.special.softmax(logits32(S_np, alpha).astype(np.float64), axis=-1)
    assert np.allclose(R, ref, rtol=1e-12, atol=1e-12)
    clear = np.abs(ref - np.floor(ref) - 0.5) > 1e-9
    assert np.array_equal(P[clear], np.rint(ref[clear]).astype(np.int8))
    assert P.min() >= 0 and P.max() <= 127


def test_mha_closed_forms():
    B, Lq, H, D = 1, 6, 2, 16
    Q, K, V, bias, alpha, pv, om = qi.mha_problem(B, Lq, 1, H, D, 710)
    _, P, _ = oracle.mha_int8_probs(Q, K, alpha)
    assert (P == 127).all()  # one key: p = 1
    for Lk in (2, 3, 7, 254):
        Kc = np.repeat(K[:, :1], Lk, axis=1)  # identical keys: uniform p = 1/Lk
        _, P, R = oracle.mha_int8_probs(Q, Kc, alpha)
        assert (P == np.rint(127.0 / Lk)).all(), Lk
    # a dominant logit: one-hot
    Q1 = np.zeros((1, 1, 1, 4), np.int8)
    Q1[..., 0] = 100
    K1 = np.zeros((1, 5, 1, 4), np.int8)
    K1[0, 3, 0, 0] = 100
    _, P, _ = oracle.mha_int8_probs(Q1, K1, 1.0)
    assert P[0, 0].tolist() == [0, 0, 0, 127, 0]


def test_mha_out_against_integer_matmul_and_fp32_steps():
    B, Lq, Lk, H, D = 2, 7, 19, 3, 32
    Q, K, V, bias, alpha, pv, om = qi.mha_problem(B, Lq, Lk, H, D, 720)
    _, P, _ = oracle.mha_int8_probs(Q, K, alpha)
    A = np.einsum("bhij,bjhc->bihc", P.reshape(B, H, Lq, Lk).astype(np.int64), V.astype(np.int64))
    for flags in (0, 1):
        t = A.astype(np.float32) * np.float32(pv)
        if flags:
            t = (t + bias.astype(np.float32).reshape(H, D)[None, None]).astype(np.float32)
        want = np.clip(np.rint((t * np.float32(om)).astype(np.float32)), -127, 127).astype(np.int8)
        assert np.array_equal(oracle.mha_int8_out(P, V, bias, pv, om, flags, Lq), want), flags


def test_mha_key_permutation_invariance():
    B, Lq, Lk, H, D = 1, 8, 40, 2, 16
    Q, K, V, bias, alpha, pv, om = qi.mha_problem(B, Lq, Lk, H, D, 730)
    perm = qi.rng(731).permutation(Lk)
    O1, _, P1, _ = oracle.mha_int8(Q, K, V, bias, alpha, pv, om, 1)
    O2, _, P2, _ = oracle.mha_int8(Q, K[:, perm], V[:, perm], bias, alpha, pv, om, 1)
    assert np.array_equal(O1, O2)
    assert np.array_equal(P1[:, :, perm], P2)


def test_mha_head_isolation_and_subsets():
    B, Lq, Lk, H, D = 2, 5, 11, 3, 8
    Q, K, V, bias, alpha, pv, om = qi.mha_problem(B, Lq, Lk, H, D, 740)
    O, S, P, R = oracle.mha_int8(Q, K, V, bias, alpha, pv, om, 1)
    heads = [4, 1]
    Os, Ss, Ps, Rs = oracle.mha_int8(Q, K, V, bias, alpha, pv, om, 1, heads=heads)
    assert np.array_equal(Ss, S[heads]) and np.array_equal(Ps, P[heads])
    for hh in heads:
        b, h = divmod(hh, H)
        assert np.array_equal(Os[b, :, h], O[b, :, h])
    # changing head (0, 0)'s inputs leaves every other head's output unchanged
    Q2, K2, V2 = Q.copy(), K.copy(), V.copy()
    Q2[0, :, 0] = -Q2[0, :, 0]
    K2[0, :, 0] = 7
    V2[0, :, 0] = -3
    O2, _, _, _ = oracle.mha_int8(Q2, K2, V2, bias, alpha, pv, om, 1)
    mask = np.ones((B, H), bool)
    mask[0, 0] = False
    for b in range(B):
        for h in range(H):
            if mask[b, h]:
                assert np.array_equal(O2[b, :, h], O[b, :, h])
    assert not np.array_equal(O2[0, :, 0], O[0, :, 0])


def test_mha_probability_mass():
    # rne(127 p) over a row sums to 127 within half a code per key, and each code is within 1/2 of 127 p
    B, Lq, Lk, H, D = 1, 16, 300, 2, 64
    Q, K, V, bias, alpha, pv, om = qi.mha_problem(B, Lq, Lk, H, D, 750)
    _, P, R = oracle.mha_int8_probs(Q, K, alpha)
    assert np.allclose(R.sum(-1), 127.0, rtol=0, atol=1e-9)
    assert np.all(np.abs(P - R) <= 0.5)
    assert np.all(np.abs(P.sum(-1).astype(np.float64) - 127.0) <= 0.5 * Lk)
