"""GPU parity of the INT8 multi-head attention chain against the CPU oracle.

Bars: logits S bit-exact; probability codes P within one code of the
oracle's rne(127 p) everywhere and equal wherever 127 p lies more than
1e-3 of a code from a rounding boundary (the kernel's softmax runs in fp32:
exp2 of max-shifted logits, an online sum over key blocks, e * fl(127 / l);
its error in 127 p is below 6.4e-4 of a code -- a few fp32 ulps of e, l and
the product); the output O bit-exact against the oracle's P.V and
requantization applied to the kernel's own codes (integer products and a
fixed fp32 sequence).  Launches without the debug outputs must give the same
O.  Shapes cover ragged query and key counts, head_dim 64 and 128, several
batches and heads, and the benchmark shape (sampled heads).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import qgemm_inputs as qi

pytestmark = pytest.mark.gpu

BAND = 1e-3


@pytest.fixture(scope="module")
def qg():
    import bit_quantized_gemm_qgemm_amd as qg
    if not os.path.exists(qg.LIB_PATH):
        from bit_quantized_gemm_qgemm_amd import build
        build.build()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qg.lib()
    return qg


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_codes(P, R, what):
    ref = np.rint(R).astype(np.int64)
    diff = np.abs(P.astype(np.int64) - ref)
    assert diff.max() <= 1, f"{what}: a probability code is off by {diff.max()}"
    frac = R - np.floor(R)
    clear = np.abs(frac - 0.5) > BAND
    bad = (diff > 0) & clear
    assert not bad.any(), f"{what}: {bad.sum()} codes differ away from a rounding boundary"
    return int((diff > 0).sum())


def run_case(qg, B, Lq, Lk, H, D, seed, use_bias=True, inputs=None, heads=None):
    Q, K, V, bias, alpha, pv, om = inputs if inputs is not None else qi.mha_problem(B, Lq, Lk, H, D, seed)
    S_d = torch.empty((B, H, Lq, Lk), dtype=torch.int32, device="cuda")
    P_d = torch.empty((B, H, Lq, Lk), dtype=torch.int8, device="cuda")
    args = (dev(Q), dev(K), dev(V), alpha, pv, om)
    bd = dev(bias) if use_bias else None
    O = host(qg.mha_int8(*args, bias=bd, s_out=S_d, p_out=P_d))
    O2 = host(qg.mha_int8(*args, bias=bd))
    assert np.array_equal(O, O2), "debug outputs changed O"
    S = host(S_d).reshape(B * H, Lq, Lk)
    P = host(P_d).reshape(B * H, Lq, Lk)
    hs = np.arange(B * H) if heads is None else np.asarray(heads)
    S_ref, P_ref, R = oracle.mha_int8_probs(Q, K, alpha, heads=hs)
    assert np.array_equal(S[hs], S_ref), "logits"
    nd = check_codes(P[hs], R, f"B={B} Lq={Lq} Lk={Lk} H={H} D={D}")
    O_ref = oracle.mha_int8_out(P[hs], V, bias, pv, om, 1 if use_bias else 0, Lq, heads=hs)
    for hh in hs:
        b, h = divmod(int(hh), H)
        assert np.array_equal(O[b, :, h], O_ref[b, :, h]), f"O head {hh}"
    return nd


# batch x heads a multiple of 8 (the last two cases) takes the XCD-grouped workgroup
# order: every query tile of a head on one XCD
@pytest.mark.parametrize("B,Lq,Lk,H,D", [(1, 1, 1, 1, 64), (2, 37, 53, 3, 64), (1, 128, 128, 2, 128),
                                         (1, 77, 197, 12, 64), (2, 129, 31, 2, 128), (1, 300, 1000, 2, 128),
                                         (3, 5, 65, 4, 64), (1, 256, 33, 1, 128), (2, 300, 100, 4, 64),
                                         (1, 130, 64, 8, 128)])
def test_mha_shapes(qg, B, Lq, Lk, H, D):
    run_case(qg, B, Lq, Lk, H, D, 800 + Lq + Lk)


def test_mha_no_bias(qg):
    run_case(qg, 1, 64, 100, 2, 64, 810, use_bias=False)


def test_mha_closed_forms(qg):
    B, Lq, H, D = 1, 40, 2, 64
    Q, K, V, bias, alpha, pv, om = qi.mha_problem(B, Lq, 1, H, D, 820)
    P_d = torch.empty((B, H, Lq, 1), dtype=torch.int8, device="cuda")
    qg.mha_int8(dev(Q), dev(K), dev(V), alpha, pv, om, bias=dev(bias), p_out=P_d)
    assert (host(P_d) == 127).all()  # one key
    for Lk in (2, 3, 45, 254):  # identical keys: uniform codes rne(127 / Lk)
        Kc = np.ascontiguousarray(np.repeat(K[:, :1], Lk, axis=1))
        Vc = np.ascontiguousarray(np.repeat(V[:, :1], Lk, axis=1))
        run_case(qg, B, Lq, Lk, H, D, 0, inputs=(Q, Kc, Vc, bias, alpha, pv, om))
    # a dominant logit: one-hot codes
    Q1 = np.zeros((1, 8, 1, 64), np.int8)
    Q1[..., 0] = 100
    K1 = np.zeros((1, 50, 1, 64), np.int8)
    K1[0, 17, 0, 0] = 100
    V1 = qi.mha_problem(1, 1, 50, 1, 64, 821)[2]
    P_d = torch.empty((1, 1, 8, 50), dtype=torch.int8, device="cuda")
    qg.mha_int8(dev(Q1), dev(K1), dev(V1), 1.0, pv, om, p_out=P_d)
    P = host(P_d)[0, 0]
    assert (P[:, 17] == 127).all() and (np.delete(P, 17, axis=1) == 0).all()


def test_mha_extreme_values(qg):
    # +-127 everywhere: |S| = D * 16129, exact in fp32; outputs saturate
    B, Lq, Lk, H, D = 1, 33, 70, 2, 128
    Q, K, V, bias, alpha, pv, om = qi.mha_problem(B, Lq, Lk, H, D, 830)
    sgn = np.where(qi.rng(831).random((B, Lq, H, D)) < 0.5, -127, 127).astype(np.int8)
    Kx = np.where(qi.rng(832).random((B, Lk, H, D)) < 0.5, -127, 127).astype(np.int8)
    Vx = np.full((B, Lk, H, D), 127, np.int8)
    run_case(qg, B, Lq, Lk, H, D, 0, inputs=(sgn, Kx, Vx, bias, np.float32(1e-6), pv, om))


def test_mha_full_shape_sampled(qg):
    # 8 sequences x 512 tokens, 32 heads of 128 (the W8A8 token batch), 6 heads checked
    B, Lq, Lk, H, D = 8, 512, 512, 32, 128
    run_case(qg, B, Lq, Lk, H, D, 840, heads=[0, 33, 100, 161, 222, 255])


def test_mha_zero_queries_is_noop(qg):
    Q, K, V, bias, alpha, pv, om = qi.mha_problem(1, 1, 8, 1, 64, 850)
    O = torch.full((1, 1, 1, 64), 5, dtype=torch.int8, device="cuda")
    qg.mha_int8(dev(Q)[:, :0], dev(K), dev(V), alpha, pv, om, O=O[:, :0])
    assert (host(O) == 5).all()
