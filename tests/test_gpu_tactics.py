"""GPU parity of every W4A16 tactic (kernel variant) against the CPU oracle.

Each tactic the library lists as valid for a shape must meet the fp16 bar
|y - y_ref| <= 1e-2 |y_ref| + 1e-3 max|y_ref| and be deterministic; tactic 0
must give exactly qgemm_w4a16's bits; the autotune call must return a valid
tactic, and "auto" must give exactly that tactic's bits.  Shapes cover each
tactic's range (decode-sized M with the prefill tactics, mid M with split-K,
N not a multiple of 256).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import qgemm_inputs as qi

pytestmark = pytest.mark.gpu


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


def bits(a):
    return np.asarray(a).view(np.uint16)


def assert_fp16_close(y, ref, what=""):
    y64 = y.astype(np.float64)
    r64 = ref.astype(np.float64)
    assert np.all(np.isfinite(y64)), f"{what}: non-finite outputs"
    bad = np.abs(y64 - r64) > 1e-2 * np.abs(r64) + 1e-3 * np.abs(r64).max()
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside tolerance"


@pytest.mark.parametrize("M,K,N,G", [(1, 512, 256, 128), (2, 1152, 512, 32), (3, 512, 384, 64),
                                     (16, 512, 512, 128), (17, 1152, 256, 64), (64, 512, 384, 128),
                                     (200, 384, 512, 32), (600, 256, 512, 128)])
def test_every_tactic(qg, M, K, N, G):
    A, Wb, S = qi.w4a16_problem(M, K, N, G, 1100 + M + K + N)
    Wf = qg.qgemm_w4a16_prepack(dev(Wb), K, N)
    Ad, Sd = dev(A), dev(S)
    ref = oracle.w4a16(A, Wb, S, G)
    tactics = qg.qgemm_w4a16_tactics(M, N, K, G)
    assert qg.QGEMM_W4A16_TACTIC_PREFILL in tactics
    for t in tactics:
        y1 = host(qg.qgemm_w4a16(Ad, Wf, Sd, G, tactic=t))
        assert_fp16_close(y1, ref, f"M={M} K={K} N={N} G={G} tactic={t}")
        y2 = host(qg.qgemm_w4a16(Ad, Wf, Sd, G, tactic=t))
        assert np.array_equal(bits(y1), bits(y2)), f"tactic {t} not deterministic"
    y0 = host(qg.qgemm_w4a16(Ad, Wf, Sd, G, tactic=0))
    yd = host(qg.qgemm_w4a16(Ad, Wf, Sd, G))
    assert np.array_equal(bits(y0), bits(yd))


def test_tactics_full_decode_shape(qg):
    M, K, N, G = 8, 4096, 11008, 128
    Wb, S = qi.w4a16_weights(K, N, G, 101)
    A = qi.activations(M, K, 1108)
    Wf = qg.qgemm_w4a16_prepack(dev(Wb), K, N)
    ms, ns = qi.sample_positions(M, N, 2000, 15)
    ref = oracle.w4a16_at(A, Wb, S, G, ms, ns)
    for t in qg.qgemm_w4a16_tactics(M, N, K, G):
        y = host(qg.qgemm_w4a16(dev(A), Wf, dev(S), G, tactic=t))
        assert_fp16_close(y[ms, ns], ref, f"tactic {t}")


def test_autotune(qg):
    M, K, N, G = 24, 1024, 2048, 128
    A, Wb, S = qi.w4a16_problem(M, K, N, G, 1120)
    Wf = qg.qgemm_w4a16_prepack(dev(Wb), K, N)
    Ad, Sd = dev(A), dev(S)
    best, us = qg.qgemm_w4a16_autotune(Ad, Wf, Sd, G, reps=5)
    assert best in qg.qgemm_w4a16_tactics(M, N, K, G) and us > 0
    ya = host(qg.qgemm_w4a16(Ad, Wf, Sd, G, tactic="auto"))
    yt = host(qg.qgemm_w4a16(Ad, Wf, Sd, G, tactic=best))
    assert np.array_equal(bits(ya), bits(yt))
    assert_fp16_close(ya, oracle.w4a16(A, Wb, S, G), f"auto tactic {best}")
