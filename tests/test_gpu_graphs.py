"""Captured launches: each entry point recorded into a HIP graph (as the
benchmark runs them) and replayed several times, with eager launches and
synchronizations between the replays, must reproduce the eager result bit
for bit on every replay.  Covers kernels with device-side state between
launches of one call: the split-K partials in a workspace, the per-tensor
FP8 partial maxima (written into the head of Q by one launch, read by the
next two) and the MoE workspace.
"""
import os

import numpy as np
import pytest
import torch

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


def replay_matches(fn, outs, reps=4):
    """Eager result first, then a captured graph replayed `reps` times; outputs are
    cleared before each replay and compared with the eager bits afterwards."""
    fn()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fn()  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    for r in range(reps):
        for o in outs:
            o.zero_()
        fn()  # eager work between replays
        torch.cuda.synchronize()
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o.view(torch.uint8), w.view(torch.uint8)), f"replay {r} differs"


def test_graph_w4a16_decode_splitk_prefill(qg):
    K, N, G = 1024, 1024, 128
    Wb, S = qi.w4a16_weights(K, N, G, 1200)
    Wf, Sd = qg.qgemm_w4a16_prepack(dev(Wb), K, N), dev(S)
    for M in (1, 8, 64, 700):
        A = dev(qi.activations(M, K, 1201 + M))
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        need = qg.qgemm_w4a16_workspace_bytes(M, N, K, G)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda") if need else None
        replay_matches(lambda: qg.qgemm_w4a16(A, Wf, Sd, G, Y=Y, workspace=ws), [Y])
        if M == 700:  # the 128x256 kernel by its tactic
            replay_matches(lambda: qg.qgemm_w4a16(A, Wf, Sd, G, Y=Y, tactic=qg.QGEMM_W4A16_TACTIC_PREFILL_LARGE), [Y])


def test_graph_w8a8_and_quant(qg):
    M, N, K = 300, 512, 512
    X, Wf16, bias, om = qi.w8a8_problem(M, N, K, 1210)
    Xd, Wd, bd = dev(X), dev(Wf16), dev(bias)
    qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sa = torch.empty(M, dtype=torch.float32, device="cuda")
    qw, sw = qg.quant_sym_int8(Wd)
    Y = torch.empty((M, N), dtype=torch.int8, device="cuda")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")

    def step():
        qg.quant_sym_int8(Xd, Q=qa, scales=sa)
        qg.qgemm_w8a8_epilogue(qa, qw, sa, sw, bd, float(om), 3, Y=Y, acc_out=acc)
    replay_matches(step, [qa, sa, Y, acc])


def test_graph_fp8_per_tensor(qg):
    M, N, K = 260, 384, 512
    X, Wf16, _, _ = qi.w8a8_problem(M, N, K, 1220)
    Xd = dev(X)
    qw, sw = qg.quant_fp8_e4m3(dev(Wf16), per_row=False)
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty(1, dtype=torch.float32, device="cuda")
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")

    def step():
        qg.quant_fp8_e4m3(Xd, per_row=False, Q=qa, scales=sa)
        qg.qgemm_fp8(qa, qw, sa, sw, Y=Y)
    replay_matches(step, [qa, sa, Y])


def test_graph_moe(qg):
    T, H, I, E, topK, G = 40, 256, 256, 4, 2, 128
    X, logits, Wg, Wu, Wd, Sg, Su, Sd = qi.moe_problem(T, H, I, E, G, 1230)
    pg = torch.cat([qg.qgemm_w4a16_prepack(dev(Wg[e]), H, I) for e in range(E)])
    pu = torch.cat([qg.qgemm_w4a16_prepack(dev(Wu[e]), H, I) for e in range(E)])
    pd = torch.cat([qg.qgemm_w4a16_prepack(dev(Wd[e]), I, H) for e in range(E)])
    args = [dev(X), dev(logits), pg, pu, pd, dev(Sg), dev(Su), dev(Sd)]
    ws = torch.empty(qg.moe_w4a16_workspace_bytes(T, H, I, E, topK), dtype=torch.uint8, device="cuda")
    Y = torch.empty((T, H), dtype=torch.float16, device="cuda")
    ids = torch.empty((T, topK), dtype=torch.int32, device="cuda")
    w = torch.empty((T, topK), dtype=torch.float32, device="cuda")
    replay_matches(lambda: qg.moe_w4a16(*args, topK, G, Y=Y, topk_ids=ids, topk_w=w, workspace=ws), [Y, ids, w])


def test_graph_mha(qg):
    Q, K, V, bias, alpha, pv, om = qi.mha_problem(2, 100, 90, 4, 64, 1240)
    args, bd = [dev(Q), dev(K), dev(V)], dev(bias)
    O = torch.empty(Q.shape, dtype=torch.int8, device="cuda")
    replay_matches(lambda: qg.mha_int8(*args, alpha, pv, om, bias=bd, O=O), [O])
