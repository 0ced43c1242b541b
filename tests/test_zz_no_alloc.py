"""moe_w4a16_no_alloc -- the MoE layer on the library's per-GPU scratch array,
for callers that cannot allocate -- against moe_w4a16 with a caller-owned
workspace, on the same inputs, twice in a row (the second call smaller, so it
runs over what the first left in the scratch array).  Routing ids bit-exact,
gate weights and the layer output bit-identical (the same kernels), and the
output within the fp16 tolerance of the CPU oracle."""
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
    assert os.path.exists(qg.LIB_PATH), "libqgemm.so is not built"
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qg.lib()
    return qg


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def run_both(qg, T, H, I, E, topK, G, seed):
    print(f"no-alloc MoE T={T} H={H} I={I} E={E} topK={topK} G={G}", flush=True)
    X, logits, Wg, Wu, Wd, Sg, Su, Sd = qi.moe_problem(T, H, I, E, G, seed)
    pg = torch.cat([qg.qgemm_w4a16_prepack(dev(Wg[e]), H, I) for e in range(E)])
    pu = torch.cat([qg.qgemm_w4a16_prepack(dev(Wu[e]), H, I) for e in range(E)])
    pd = torch.cat([qg.qgemm_w4a16_prepack(dev(Wd[e]), I, H) for e in range(E)])
    args = (dev(X), dev(logits), pg, pu, pd, dev(Sg), dev(Su), dev(Sd), topK, G)
    Y = torch.empty((T, H), dtype=torch.float16, device="cuda")
    ids = torch.empty((T, topK), dtype=torch.int32, device="cuda")
    w = torch.empty((T, topK), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    qg.moe_w4a16_no_alloc(*args, Y=Y, topk_ids=ids, topk_w=w)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    Yr, idr, wr, _ = qg.moe_w4a16(*args)
    assert np.array_equal(host(ids), host(idr))
    assert np.array_equal(host(w).view(np.uint32), host(wr).view(np.uint32))
    assert np.array_equal(host(Y).view(np.uint16), host(Yr).view(np.uint16))
    Yo, ido, _ = oracle.moe(X, logits, Wg, Wu, Wd, Sg, Su, Sd, topK, G)
    assert np.array_equal(host(ids), ido)
    y = host(Y).astype(np.float64)
    r = Yo.astype(np.float64)
    assert np.all(np.abs(y - r) <= 1e-2 * np.abs(r) + 1e-3 * np.abs(r).max())


def test_no_alloc_matches_workspace_entry_point_twice(qg):
    run_both(qg, 64, 512, 1024, 8, 2, 128, 1201)
    run_both(qg, 9, 256, 384, 4, 2, 64, 1202)


def test_no_alloc_rejects_a_layer_beyond_the_scratch_size(qg):
    T, H, I, E, topK, G = 4096, 4096, 14336, 8, 2, 128
    assert qg.moe_w4a16_workspace_bytes(T, H, I, E, topK) > qg.MOE_NO_ALLOC_SCRATCH_BYTES
    X = torch.empty((T, H), dtype=torch.float16, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float16, device="cuda")
    wq = torch.empty(16, dtype=torch.uint8, device="cuda")
    s = torch.empty((E, H // G, I), dtype=torch.float16, device="cuda")
    Y = torch.empty((T, H), dtype=torch.float16, device="cuda")
    ids = torch.empty((T, topK), dtype=torch.int32, device="cuda")
    w = torch.empty((T, topK), dtype=torch.float32, device="cuda")
    with pytest.raises(qg.QGemmError) as e:
        qg.moe_w4a16_no_alloc(X, logits, wq, wq, wq, s, s, s, topK, G, Y=Y, topk_ids=ids,
                              topk_w=w, I=I)
    assert e.value.status == qg.WORKSPACE_TOO_SMALL
