"""The two measurement aids (streaming read, read+write in the quantizer's
and dequantizer's traffic shapes): they run at the benchmark's sizes and
produce exactly the words their header comment defines."""
import os

import numpy as np
import pytest
import torch

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


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 23413201 // 16 * 16])
def test_stream_read_leaves_sink(qg, nbytes):
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    qg.qgemm_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7          # all-zero data never XOR to the trigger value


@pytest.mark.parametrize("nbytes", [32, 4096 + 32, 32 * 2048 * 128 * 2])
def test_stream_copy_words(qg, nbytes):
    r = np.random.default_rng(nbytes)
    src = r.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint32)
    s = torch.from_numpy(src.view(np.int32)).cuda()
    half = torch.full((nbytes // 8,), -1, dtype=torch.int32, device="cuda")
    qg.qgemm_stream_copy(s, half)
    want = src[0::2] ^ src[1::2]
    assert np.array_equal(half.cpu().numpy().view(np.uint32), want)
    dbl = torch.full((nbytes // 2,), -1, dtype=torch.int32, device="cuda")
    qg.qgemm_stream_copy(s, dbl)
    w = np.empty(nbytes // 2, np.uint32)
    w[0::4], w[1::4] = src[0::2], src[1::2]
    w[2::4], w[3::4] = src[0::2] + np.uint32(1), src[1::2] + np.uint32(1)
    assert np.array_equal(dbl.cpu().numpy().view(np.uint32), w)
