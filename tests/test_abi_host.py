"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library loads, exports every function include/libqgemm.h declares, and
rejects invalid requests with the documented status codes before touching the
GPU (validation happens before any launch).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libqgemm.h")
LIB = os.path.join(ROOT, "bit_quantized_gemm_qgemm_amd", "libqgemm.so")

P = ctypes.c_void_p
I32 = ctypes.c_int32


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"QGEMM_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


@pytest.fixture(scope="module")
def L():
    import torch  # noqa: F401  -- load torch's HIP runtime first, as the binding does
    if not os.path.exists(LIB):
        from bit_quantized_gemm_qgemm_amd import build
        build.build()
    import bit_quantized_gemm_qgemm_amd as qg
    return qg.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    assert sorted(names) == sorted([
        "qgemm_abi_version", "qgemm_status_str", "qgemm_w4a16_packed_bytes",
        "qgemm_w4a16_prepack", "qgemm_w4a16_workspace_bytes", "qgemm_w4a16", "quant_sym_int8",
        "dequant_sym_int8", "qgemm_w8a8_epilogue", "moe_w4a16_workspace_bytes", "moe_w4a16",
        "quant_fp8_e4m3", "dequant_fp8_e4m3", "qgemm_fp8", "qgemm_w8a16_packed_bytes",
        "qgemm_w8a16_prepack", "qgemm_w8a16_workspace_bytes", "qgemm_w8a16", "mha_int8",
        "qgemm_w4a16_tactics", "qgemm_w4a16_tactic_workspace_bytes", "qgemm_w4a16_tactic",
        "qgemm_w4a16_autotune", "moe_w4a16_no_alloc", "qgemm_stream_read", "qgemm_stream_copy"])


def test_library_exports_every_declared_symbol(L):
    import bit_quantized_gemm_qgemm_amd as qg
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) == set(qg.EXPORTS)


def test_version_and_status_strings(L):
    assert L.qgemm_abi_version() == 1
    assert L.qgemm_status_str(0) == b"ok"
    assert L.qgemm_status_str(4) == b"workspace too small"
    assert L.qgemm_status_str(99) == b"unknown status"


def test_size_queries(L):
    assert L.qgemm_w4a16_packed_bytes(4096, 11008) == 4096 * 11008 // 2
    # ragged K and N pad to whole 128 x 128 tiles; K and N must be multiples of 8
    assert L.qgemm_w4a16_packed_bytes(4000, 11008) == 4096 * 11008 // 2
    assert L.qgemm_w4a16_packed_bytes(200, 136) == 256 * 256 // 2
    assert L.qgemm_w4a16_packed_bytes(4096, 100) == 0
    assert L.qgemm_w4a16_packed_bytes(4092, 128) == 0
    assert L.qgemm_w4a16_workspace_bytes(1, 11008, 4096, 128) == 0
    assert L.qgemm_w4a16_workspace_bytes(16, 11008, 4096, 128) == 0
    assert L.qgemm_w4a16_workspace_bytes(129, 11008, 4096, 128) == 0
    # mid M: S * M * N * 4 with S = max(1, min(floor(512 / (N/128)), K/128, 16)), by the header's rule
    for M, N, K in [(17, 11008, 4096), (64, 11008, 4096), (64, 4096, 4096), (128, 256, 256), (100, 128, 512),
                    (64, 131072, 4096)]:
        S = max(1, min(512 // (N // 128), K // 128, 16))
        assert L.qgemm_w4a16_workspace_bytes(M, N, K, 128) == S * M * N * 4, (M, N, K)
    assert L.qgemm_w4a16_workspace_bytes(64, 11008, 4000, 128) == 0   # ragged K: no split-K path
    ws = L.moe_w4a16_workspace_bytes(256, 4096, 14336, 8, 2)
    P_ = 512
    # down-projection K splits, by the rule the header states
    splits, E, H, I = 1, 8, 4096, 14336
    while splits < 8 and E * (H // 128) * splits < 512 and (I // 128) % (2 * splits) == 0:
        splits *= 2
    assert splits == 2
    need = 256 + 2 * 2048 + 2 * P_ * I + 4 * splits * P_ * H
    assert need <= ws <= need + 5 * 256


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def test_w4a16_validation(L):
    f = L.qgemm_w4a16
    assert f(None, None, None, None, 0, 128, 128, 128, None, 0, None) == 0  # M == 0: no-op
    assert f(None, FAKE, FAKE, FAKE, 4, 128, 128, 128, None, 0, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, -1, 128, 128, 128, None, 0, None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 128, 128, 96, None, 0, None) == 5  # G = 96
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 124, 128, 128, None, 0, None) == 5  # N % 8
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 128, 132, 128, None, 0, None) == 5  # K % 8
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 128, 256, 256, None, 0, None) == 5  # G = 256
    assert f(FAKE + 2, FAKE, FAKE, FAKE, 4, 128, 128, 128, None, 0, None) == 3
    assert f(FAKE, FAKE, FAKE, FAKE + 8, 4, 128, 128, 128, None, 0, None) == 3


def test_w8a16_size_queries_and_validation(L):
    assert L.qgemm_w8a16_packed_bytes(4096, 11008) == 4096 * 11008
    assert L.qgemm_w8a16_packed_bytes(4000, 11008) == 4096 * 11008
    assert L.qgemm_w8a16_packed_bytes(4000, 11004) == 0
    for M, N, K, G in [(17, 11008, 4096, 128), (64, 11008, 4096, 4096), (128, 256, 256, 64)]:
        S = max(1, min(512 // (N // 128), K // 128, 16))
        assert L.qgemm_w8a16_workspace_bytes(M, N, K, G) == S * M * N * 4, (M, N, K, G)
    assert L.qgemm_w8a16_workspace_bytes(8, 11008, 4096, 128) == 0
    assert L.qgemm_w8a16_workspace_bytes(64, 11008, 4096, 256) == 0  # G neither <= 128 nor K
    f = L.qgemm_w8a16
    assert f(None, None, None, None, 0, 128, 128, 128, None, 0, None) == 0
    assert f(None, FAKE, FAKE, FAKE, 4, 128, 128, 128, None, 0, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, 4, -128, 128, 128, None, 0, None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 128, 384, 256, None, 0, None) == 5  # G = 256, neither <= 128 nor K
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 128, 512, 256, None, 0, None) == 5  # G = 256 < K
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 128, 204, 204, None, 0, None) == 5  # K % 8
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 100, 128, 128, None, 0, None) == 5  # N % 8
    assert f(FAKE, FAKE, FAKE + 2, FAKE, 4, 128, 128, 128, None, 0, None) == 3
    p = L.qgemm_w8a16_prepack
    assert p(None, FAKE, 128, 128, None) == 1
    assert p(FAKE, FAKE, 128, 0, None) == 0
    assert p(FAKE, FAKE, -128, 128, None) == 2
    assert p(FAKE, FAKE, 128, 196, None) == 5
    assert p(FAKE + 4, FAKE + 65536, 128, 128, None) == 3
    assert p(FAKE, FAKE + 8192, 128, 128, None) == 2  # overlapping buffers


def test_mha_validation(L):
    f = L.mha_int8
    args = lambda B, H, Lq, Lk, D, flags=0, q=FAKE, k=FAKE, v=FAKE, bias=FAKE, o=FAKE: (
        q, k, v, bias, o, None, None, B, H, Lq, Lk, D, 1.0, 1.0, 1.0, flags, None)
    assert f(*args(1, 1, 0, 16, 64)) == 0                      # Lq == 0: no-op
    assert f(*args(0, 1, 8, 16, 64, q=None)) == 0              # B == 0: no-op before pointer checks
    assert f(*args(1, 1, 8, 16, 64, q=None)) == 1
    assert f(*args(1, 1, 8, 16, 64, flags=1, bias=None)) == 1  # bias flagged but missing
    assert f(*args(1, 1, -8, 16, 64)) == 2
    assert f(*args(1, 1, 8, 0, 64)) == 2                       # softmax over no keys
    assert f(*args(1, 1, 8, 16, 96)) == 5                      # head_dim
    assert f(*args(1, 1, 8, 16, 64, flags=2)) == 5             # no GELU in this chain
    assert f(*args(1, 1, 8, 133144, 64)) == 5                  # P V would overflow int32
    assert f(*args(1, 1, 8, 16, 64, k=FAKE + 8)) == 3
    assert f(*args(1, 1, 8, 16, 64, flags=1, bias=FAKE + 2)) == 3


def test_w4a16_tactic_lists(L):
    import ctypes
    def tactics(M, N, K, G=128):
        buf = (ctypes.c_int32 * 8)()
        n = L.qgemm_w4a16_tactics(M, N, K, G, buf, 8)
        return list(buf[:n])
    # by the validity rules the header states
    assert tactics(1, 11008, 4096) == [1, 2, 3, 4, 5]  # 11008 = 43 * 256
    assert tactics(1, 11136, 4096) == [1, 2, 3, 4]     # 11136 = 87 * 128
    assert tactics(2, 4096, 4096) == [1, 2, 3, 4, 5]
    assert tactics(16, 4096, 4096) == [2, 3, 4, 5]
    assert tactics(64, 11008, 4096) == [3, 4, 5]
    assert tactics(512, 4096, 4096) == [3, 4, 5]
    assert tactics(513, 4096, 4096) == [4, 5]
    assert tactics(2048, 384, 4096) == [4]
    assert tactics(0, 4096, 4096) == [] and tactics(8, 4096, 4092) == [] and tactics(8, 4096, 4096, 256) == []
    # ragged K or N: the decode kernels and the 128x128 prefill only
    assert tactics(8, 4096, 4000) == [2, 4] and tactics(1, 136, 4096) == [1, 2, 4]
    assert tactics(64, 4096, 200) == [4] and tactics(2048, 4104, 4096) == [4]
    assert L.qgemm_w4a16_tactics(1, 4096, 4096, 128, None, 0) == 5
    buf = (ctypes.c_int32 * 2)()
    assert L.qgemm_w4a16_tactics(1, 4096, 4096, 128, buf, 2) == 5 and list(buf) == [1, 2]
    S = max(1, min(512 // (11008 // 128), 4096 // 128, 16))
    assert L.qgemm_w4a16_tactic_workspace_bytes(8, 11008, 4096, 128, 3) == S * 8 * 11008 * 4
    assert L.qgemm_w4a16_tactic_workspace_bytes(8, 11008, 4096, 128, 0) == 0
    assert L.qgemm_w4a16_tactic_workspace_bytes(64, 11008, 4096, 128, 0) == S * 64 * 11008 * 4
    assert L.qgemm_w4a16_tactic_workspace_bytes(64, 11008, 4096, 128, 4) == 0
    assert L.qgemm_w4a16_tactic_workspace_bytes(600, 11008, 4096, 128, 3) == 0  # not valid there
    f = L.qgemm_w4a16_tactic
    assert f(FAKE, FAKE, FAKE, FAKE, 64, 4096, 4096, 128, 1, None, 0, None) == 5   # narrow decode: M <= 2
    assert f(FAKE, FAKE, FAKE, FAKE, 64, 4096, 4096, 128, 9, None, 0, None) == 5   # unknown id
    assert f(FAKE, FAKE, FAKE, FAKE, 64, 384, 4096, 128, 5, None, 0, None) == 5    # N % 256
    assert f(FAKE, FAKE, FAKE, FAKE, 64, 4096, 4096, 128, 3, None, 0, None) == 4   # no workspace
    assert f(FAKE, FAKE, FAKE, FAKE, 64, 4096, 4096, 128, 3, FAKE + 8, 1 << 30, None) == 3
    assert f(None, None, None, None, 0, 4096, 4096, 128, 4, None, 0, None) == 0     # M == 0
    assert f(None, FAKE, FAKE, FAKE, 4, 4096, 4096, 128, 4, None, 0, None) == 1
    a = L.qgemm_w4a16_autotune
    best = ctypes.c_int32(-1)
    assert a(FAKE, FAKE, FAKE, FAKE, 4, 4096, 4096, 128, None, 0, 10, None, None, None) == 1
    assert a(FAKE, FAKE, FAKE, FAKE, 4, 4096, 4096, 128, None, 0, 0, ctypes.byref(best), None, None) == 2
    assert a(FAKE, FAKE, FAKE, FAKE, 0, 4096, 4096, 128, None, 0, 5, ctypes.byref(best), None, None) == 2
    assert a(FAKE, FAKE, FAKE, FAKE, 4, 100, 4096, 128, None, 0, 5, ctypes.byref(best), None, None) == 5
    assert best.value == -1


def test_prepack_validation(L):
    f = L.qgemm_w4a16_prepack
    assert f(None, FAKE, 128, 128, None) == 1
    assert f(FAKE, FAKE, 0, 128, None) == 0
    assert f(FAKE, FAKE, 100, 128, None) == 5
    assert f(FAKE, FAKE + 4, 128, 128, None) == 3
    assert f(FAKE, FAKE + 4096, 128, 128, None) == 2  # overlapping buffers


def test_quant_validation(L):
    q, d = L.quant_sym_int8, L.dequant_sym_int8
    assert q(FAKE, FAKE, FAKE, 0, 128, None) == 0
    assert q(None, FAKE, FAKE, 4, 128, None) == 1
    assert q(FAKE, FAKE, FAKE, 4, 12, None) == 5
    assert q(FAKE, FAKE, FAKE, 4, 65544, None) == 5
    assert q(FAKE + 8, FAKE, FAKE, 4, 128, None) == 3
    assert d(FAKE, FAKE, None, 4, 128, None) == 1
    assert d(FAKE, FAKE, FAKE, -4, 128, None) == 2
    assert d(FAKE, FAKE, FAKE, 4, 100, None) == 5


def test_fp8_validation(L):
    q, d, g = L.quant_fp8_e4m3, L.dequant_fp8_e4m3, L.qgemm_fp8
    assert q(FAKE, FAKE, FAKE, 0, 128, 1, None) == 0
    assert q(None, FAKE, FAKE, 4, 128, 1, None) == 1
    assert q(FAKE, FAKE, FAKE, -1, 128, 1, None) == 2
    assert q(FAKE, FAKE, FAKE, 4, 12, 1, None) == 5
    assert q(FAKE, FAKE, FAKE, 4, 4104, 1, None) == 5      # per row: at most 4096 columns
    assert q(FAKE, FAKE, FAKE, 4, 128, 2, None) == 5       # granularity is 0 or 1
    assert q(FAKE + 8, FAKE, FAKE, 4, 128, 0, None) == 3
    assert d(FAKE, FAKE, None, 4, 128, 1, None) == 1
    assert d(FAKE, FAKE, FAKE, 4, 100, 0, None) == 5
    assert d(FAKE, FAKE + 2, FAKE, 4, 128, 0, None) == 3
    assert g(FAKE, FAKE, FAKE, 1, FAKE, 1, FAKE, 0, 256, 256, None) == 0
    assert g(FAKE, FAKE, FAKE, 1, FAKE, 1, FAKE, 4, 0, 256, None) == 0
    assert g(FAKE, None, FAKE, 1, FAKE, 1, FAKE, 4, 256, 256, None) == 1
    assert g(FAKE, FAKE, FAKE, 1, FAKE, 1, FAKE, -4, 256, 256, None) == 2
    assert g(FAKE, FAKE, FAKE, 1, FAKE, 1, FAKE, 4, 256, 200, None) == 5   # K % 128
    assert g(FAKE, FAKE, FAKE, 3, FAKE, 1, FAKE, 4, 256, 256, None) == 5   # a_per_row 0 or 1
    assert g(FAKE, FAKE, FAKE, 1, FAKE, 1, FAKE, 1 << 20, 256, 4096, None) == 5  # M*K >= 2^32
    assert g(FAKE + 16, FAKE + 8, FAKE, 1, FAKE, 1, FAKE, 4, 256, 256, None) == 3


def test_w8a8_validation(L):
    f = L.qgemm_w8a8_epilogue
    args = lambda M, N, K, flags=3, bias=FAKE, a=FAKE: (a, FAKE, FAKE, FAKE, bias, 1.0, flags, FAKE,
                                                         None, M, N, K, None)
    assert f(*args(0, 128, 128)) == 0
    assert f(*args(4, 128, 128, bias=None)) == 1      # BIAS flag without a bias
    assert f(*args(4, 128, 128, flags=8)) == 5        # unknown flag
    assert f(*args(4, 100, 128)) == 5
    assert f(*args(4, 128, 133248)) == 5              # accumulator could overflow
    assert f(*args(4, 128, 128, a=FAKE + 1)) == 3
    assert f(*args(-4, 128, 128)) == 2


def test_moe_no_alloc_validation(L):
    # every rejection here happens before the library touches HIP
    f = L.moe_w4a16_no_alloc
    def call(T=4, H=128, I=128, E=4, topK=2, G=128, act=0, ptr=FAKE):
        return f(*([ptr] * 11), T, H, I, E, topK, G, act, None)
    assert call(T=0) == 0
    assert call(topK=5) == 2
    assert call(act=4) == 5
    assert call(ptr=None) == 1
    assert call(ptr=FAKE + 2) == 3
    limit = 64 << 20
    # the 256-token layer fits the scratch array; 4096 tokens do not
    assert L.moe_w4a16_workspace_bytes(256, 4096, 14336, 8, 2) <= limit
    assert L.moe_w4a16_workspace_bytes(4096, 4096, 14336, 8, 2) > limit
    assert call(T=4096, H=4096, I=14336, E=8) == 4


def test_stream_read_validation(L):
    f = L.qgemm_stream_read
    assert f(None, 0, None, None) == 0
    assert f(None, 16, FAKE, None) == 1
    assert f(FAKE, 24, FAKE, None) == 2
    assert f(FAKE + 8, 32, FAKE, None) == 3


def test_stream_copy_validation(L):
    f = L.qgemm_stream_copy
    assert f(None, 0, None, 0, None) == 0
    assert f(None, 32, FAKE, 16, None) == 1
    assert f(FAKE, 32, FAKE, 32, None) == 2       # only the 2:1 and 1:2 shapes
    assert f(FAKE, 48, FAKE, 24, None) == 2       # sizes multiples of 16
    assert f(FAKE + 8, 32, FAKE, 16, None) == 3
    assert f(FAKE, 16, FAKE + 8, 32, None) == 3


def test_moe_validation(L):
    f = L.moe_w4a16
    def call(T=4, H=128, I=128, E=4, topK=2, G=128, act=0, ws=FAKE, wsb=1 << 30):
        return f(*([FAKE] * 11), T, H, I, E, topK, G, act, ws, wsb, None)
    assert call(T=0) == 0
    assert call(topK=5) == 2
    assert call(E=0) == 2
    assert call(act=4) == 5 and call(act=-1) == 5
    assert call(E=65, topK=2) == 5
    assert call(H=192, G=64) == 5
    assert call(ws=None) == 1
    assert call(ws=FAKE + 16) == 3
    assert call(wsb=16) == 4
    # A element offsets must stay below 2^31 (32-bit byte offsets of the buffer loads)
    assert call(T=1 << 19, H=4096) == 5                    # T*H = 2^31
    assert call(T=1 << 14, topK=2, I=1 << 16) == 5         # T*topK*I = 2^31


def test_splitk_tactic_limit(L):
    # the split-K tactic needs M*K < 2^31 (32-bit byte offsets of its A loads)
    buf = (ctypes.c_int32 * 8)()
    n = L.qgemm_w4a16_tactics(64, 4096, (1 << 25) - 128, 128, buf, 8)
    assert 3 in list(buf)[:n]
    n = L.qgemm_w4a16_tactics(64, 4096, 1 << 25, 128, buf, 8)
    assert 3 not in list(buf)[:n]
