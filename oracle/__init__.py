"""CPU oracle for the quantized-GEMM hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library and
its Python binding never import it, and it imports nothing from them.

Thin numpy front end over ``liboracle.so`` (built from ``qgemm_oracle.c``).
Every function takes and returns numpy arrays in the natural formats:
fp16 data as ``np.float16`` (bit patterns passed through unchanged), int4
weights as natural packed bytes ``uint8 [K][N/2]`` (low nibble = even column),
int8 weights as ``int8 [K][N]``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
# QGEMM_ORACLE_LIB: another build of the same source (the sanitizer build of
# tests/test_oracle_sanitized.py)
_LIB_PATH = os.environ.get("QGEMM_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

EPI_BIAS = 1
EPI_GELU = 2


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            _build.build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_U32 = ctypes.c_uint32


def _declare(lib):
    sig = {
        "qo_num_threads": (ctypes.c_int, []),
        "qo_f16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
        "qo_f64_to_f16": (ctypes.c_uint16, [ctypes.c_double]),
        "qo_f16_to_f64_array": (None, [_P, _P, _I64]),
        "qo_f64_to_f16_array": (None, [_P, _P, _I64]),
        "qo_int4_at": (ctypes.c_int, [_P, _I32, _I32, _I32]),
        "qo_int4_unpack": (None, [_P, _P, _I32, _I32]),
        "qo_w4a16": (None, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32]),
        "qo_w4a16_at": (None, [_P, _P, _P, _P, _P, _I64, _P, _P, _I32, _I32, _I32, _I32]),
        "qo_frag_nibble_index": (_I64, [_I32, _I32, _I32]),
        "qo_w4a16_prepack": (None, [_P, _P, _I32, _I32]),
        "qo_w4a16_packed_bytes": (_I64, [_I32, _I32]),
        "qo_w8a16": (None, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32]),
        "qo_w8a16_at": (None, [_P, _P, _P, _P, _P, _I64, _P, _P, _I32, _I32, _I32]),
        "qo_frag8_byte_index": (_I64, [_I32, _I32, _I32]),
        "qo_w8a16_prepack": (None, [_P, _P, _I32, _I32]),
        "qo_w8a16_packed_bytes": (_I64, [_I32, _I32]),
        "qo_quant_sym_int8": (None, [_P, _P, _P, _I64, _I32]),
        "qo_dequant_sym_int8": (None, [_P, _P, _P, _I64, _I32]),
        "qo_w8a8_acc": (None, [_P, _P, _P, _I32, _I32, _I32]),
        "qo_gelu28": (_F32, [_F32]),
        "qo_w8a8_requant": (ctypes.c_int8, [ctypes.c_int32, _F32, _F32, ctypes.c_uint16, _F32, _U32]),
        "qo_w8a8_epilogue": (None, [_P, _P, _P, _P, _P, _F32, _U32, _P, _P, _I32, _I32, _I32]),
        "qo_w8a8_epilogue_at": (None, [_P, _P, _P, _P, _P, _F32, _U32, _P, _P, _I64, _P, _P, _I32]),
        "qo_moe_route": (None, [_P, _I32, _I32, _I32, _P, _P]),
        "qo_moe_permute": (None, [_P, _I32, _I32, _I32, _P, _P]),
        "qo_moe": (None, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                          _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _I32]),
        "qo_moe_act": (ctypes.c_double, [ctypes.c_double, _I32]),
        "qo_e4m3_to_f64": (ctypes.c_double, [ctypes.c_uint8]),
        "qo_f64_to_e4m3": (ctypes.c_uint8, [ctypes.c_double]),
        "qo_e4m3_to_f64_array": (None, [_P, _P, _I64]),
        "qo_f64_to_e4m3_array": (None, [_P, _P, _I64]),
        "qo_quant_fp8": (None, [_P, _P, _P, _I64, _I32, _I32]),
        "qo_dequant_fp8": (None, [_P, _P, _P, _I64, _I32, _I32]),
        "qo_fp8_gemm": (None, [_P, _P, _P, _I32, _P, _I32, _P, _P, _I32, _I32, _I32]),
        "qo_fp8_gemm_at": (None, [_P, _P, _P, _I32, _P, _I32, _I64, _P, _P, _P, _I32]),
        "qo_mha_int8_probs": (None, [_P, _P, _P, _I64, _I32, _I32, _I32, _I32, _F32, _P, _P, _P]),
        "qo_mha_int8_out": (None, [_P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _F32, _F32, _U32, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def num_threads():
    """OpenMP threads the oracle's parallel loops use."""
    return _load().qo_num_threads()


# ---------------------------------------------------------------- fp16

def f16_to_f64(h):
    h = _c(np.asarray(h, dtype=np.float16).view(np.uint16), np.uint16)
    out = np.empty(h.shape, np.float64)
    _load().qo_f16_to_f64_array(_ptr(h), _ptr(out), h.size)
    return out


def f64_to_f16(x):
    x = _c(np.asarray(x, dtype=np.float64), np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().qo_f64_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out.view(np.float16)


# ---------------------------------------------------------------- int4

def int4_unpack(w, K, N):
    w = _c(w, np.uint8)
    assert w.size == K * N // 2
    q = np.empty((K, N), np.int8)
    _load().qo_int4_unpack(_ptr(w), _ptr(q), K, N)
    return q


# ---------------------------------------------------------------- W4A16

def w4a16(A, W, S, G, want_f64=False):
    """Y = fp16(A @ dequant(W, S)) with fp64 sums; A fp16 [M,K], W uint8 [K,N/2],
    S fp16 [ceil(K/G),N]."""
    A = _c(A, np.float16)
    W = _c(W, np.uint8)
    S = _c(S, np.float16)
    M, K = A.shape
    N = S.shape[1]
    assert W.shape == (K, N // 2) and S.shape == (-(-K // G), N)
    Y = np.empty((M, N), np.float16)
    Y64 = np.empty((M, N), np.float64) if want_f64 else None
    _load().qo_w4a16(_ptr(A), _ptr(W), _ptr(S), _ptr(Y), _ptr(Y64), M, N, K, G)
    return (Y, Y64) if want_f64 else Y


def w4a16_at(A, W, S, G, ms, ns, want_f64=False):
    A = _c(A, np.float16)
    W = _c(W, np.uint8)
    S = _c(S, np.float16)
    M, K = A.shape
    N = S.shape[1]
    ms = _c(np.asarray(ms, np.int32), np.int32)
    ns = _c(np.asarray(ns, np.int32), np.int32)
    assert ms.shape == ns.shape
    assert ms.size == 0 or (ms.min() >= 0 and ms.max() < M and ns.min() >= 0 and ns.max() < N)
    y = np.empty(ms.shape, np.float16)
    y64 = np.empty(ms.shape, np.float64) if want_f64 else None
    _load().qo_w4a16_at(_ptr(A), _ptr(W), _ptr(S), _ptr(ms), _ptr(ns), ms.size, _ptr(y),
                        _ptr(y64), M, N, K, G)
    return (y, y64) if want_f64 else y


def frag_nibble_index(K, k, n):
    return _load().qo_frag_nibble_index(K, k, n)


def w4a16_prepack(W, K, N):
    """Fragment-layout bytes (padded to whole 128 x 128 tiles) of natural int4 W [K][N/2]."""
    W = _c(W, np.uint8)
    assert W.size == K * N // 2 and N % 2 == 0
    F = np.empty(_load().qo_w4a16_packed_bytes(K, N), np.uint8)
    _load().qo_w4a16_prepack(_ptr(W), _ptr(F), K, N)
    return F


# ---------------------------------------------------------------- W8A16

def w8a16(A, W, S, G, want_f64=False):
    """Y = fp16(A @ (W * S)) with fp64 sums; A fp16 [M,K], W int8 [K,N], S fp16 [ceil(K/G),N]
    (G == K: one scale per column)."""
    A = _c(A, np.float16)
    W = _c(W, np.int8)
    S = _c(S, np.float16)
    M, K = A.shape
    N = W.shape[1]
    assert W.shape == (K, N) and S.shape == (-(-K // G), N)
    Y = np.empty((M, N), np.float16)
    Y64 = np.empty((M, N), np.float64) if want_f64 else None
    _load().qo_w8a16(_ptr(A), _ptr(W), _ptr(S), _ptr(Y), _ptr(Y64), M, N, K, G)
    return (Y, Y64) if want_f64 else Y


def w8a16_at(A, W, S, G, ms, ns, want_f64=False):
    A = _c(A, np.float16)
    W = _c(W, np.int8)
    S = _c(S, np.float16)
    M, K = A.shape
    N = W.shape[1]
    assert W.shape == (K, N) and S.shape == (-(-K // G), N)
    ms = _c(np.asarray(ms, np.int32), np.int32)
    ns = _c(np.asarray(ns, np.int32), np.int32)
    assert ms.shape == ns.shape
    assert ms.size == 0 or (ms.min() >= 0 and ms.max() < M and ns.min() >= 0 and ns.max() < N)
    y = np.empty(ms.shape, np.float16)
    y64 = np.empty(ms.shape, np.float64) if want_f64 else None
    _load().qo_w8a16_at(_ptr(A), _ptr(W), _ptr(S), _ptr(ms), _ptr(ns), ms.size, _ptr(y), _ptr(y64),
                        N, K, G)
    return (y, y64) if want_f64 else y


def frag8_byte_index(K, k, n):
    return _load().qo_frag8_byte_index(K, k, n)


def w8a16_prepack(W, K, N):
    """Fragment-layout bytes (padded to whole 128 x 128 tiles) of int8 W [K][N]."""
    W = _c(W, np.int8)
    assert W.shape == (K, N)
    F = np.empty(_load().qo_w8a16_packed_bytes(K, N), np.uint8)
    _load().qo_w8a16_prepack(_ptr(W), _ptr(F), K, N)
    return F


# ---------------------------------------------------------------- int8 quant

def quant_sym_int8(X):
    X = _c(X, np.float16)
    rows, cols = X.reshape(-1, X.shape[-1]).shape
    Q = np.empty(X.shape, np.int8)
    S = np.empty(rows, np.float32)
    _load().qo_quant_sym_int8(_ptr(X), _ptr(Q), _ptr(S), rows, cols)
    return Q, S


def dequant_sym_int8(Q, S):
    Q = _c(Q, np.int8)
    S = _c(S, np.float32)
    rows, cols = Q.reshape(-1, Q.shape[-1]).shape
    assert S.size == rows
    X = np.empty(Q.shape, np.float16)
    _load().qo_dequant_sym_int8(_ptr(Q), _ptr(S), _ptr(X), rows, cols)
    return X


# ---------------------------------------------------------------- FP8 E4M3

def e4m3_to_f64(codes):
    b = _c(codes, np.uint8)
    out = np.empty(b.shape, np.float64)
    _load().qo_e4m3_to_f64_array(_ptr(b), _ptr(out), b.size)
    return out


def f64_to_e4m3(x):
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint8)
    _load().qo_f64_to_e4m3_array(_ptr(x), _ptr(out), x.size)
    return out


def quant_fp8(X, per_row=True):
    """Codes uint8 [rows][cols] and scales fp32 ([rows] per row, [1] per tensor)."""
    X = _c(X, np.float16)
    rows, cols = X.reshape(-1, X.shape[-1]).shape
    Q = np.empty(X.shape, np.uint8)
    S = np.empty(rows if per_row else 1, np.float32)
    _load().qo_quant_fp8(_ptr(X), _ptr(Q), _ptr(S), rows, cols, 1 if per_row else 0)
    return Q, S


def dequant_fp8(Q, S, per_row=True):
    Q = _c(Q, np.uint8)
    S = _c(S, np.float32)
    rows, cols = Q.reshape(-1, Q.shape[-1]).shape
    assert S.size == (rows if per_row else 1)
    X = np.empty(Q.shape, np.float16)
    _load().qo_dequant_fp8(_ptr(Q), _ptr(S), _ptr(X), rows, cols, 1 if per_row else 0)
    return X


def fp8_gemm(A, W, sa, sw, want_f64=False):
    """A e4m3 codes [M][K], W e4m3 codes [N][K]; sa of size M or 1, sw of size N or 1."""
    A = _c(A, np.uint8)
    W = _c(W, np.uint8)
    sa = _c(sa, np.float32).ravel()
    sw = _c(sw, np.float32).ravel()
    M, K = A.shape
    N = W.shape[0]
    assert W.shape[1] == K and sa.size in (1, M) and sw.size in (1, N)
    Y = np.empty((M, N), np.float16)
    Y64 = np.empty((M, N), np.float64) if want_f64 else None
    _load().qo_fp8_gemm(_ptr(A), _ptr(W), _ptr(sa), int(sa.size == M and M > 1), _ptr(sw),
                        int(sw.size == N and N > 1), _ptr(Y), _ptr(Y64), M, N, K)
    return (Y, Y64) if want_f64 else Y


def fp8_gemm_at(A, W, sa, sw, ms, ns):
    A = _c(A, np.uint8)
    W = _c(W, np.uint8)
    sa = _c(sa, np.float32).ravel()
    sw = _c(sw, np.float32).ravel()
    ms = _c(ms, np.int32)
    ns = _c(ns, np.int32)
    M, K = A.shape
    N = W.shape[0]
    Y = np.empty(ms.size, np.float16)
    _load().qo_fp8_gemm_at(_ptr(A), _ptr(W), _ptr(sa), int(sa.size == M and M > 1), _ptr(sw),
                           int(sw.size == N and N > 1), ms.size, _ptr(ms), _ptr(ns), _ptr(Y), K)
    return Y


# ---------------------------------------------------------------- W8A8

def w8a8_acc(A, W):
    A = _c(A, np.int8)
    W = _c(W, np.int8)
    M, K = A.shape
    N = W.shape[0]
    assert W.shape[1] == K
    acc = np.empty((M, N), np.int32)
    _load().qo_w8a8_acc(_ptr(A), _ptr(W), _ptr(acc), M, N, K)
    return acc


def gelu28(y):
    lib = _load()
    y = np.asarray(y, np.float32)
    return np.array([lib.qo_gelu28(float(v)) for v in y.ravel()], np.float32).reshape(y.shape)


def w8a8_requant(acc, sa, sw, bias_f16_bits, out_mult, flags):
    return int(_load().qo_w8a8_requant(int(acc), float(sa), float(sw), int(bias_f16_bits),
                                       float(out_mult), int(flags)))


def w8a8_epilogue(A, W, sa, sw, bias, out_mult, flags, want_acc=False):
    A = _c(A, np.int8)
    W = _c(W, np.int8)
    sa = _c(sa, np.float32)
    sw = _c(sw, np.float32)
    bias = None if bias is None else _c(bias, np.float16)
    M, K = A.shape
    N = W.shape[0]
    Y = np.empty((M, N), np.int8)
    acc = np.empty((M, N), np.int32) if want_acc else None
    _load().qo_w8a8_epilogue(_ptr(A), _ptr(W), _ptr(sa), _ptr(sw), _ptr(bias),
                             float(np.float32(out_mult)), flags, _ptr(Y), _ptr(acc), M, N, K)
    return (Y, acc) if want_acc else Y


def w8a8_epilogue_at(A, W, sa, sw, bias, out_mult, flags, ms, ns):
    A = _c(A, np.int8)
    W = _c(W, np.int8)
    sa = _c(sa, np.float32)
    sw = _c(sw, np.float32)
    bias = None if bias is None else _c(bias, np.float16)
    K = A.shape[1]
    ms = _c(np.asarray(ms, np.int32), np.int32)
    ns = _c(np.asarray(ns, np.int32), np.int32)
    y = np.empty(ms.shape, np.int8)
    acc = np.empty(ms.shape, np.int32)
    _load().qo_w8a8_epilogue_at(_ptr(A), _ptr(W), _ptr(sa), _ptr(sw), _ptr(bias),
                                float(np.float32(out_mult)), flags, _ptr(ms), _ptr(ns), ms.size,
                                _ptr(y), _ptr(acc), K)
    return y, acc


# ---------------------------------------------------------------- MoE

def moe_route(logits, topK):
    logits = _c(logits, np.float16)
    T, E = logits.shape
    ids = np.empty((T, topK), np.int32)
    w = np.empty((T, topK), np.float64)
    _load().qo_moe_route(_ptr(logits), T, E, topK, _ptr(ids), _ptr(w))
    return ids, w


def moe_permute(ids, E):
    ids = _c(ids, np.int32)
    T, topK = ids.shape
    offsets = np.empty(E + 1, np.int32)
    pairs = np.empty(T * topK, np.int32)
    _load().qo_moe_permute(_ptr(ids), T, topK, E, _ptr(offsets), _ptr(pairs))
    return offsets, pairs


MOE_SILU, MOE_GELU_ERF, MOE_GELU_TANH, MOE_RELU = 0, 1, 2, 3


def moe_act(z, activation):
    """The gate activation of the gated expert FFN, in fp64 (0 SiLU, 1 GELU erf form,
    2 GELU tanh form, 3 ReLU)."""
    return _load().qo_moe_act(float(z), int(activation))


def moe(X, logits, Wg, Wu, Wd, Sg, Su, Sd, topK, G, tokens=None, want_f64=False, activation=0):
    """Gated INT4 MoE, h = fp16(act(g) * u).  Wg/Wu uint8 [E,H,I/2], Wd uint8 [E,I,H/2];
    Sg/Su fp16 [E,H/G,I], Sd fp16 [E,I/G,H].  Returns (Y, ids, w[, Y64]);
    with ``tokens`` only those rows of Y are computed (others are zero)."""
    X = _c(X, np.float16)
    logits = _c(logits, np.float16)
    T, H = X.shape
    E = logits.shape[1]
    I = Sg.shape[2]
    Wg, Wu, Wd = (_c(a, np.uint8) for a in (Wg, Wu, Wd))
    Sg, Su, Sd = (_c(a, np.float16) for a in (Sg, Su, Sd))
    assert Wg.size == E * H * I // 2 and Wu.size == Wg.size and Wd.size == Wg.size
    assert Sg.shape == (E, H // G, I) and Su.shape == Sg.shape and Sd.shape == (E, I // G, H)
    Y = np.zeros((T, H), np.float16)
    Y64 = np.zeros((T, H), np.float64) if want_f64 else None
    ids = np.empty((T, topK), np.int32)
    w = np.empty((T, topK), np.float64)
    tok = None if tokens is None else _c(np.asarray(tokens, np.int32), np.int32)
    _load().qo_moe(_ptr(X), _ptr(logits), _ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(Sg), _ptr(Su),
                   _ptr(Sd), _ptr(Y), _ptr(Y64), _ptr(ids), _ptr(w), T, H, I, E, topK, G,
                   int(activation), _ptr(tok), 0 if tok is None else tok.size)
    return (Y, ids, w, Y64) if want_f64 else (Y, ids, w)


# ---------------------------------------------------------------- INT8 attention chain

def _heads(heads, B, H):
    heads = np.arange(B * H, dtype=np.int32) if heads is None else np.asarray(heads, np.int32)
    assert heads.ndim == 1 and (heads.size == 0 or (heads.min() >= 0 and heads.max() < B * H))
    return _c(heads, np.int32)


def mha_int8_probs(Q, K, alpha, heads=None):
    """S int32, P int8 and R = 127 p (fp64), each [len(heads), Lq, Lk], for the listed heads
    (b * H + h; default all) of Q [B, Lq, H, D], K [B, Lk, H, D] int8."""
    Q = _c(Q, np.int8)
    K = _c(K, np.int8)
    B, Lq, H, D = Q.shape
    Lk = K.shape[1]
    assert K.shape == (B, Lk, H, D)
    hs = _heads(heads, B, H)
    S = np.empty((hs.size, Lq, Lk), np.int32)
    P = np.empty((hs.size, Lq, Lk), np.int8)
    R = np.empty((hs.size, Lq, Lk), np.float64)
    _load().qo_mha_int8_probs(_ptr(Q), _ptr(K), _ptr(hs), hs.size, H, Lq, Lk, D, float(np.float32(alpha)),
                              _ptr(S), _ptr(P), _ptr(R))
    return S, P, R


def mha_int8_out(P, V, bias, pv_scale, out_mult, flags, Lq, heads=None, O=None):
    """O int8 [B, Lq, H, D] of the listed heads from their probabilities P [len(heads), Lq, Lk];
    other heads of O (zeros when O is None) are left as they are."""
    V = _c(V, np.int8)
    B, Lk, H, D = V.shape
    hs = _heads(heads, B, H)
    P = _c(P, np.int8)
    assert P.shape == (hs.size, Lq, Lk)
    bias = _c(np.zeros(H * D, np.float16) if bias is None else bias, np.float16)
    assert bias.size == H * D
    if O is None:
        O = np.zeros((B, Lq, H, D), np.int8)
    O = _c(O, np.int8)
    _load().qo_mha_int8_out(_ptr(P), _ptr(V), _ptr(bias), _ptr(hs), hs.size, H, Lq, Lk, D,
                            float(np.float32(pv_scale)), float(np.float32(out_mult)), int(flags), _ptr(O))
    return O


def mha_int8(Q, K, V, bias, alpha, pv_scale, out_mult, flags, heads=None):
    """The whole chain: (O, S, P, R) for the listed heads (O holds zeros for the others)."""
    S, P, R = mha_int8_probs(Q, K, alpha, heads)
    O = mha_int8_out(P, V, bias, pv_scale, out_mult, flags, Q.shape[1], heads)
    return O, S, P, R
