"""Python binding for libqgemm (HIP, gfx950) -- argument marshalling only.

Every function has the name of the C entry point it calls (include/libqgemm.h)
and takes torch tensors that live on the GPU; the work itself runs in the
library's kernels on ``torch.cuda.current_stream()``.  Outputs may be passed
in (no allocation then) or are allocated here with ``torch.empty``.  A non-zero
status raises ``QGemmError``.  There is no fallback: without the built
library (``python -m bit_quantized_gemm_qgemm_amd.build``) every call raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# QGEMM_LIB: another build of the same sources (e.g. the host-sanitizer build)
LIB_PATH = os.environ.get("QGEMM_LIB") or os.path.join(_HERE, "libqgemm.so")

OK = 0
NULL_PTR = 1
BAD_SHAPE = 2
MISALIGNED = 3
WORKSPACE_TOO_SMALL = 4
UNSUPPORTED = 5
HIP_ERROR = 6

EPI_BIAS = 1
EPI_GELU = 2

MOE_ACT_SILU = 0
MOE_ACT_GELU_ERF = 1
MOE_ACT_GELU_TANH = 2
MOE_ACT_RELU = 3

FP8_PER_TENSOR = 0
FP8_PER_ROW = 1

TACTIC_DEFAULT = 0
QGEMM_W4A16_TACTIC_DECODE_NARROW = 1
QGEMM_W4A16_TACTIC_DECODE_BALANCED = 2
QGEMM_W4A16_TACTIC_SPLITK = 3
QGEMM_W4A16_TACTIC_PREFILL = 4
QGEMM_W4A16_TACTIC_PREFILL_LARGE = 5

_lib = None


class QGemmError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({qgemm_status_str(status)})")


def _hip_runtimes_loaded():
    with open("/proc/self/maps") as f:
        return sorted({line.split()[-1] for line in f if "libamdhip64" in line})


def lib():
    """Load libqgemm.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run bit_quantized_gemm_qgemm_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    rts = _hip_runtimes_loaded()
    if len(rts) > 1:
        raise RuntimeError(f"two HIP runtimes in one process: {rts}")
    _declare(L)
    _lib = L
    return L


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t


def _declare(L):
    sig = {
        "qgemm_abi_version": (_I32, []),
        "qgemm_status_str": (ctypes.c_char_p, [_I32]),
        "qgemm_w4a16_packed_bytes": (_SZ, [_I32, _I32]),
        "qgemm_w4a16_prepack": (_I32, [_P, _P, _I32, _I32, _P]),
        "qgemm_w4a16_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
        "qgemm_w4a16": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _SZ, _P]),
        "mha_int8": (_I32, [_P] * 7 + [_I32] * 5 + [ctypes.c_float] * 3 + [ctypes.c_uint32, _P]),
        "qgemm_w4a16_tactics": (_I32, [_I32, _I32, _I32, _I32, _P, _I32]),
        "qgemm_w4a16_tactic_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
        "qgemm_w4a16_tactic": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _SZ, _P]),
        "qgemm_w4a16_autotune": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _SZ, _I32, _P, _P, _P]),
        "qgemm_w8a16_packed_bytes": (_SZ, [_I32, _I32]),
        "qgemm_w8a16_prepack": (_I32, [_P, _P, _I32, _I32, _P]),
        "qgemm_w8a16_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
        "qgemm_w8a16": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _SZ, _P]),
        "quant_sym_int8": (_I32, [_P, _P, _P, _I32, _I32, _P]),
        "dequant_sym_int8": (_I32, [_P, _P, _P, _I32, _I32, _P]),
        "qgemm_w8a8_epilogue": (_I32, [_P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_uint32, _P, _P,
                                       _I32, _I32, _I32, _P]),
        "moe_w4a16_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
        "moe_w4a16": (_I32, [_P] * 11 + [_I32] * 7 + [_P, _SZ, _P]),
        "moe_w4a16_no_alloc": (_I32, [_P] * 11 + [_I32] * 7 + [_P]),
        "qgemm_stream_read": (_I32, [_P, _SZ, _P, _P]),
        "qgemm_stream_copy": (_I32, [_P, _SZ, _P, _SZ, _P]),
        "quant_fp8_e4m3": (_I32, [_P, _P, _P, _I32, _I32, _I32, _P]),
        "dequant_fp8_e4m3": (_I32, [_P, _P, _P, _I32, _I32, _I32, _P]),
        "qgemm_fp8": (_I32, [_P, _P, _P, _I32, _P, _I32, _P, _I32, _I32, _I32, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


EXPORTS = ("qgemm_abi_version", "qgemm_status_str", "qgemm_w4a16_packed_bytes",
           "qgemm_w4a16_prepack", "qgemm_w4a16_workspace_bytes", "qgemm_w4a16", "quant_sym_int8",
           "dequant_sym_int8", "qgemm_w8a8_epilogue", "moe_w4a16_workspace_bytes", "moe_w4a16",
           "quant_fp8_e4m3", "dequant_fp8_e4m3", "qgemm_fp8", "qgemm_w8a16_packed_bytes",
           "qgemm_w8a16_prepack", "qgemm_w8a16_workspace_bytes", "qgemm_w8a16", "mha_int8",
           "qgemm_w4a16_tactics", "qgemm_w4a16_tactic_workspace_bytes", "qgemm_w4a16_tactic",
           "qgemm_w4a16_autotune", "moe_w4a16_no_alloc", "qgemm_stream_read", "qgemm_stream_copy")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check(fn, status):
    if status != OK:
        raise QGemmError(fn, status)


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name}: expected a contiguous CUDA tensor of {dtype}")
    return t


# ---------------------------------------------------------------- ABI

def qgemm_abi_version():
    return lib().qgemm_abi_version()


def qgemm_status_str(status):
    return lib().qgemm_status_str(int(status)).decode()


# ---------------------------------------------------------------- W4A16

def qgemm_w4a16_packed_bytes(K, N):
    return lib().qgemm_w4a16_packed_bytes(K, N)


def qgemm_w4a16_prepack(w_natural, K, N, w_frag=None):
    """Natural int4 bytes uint8 [K, N/2] -> fragment-layout bytes uint8 [K*N/2]."""
    _need(w_natural, torch.uint8, "w_natural")
    if w_frag is None:
        w_frag = torch.empty(max(qgemm_w4a16_packed_bytes(K, N), 1), dtype=torch.uint8,
                             device=w_natural.device)
    _need(w_frag, torch.uint8, "w_frag")
    _check("qgemm_w4a16_prepack",
           lib().qgemm_w4a16_prepack(_ptr(w_natural), _ptr(w_frag), K, N, _stream()))
    return w_frag


def qgemm_w4a16_workspace_bytes(M, N, K, G):
    return lib().qgemm_w4a16_workspace_bytes(M, N, K, G)


def qgemm_w4a16(A, w_frag, scales, G, N=None, Y=None, workspace=None, tactic=0):
    """Y[M, N] = A[M, K] (fp16) x dequant(w_frag, scales [K/G, N] fp16).  Without a
    workspace the one the library asks for (for the tactic) is allocated here; an
    empty tensor selects the kernels that need none.  tactic: 0 = the library's
    choice, an id from qgemm_w4a16_tactics, or "auto" = the fastest id found by
    qgemm_w4a16_autotune for this shape (tuned on first use, then remembered)."""
    _need(A, torch.float16, "A")
    _need(w_frag, torch.uint8, "w_frag")
    _need(scales, torch.float16, "scales")
    M, K = A.shape
    N = scales.shape[1] if N is None else N
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=A.device)
    _need(Y, torch.float16, "Y")
    if tactic == "auto":
        tactic = _TUNED.get((M, N, K, G))
        if tactic is None:
            tactic = qgemm_w4a16_autotune(A, w_frag, scales, G, N=N)[0] if M else 0
    if workspace is None:
        need = qgemm_w4a16_tactic_workspace_bytes(M, N, K, G, tactic)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=A.device)
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("qgemm_w4a16", lib().qgemm_w4a16_tactic(_ptr(A), _ptr(w_frag), _ptr(scales), _ptr(Y), M, N, K, G,
                                                    int(tactic), _ptr(workspace) if ws else None, ws, _stream()))
    return Y


_TUNED = {}


def qgemm_w4a16_tactics(M, N, K, G):
    """Ids of the W4A16 kernels valid for the shape (ascending)."""
    n = lib().qgemm_w4a16_tactics(M, N, K, G, None, 0)
    buf = (ctypes.c_int32 * max(n, 1))()
    lib().qgemm_w4a16_tactics(M, N, K, G, buf, n)
    return list(buf[:n])


def qgemm_w4a16_tactic_workspace_bytes(M, N, K, G, tactic):
    return lib().qgemm_w4a16_tactic_workspace_bytes(M, N, K, G, int(tactic))


def qgemm_w4a16_autotune(A, w_frag, scales, G, N=None, reps=20):
    """Times every valid tactic on these operands (the library's autotune call)
    and remembers the fastest for the shape; returns (tactic, us per launch)."""
    _need(A, torch.float16, "A")
    M, K = A.shape
    N = scales.shape[1] if N is None else N
    Y = torch.empty((M, N), dtype=torch.float16, device=A.device)
    need = qgemm_w4a16_tactic_workspace_bytes(M, N, K, G, QGEMM_W4A16_TACTIC_SPLITK)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=A.device)
    best = ctypes.c_int32(0)
    us = ctypes.c_float(0.0)
    _check("qgemm_w4a16_autotune",
           lib().qgemm_w4a16_autotune(_ptr(A), _ptr(w_frag), _ptr(scales), _ptr(Y), M, N, K, G, _ptr(ws),
                                      ws.numel(), int(reps), ctypes.byref(best), ctypes.byref(us), _stream()))
    _TUNED[(M, N, K, G)] = best.value
    return best.value, us.value


# ---------------------------------------------------------------- W8A16

def qgemm_w8a16_packed_bytes(K, N):
    return lib().qgemm_w8a16_packed_bytes(K, N)


def qgemm_w8a16_prepack(w_natural, K, N, w_frag=None):
    """Natural int8 weights [K, N] -> int8 fragment-layout bytes uint8 [K*N]."""
    _need(w_natural, torch.int8, "w_natural")
    if w_frag is None:
        w_frag = torch.empty(max(qgemm_w8a16_packed_bytes(K, N), 1), dtype=torch.uint8,
                             device=w_natural.device)
    _need(w_frag, torch.uint8, "w_frag")
    _check("qgemm_w8a16_prepack",
           lib().qgemm_w8a16_prepack(_ptr(w_natural), _ptr(w_frag), K, N, _stream()))
    return w_frag


def qgemm_w8a16_workspace_bytes(M, N, K, G):
    return lib().qgemm_w8a16_workspace_bytes(M, N, K, G)


def qgemm_w8a16(A, w_frag, scales, G, N=None, Y=None, workspace=None):
    """Y[M, N] = A[M, K] (fp16) x (W * scales), W int8 from w_frag, scales fp16
    [K/G, N] (G == K: [1, N], one per column).  Workspace as for qgemm_w4a16."""
    _need(A, torch.float16, "A")
    _need(w_frag, torch.uint8, "w_frag")
    _need(scales, torch.float16, "scales")
    M, K = A.shape
    N = scales.shape[1] if N is None else N
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=A.device)
    _need(Y, torch.float16, "Y")
    if workspace is None:
        need = qgemm_w8a16_workspace_bytes(M, N, K, G)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=A.device)
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("qgemm_w8a16", lib().qgemm_w8a16(_ptr(A), _ptr(w_frag), _ptr(scales), _ptr(Y), M, N, K, G,
                                             _ptr(workspace) if ws else None, ws, _stream()))
    return Y


# ---------------------------------------------------------------- int8 quant

def quant_sym_int8(X, Q=None, scales=None):
    """Per-row symmetric int8 codes and fp32 dequant scales of fp16 X [..., cols]."""
    _need(X, torch.float16, "X")
    cols = X.shape[-1]
    rows = X.numel() // cols if cols else 0
    if Q is None:
        Q = torch.empty(X.shape, dtype=torch.int8, device=X.device)
    if scales is None:
        scales = torch.empty(max(rows, 1), dtype=torch.float32, device=X.device)[:rows]
    _need(Q, torch.int8, "Q")
    _need(scales, torch.float32, "scales")
    _check("quant_sym_int8",
           lib().quant_sym_int8(_ptr(X), _ptr(Q), _ptr(scales), rows, cols, _stream()))
    return Q, scales


def dequant_sym_int8(Q, scales, X=None):
    _need(Q, torch.int8, "Q")
    _need(scales, torch.float32, "scales")
    cols = Q.shape[-1]
    rows = Q.numel() // cols if cols else 0
    if X is None:
        X = torch.empty(Q.shape, dtype=torch.float16, device=Q.device)
    _need(X, torch.float16, "X")
    _check("dequant_sym_int8",
           lib().dequant_sym_int8(_ptr(Q), _ptr(scales), _ptr(X), rows, cols, _stream()))
    return X


# ---------------------------------------------------------------- W8A8

def qgemm_w8a8_epilogue(A, W, a_scale, w_scale, bias, out_mult, flags, Y=None, acc_out=None):
    """int8 Y[M, N] from int8 A [M, K], W [N, K] with the fused requantizing epilogue."""
    _need(A, torch.int8, "A")
    _need(W, torch.int8, "W")
    _need(a_scale, torch.float32, "a_scale")
    _need(w_scale, torch.float32, "w_scale")
    if bias is not None:
        _need(bias, torch.float16, "bias")
    M, K = A.shape
    N = W.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.int8, device=A.device)
    _need(Y, torch.int8, "Y")
    if acc_out is not None:
        _need(acc_out, torch.int32, "acc_out")
    _check("qgemm_w8a8_epilogue",
           lib().qgemm_w8a8_epilogue(_ptr(A), _ptr(W), _ptr(a_scale), _ptr(w_scale), _ptr(bias),
                                     float(out_mult), int(flags), _ptr(Y), _ptr(acc_out), M, N, K,
                                     _stream()))
    return Y


# ---------------------------------------------------------------- MoE

def moe_w4a16_workspace_bytes(T, H, I, E, topK):
    return lib().moe_w4a16_workspace_bytes(T, H, I, E, topK)


def moe_w4a16(X, logits, w_gate_frag, w_up_frag, w_down_frag, s_gate, s_up, s_down, topK, G,
              I=None, activation=0, Y=None, topk_ids=None, topk_w=None, workspace=None):
    """Gated INT4 MoE layer, h = fp16(act(g) * u) with act = MOE_ACT_SILU, MOE_ACT_GELU_ERF,
    MOE_ACT_GELU_TANH or MOE_ACT_RELU.  Returns (Y, topk_ids, topk_w, workspace)."""
    _need(X, torch.float16, "X")
    _need(logits, torch.float16, "logits")
    for name, t in (("w_gate_frag", w_gate_frag), ("w_up_frag", w_up_frag),
                    ("w_down_frag", w_down_frag)):
        _need(t, torch.uint8, name)
    for name, t in (("s_gate", s_gate), ("s_up", s_up), ("s_down", s_down)):
        _need(t, torch.float16, name)
    T, H = X.shape
    E = logits.shape[1]
    I = s_gate.shape[-1] if I is None else I
    dev = X.device
    if Y is None:
        Y = torch.empty((T, H), dtype=torch.float16, device=dev)
    if topk_ids is None:
        topk_ids = torch.empty((T, topK), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, topK), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(moe_w4a16_workspace_bytes(T, H, I, E, topK), 1),
                                dtype=torch.uint8, device=dev)
    _check("moe_w4a16",
           lib().moe_w4a16(_ptr(X), _ptr(logits), _ptr(w_gate_frag), _ptr(w_up_frag),
                           _ptr(w_down_frag), _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(Y),
                           _ptr(topk_ids), _ptr(topk_w), T, H, I, E, topK, G, activation,
                           _ptr(workspace), workspace.numel(), _stream()))
    return Y, topk_ids, topk_w, workspace


MOE_NO_ALLOC_SCRATCH_BYTES = 64 << 20


def moe_w4a16_no_alloc(X, logits, w_gate_frag, w_up_frag, w_down_frag, s_gate, s_up, s_down,
                       topK, G, Y, topk_ids, topk_w, I=None, activation=0):
    """moe_w4a16 on the library's per-GPU scratch array: every output is passed in and nothing
    is allocated.  Returns (Y, topk_ids, topk_w)."""
    _need(X, torch.float16, "X")
    _need(logits, torch.float16, "logits")
    for name, t in (("w_gate_frag", w_gate_frag), ("w_up_frag", w_up_frag),
                    ("w_down_frag", w_down_frag)):
        _need(t, torch.uint8, name)
    for name, t in (("s_gate", s_gate), ("s_up", s_up), ("s_down", s_down)):
        _need(t, torch.float16, name)
    _need(Y, torch.float16, "Y")
    _need(topk_ids, torch.int32, "topk_ids")
    _need(topk_w, torch.float32, "topk_w")
    T, H = X.shape
    E = logits.shape[1]
    I = s_gate.shape[-1] if I is None else I
    _check("moe_w4a16_no_alloc",
           lib().moe_w4a16_no_alloc(_ptr(X), _ptr(logits), _ptr(w_gate_frag), _ptr(w_up_frag),
                                    _ptr(w_down_frag), _ptr(s_gate), _ptr(s_up), _ptr(s_down),
                                    _ptr(Y), _ptr(topk_ids), _ptr(topk_w), T, H, I, E, topK, G,
                                    activation, _stream()))
    return Y, topk_ids, topk_w


# ---------------------------------------------------------------- FP8 E4M3

def quant_fp8_e4m3(X, per_row=True, Q=None, scales=None):
    """E4M3 codes (uint8) and fp32 scales ([rows] per row, [1] per tensor) of fp16 X [..., cols]."""
    _need(X, torch.float16, "X")
    cols = X.shape[-1]
    rows = X.numel() // cols if cols else 0
    if Q is None:
        Q = torch.empty(X.shape, dtype=torch.uint8, device=X.device)
    if scales is None:
        n = rows if per_row else 1
        scales = torch.empty(max(n, 1), dtype=torch.float32, device=X.device)[:n]
    _need(Q, torch.uint8, "Q")
    _need(scales, torch.float32, "scales")
    _check("quant_fp8_e4m3", lib().quant_fp8_e4m3(_ptr(X), _ptr(Q), _ptr(scales), rows, cols,
                                                   FP8_PER_ROW if per_row else FP8_PER_TENSOR, _stream()))
    return Q, scales


def dequant_fp8_e4m3(Q, scales, per_row=True, X=None):
    _need(Q, torch.uint8, "Q")
    _need(scales, torch.float32, "scales")
    cols = Q.shape[-1]
    rows = Q.numel() // cols if cols else 0
    if X is None:
        X = torch.empty(Q.shape, dtype=torch.float16, device=Q.device)
    _need(X, torch.float16, "X")
    _check("dequant_fp8_e4m3", lib().dequant_fp8_e4m3(_ptr(Q), _ptr(scales), _ptr(X), rows, cols,
                                                       FP8_PER_ROW if per_row else FP8_PER_TENSOR, _stream()))
    return X


def qgemm_fp8(A, W, a_scale, w_scale, Y=None):
    """fp16 Y[M, N] from E4M3 codes A [M, K] and W [N, K]; a scale vector of one
    element is per tensor, of M (N) elements per row (column)."""
    _need(A, torch.uint8, "A")
    _need(W, torch.uint8, "W")
    _need(a_scale, torch.float32, "a_scale")
    _need(w_scale, torch.float32, "w_scale")
    M, K = A.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("A and W disagree on K")
    a_per_row = 1 if (a_scale.numel() == M and M > 1) else 0
    w_per_row = 1 if (w_scale.numel() == N and N > 1) else 0
    if (not a_per_row and a_scale.numel() != 1) or (not w_per_row and w_scale.numel() != 1):
        raise ValueError("a scale vector must have one element or one per row / column")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=A.device)
    _need(Y, torch.float16, "Y")
    _check("qgemm_fp8", lib().qgemm_fp8(_ptr(A), _ptr(W), _ptr(a_scale), a_per_row, _ptr(w_scale),
                                         w_per_row, _ptr(Y), M, N, K, _stream()))
    return Y



# ---------------------------------------------------------------- INT8 attention chain

def mha_int8(Q, K, V, alpha, pv_scale, out_mult, bias=None, O=None, s_out=None, p_out=None):
    """O [B, Lq, H, D] int8 = requant(P V) with P = int8 softmax of Q K^T * alpha;
    Q [B, Lq, H, D], K and V [B, Lk, H, D] int8; bias fp16 [H * D] (applied when given).
    Optional s_out int32 / p_out int8 [B, H, Lq, Lk] receive the logits and the codes."""
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _need(t, torch.int8, n)
    B, Lq, H, D = Q.shape
    Lk = K.shape[1]
    if tuple(K.shape) != (B, Lk, H, D) or tuple(V.shape) != (B, Lk, H, D):
        raise ValueError("mha_int8: K and V must be [B, Lk, H, D] matching Q [B, Lq, H, D]")
    if bias is not None:
        _need(bias, torch.float16, "bias")
    if O is None:
        O = torch.empty((B, Lq, H, D), dtype=torch.int8, device=Q.device)
    _need(O, torch.int8, "O")
    if s_out is not None:
        _need(s_out, torch.int32, "s_out")
    if p_out is not None:
        _need(p_out, torch.int8, "p_out")
    flags = EPI_BIAS if bias is not None else 0
    _check("mha_int8", lib().mha_int8(_ptr(Q), _ptr(K), _ptr(V), _ptr(bias), _ptr(O), _ptr(s_out), _ptr(p_out),
                                      B, H, Lq, Lk, D, float(alpha), float(pv_scale), float(out_mult), flags,
                                      _stream()))
    return O


# ---------------------------------------------------------------- measurement aid

def qgemm_stream_read(buf, sink):
    """Read every byte of the CUDA tensor ``buf`` (a multiple of 16 bytes) with 16-byte loads;
    ``sink`` is a 1-element int32 tensor the kernel may write.  For bandwidth reference runs."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf: expected a contiguous CUDA tensor")
    _need(sink, torch.int32, "sink")
    _check("qgemm_stream_read", lib().qgemm_stream_read(_ptr(buf), buf.numel() * buf.element_size(),
                                                         _ptr(sink), _stream()))


def qgemm_stream_copy(src, dst):
    """Read every byte of the CUDA tensor ``src`` and write every byte of ``dst`` (one half or
    twice its size, multiples of 16 bytes) in the traffic shapes of the int8 quantizer and
    dequantizer (dst words: XOR of word pairs when halving, each word pair then the pair plus
    one when doubling).  For bandwidth reference runs."""
    for t, name in ((src, "src"), (dst, "dst")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name}: expected a contiguous CUDA tensor")
    _check("qgemm_stream_copy", lib().qgemm_stream_copy(_ptr(src), src.numel() * src.element_size(), _ptr(dst),
                                                         dst.numel() * dst.element_size(), _stream()))
