"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Random draws only: nothing here quantizes, dequantizes, multiplies or
reorders.  Signed int4 weights uniform in [-8, 7], packed two per byte, are
exactly uniform random bytes, so weights are drawn as bytes in the natural
layout ``uint8 [K][N/2]`` (low nibble = even column).

All generators use numpy ``Generator(PCG64(seed))``; fp16 values are drawn in
float64 and converted with ``astype(float16)``.  Draw order: activations,
weights, scales, then the rest.
"""
import math

import numpy as np


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def groups(K, G):
    """Scale rows of a K-deep weight matrix with group size G: ceil(K / G)."""
    return -(-K // G)


def w4a16_weights(K, N, G, seed):
    """int4 weights (natural packed bytes) and fp16 group scales U[0.005, 0.02]."""
    r = rng(seed)
    W = r.integers(0, 256, size=(K, N // 2), dtype=np.uint8)
    S = r.uniform(0.005, 0.02, size=(groups(K, G), N)).astype(np.float16)
    return W, S


def activations(M, K, seed):
    """fp16 activations ~ N(0, 1)."""
    return rng(seed).standard_normal((M, K)).astype(np.float16)


def w4a16_problem(M, K, N, G, seed):
    r = rng(seed)
    A = r.standard_normal((M, K)).astype(np.float16)
    W = r.integers(0, 256, size=(K, N // 2), dtype=np.uint8)
    S = r.uniform(0.005, 0.02, size=(groups(K, G), N)).astype(np.float16)
    return A, W, S


def w8a16_problem(M, K, N, G, seed):
    """fp16 activations ~ N(0, 1); int8 weights [K][N] uniform over [-128, 127]
    (random bytes); fp16 scales [ceil(K/G)][N] U[0.0005, 0.002] (G == K: per column)."""
    r = rng(seed)
    A = r.standard_normal((M, K)).astype(np.float16)
    W = r.integers(0, 256, size=(K, N), dtype=np.uint8).view(np.int8)
    S = r.uniform(0.0005, 0.002, size=(groups(K, G), N)).astype(np.float16)
    return A, W, S


def mha_problem(B, Lq, Lk, H, D, seed):
    """INT8 attention inputs: Q [B, Lq, H, D], K and V [B, Lk, H, D] int8 drawn as N(0, 32^2)
    rounded and clipped to [-127, 127] (the codes N(0, 1) data gets with amax = 4 sigma); fp16
    bias [H * D] ~ N(0, 0.02^2); and the recipe's fp32 factors: alpha = (4/127)^2 / sqrt(D)
    (logits of unit spread), pv_scale = (1/127) (4/127), out_mult = 127 / 0.3."""
    r = rng(seed)
    Q = np.clip(np.rint(r.normal(0.0, 32.0, (B, Lq, H, D))), -127, 127).astype(np.int8)
    K = np.clip(np.rint(r.normal(0.0, 32.0, (B, Lk, H, D))), -127, 127).astype(np.int8)
    V = np.clip(np.rint(r.normal(0.0, 32.0, (B, Lk, H, D))), -127, 127).astype(np.int8)
    bias = r.normal(0.0, 0.02, H * D).astype(np.float16)
    alpha = np.float32((4.0 / 127.0) ** 2 / math.sqrt(D))
    pv_scale = np.float32((1.0 / 127.0) * (4.0 / 127.0))
    out_mult = np.float32(127.0 / 0.3)
    return Q, K, V, bias, alpha, pv_scale, out_mult


def w8a8_problem(M, N, K, seed):
    """fp16 activations X [M,K] and weights Wf [N,K] ~ N(0,1); bias [N] ~ N(0, 0.1^2);
    the static output multiplier of the recipe, 127 / (4 sqrt(K)) in fp32."""
    r = rng(seed)
    X = r.standard_normal((M, K)).astype(np.float16)
    Wf = r.standard_normal((N, K)).astype(np.float16)
    bias = (0.1 * r.standard_normal(N)).astype(np.float16)
    out_mult = np.float32(127.0 / (4.0 * math.sqrt(K)))
    return X, Wf, bias, out_mult


def kv_problem(heads, seq, dim, seed):
    """KV-cache block fp16 [heads, seq, dim] uniform in [-0.5, 0.5)."""
    return rng(seed).uniform(-0.5, 0.5, size=(heads, seq, dim)).astype(np.float16)


def moe_problem(T, H, I, E, G, seed):
    """Hidden states X [T,H] and router logits [T,E] ~ N(0,1) fp16; per-expert
    natural int4 gate/up [E,H,I/2], down [E,I,H/2]; scales U[0.005, 0.02]."""
    r = rng(seed)
    X = r.standard_normal((T, H)).astype(np.float16)
    logits = r.standard_normal((T, E)).astype(np.float16)
    Wg = r.integers(0, 256, size=(E, H, I // 2), dtype=np.uint8)
    Wu = r.integers(0, 256, size=(E, H, I // 2), dtype=np.uint8)
    Wd = r.integers(0, 256, size=(E, I, H // 2), dtype=np.uint8)
    Sg = r.uniform(0.005, 0.02, size=(E, H // G, I)).astype(np.float16)
    Su = r.uniform(0.005, 0.02, size=(E, H // G, I)).astype(np.float16)
    Sd = r.uniform(0.005, 0.02, size=(E, I // G, H)).astype(np.float16)
    return X, logits, Wg, Wu, Wd, Sg, Su, Sd


def sample_positions(M, N, count, seed):
    """Output positions to check at full size: the four corners plus uniform draws."""
    r = rng(seed)
    ms = list(r.integers(0, M, size=count))
    ns = list(r.integers(0, N, size=count))
    ms += [0, 0, M - 1, M - 1]
    ns += [0, N - 1, 0, N - 1]
    return np.array(ms, np.int32), np.array(ns, np.int32)
