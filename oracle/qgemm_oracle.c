/*
 * qgemm_oracle.c -- plain, slow CPU oracle for the quantized-GEMM hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this library.  The HIP
 * library never includes, links or calls it, and this file includes nothing
 * from the HIP side.  It reads only the *natural* weight format
 * (int4 [K][N/2], low nibble = even column; int8 [K][N]), never the GPU
 * fragment layouts,
 * except in qo_w4a16_prepack and qo_w8a16_prepack, which write those
 * layouts from their written definitions so the GPU prepacks can be checked
 * byte for byte.
 *
 * Arithmetic rules:
 *   - fp16 <-> binary64 conversion is written here from IEEE 754 binary16
 *     (round to nearest, ties to even; subnormals kept; no hardware half type).
 *   - Dequantized weights q*s are exact in fp32 and fp64 (4-bit x 11-bit).
 *   - Every GEMM product and sum is formed in fp64 in ascending k order and
 *     rounded once, directly from fp64 to fp16, at the end.
 *   - Where a floating-point value decides an integer (int8 quantization,
 *     requantization), the steps are single IEEE fp32 operations in the order
 *     written below; built with -ffp-contract=off and without fast-math so
 *     the compiler neither fuses nor reorders them.
 *   - OpenMP splits work over output elements; each output is produced by
 *     exactly one thread in a fixed order, so results do not depend on the
 *     thread count.
 *
 * Sources (web pages this implements):
 *   [P1] Interview Q&A "INT8 cross-modal multi-head-attention TensorRT plugin"
 *        (cms365.cn): knowledge points 1-2 (INT8 data path; per-channel and
 *        per-token symmetric quantization; rescale + bias + GELU, then
 *        requantize), answer step 1 (scale = 127 / max|x|), knowledge point 5
 *        (saturation to [-127, 127]), answer steps 2-3 (the attention chain:
 *        QK^T, int8 softmax, P.V, requantization with bias).
 *   [P2] FP8 vs INT8 low-precision inference in TensorRT-LLM (itzkxy.com):
 *        FP8 E4M3 for GEMMs and the KV cache, per-tensor scaling factors
 *        derived from the activation A-max; the INT8 configurations it
 *        compares (weight-only int8 with fp16 activations among them).
 *   [P3] "Int4 Groupwise GEMM Plugin V2" (TensorRT-Edge-LLM C++ API docs):
 *        class summary (W4A16 group-wise GEMM; inputs: fp16 activations
 *        [b,seq,K], int4 weights, fp16 scales [ceil(K/G), N]; output fp16
 *        [b,seq,N]) and the constructor parameters (N = output dimension =
 *        weight columns, K = input dimension = weight rows, group size).
 *   [P4] "KV Cache INT8量化" (ainanfeng.cn): quantize_symmetric
 *        (scale = max|x| / 127, x_int8 = round(x / scale)) and
 *        dequantize_symmetric (x_fp16 = x_int8 * scale).
 *   [P5] "Int4 Moe Plugin" (TensorRT-Edge-LLM C++ API docs): constructor
 *        (numExperts, topK, hiddenSize, moeInterSize, activationType,
 *        quantizationGroupSize).
 */
#define _GNU_SOURCE
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QO_API __attribute__((visibility("default")))

/* Number of OpenMP threads the parallel loops below use. */
QO_API int qo_num_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16                                                        */
/* ------------------------------------------------------------------------ */

/* binary16 bit pattern -> exact binary64 value. */
QO_API double qo_f16_to_f64(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* binary64 -> binary16, round to nearest, ties to even, in one rounding. */
QO_API uint16_t qo_f64_to_f16(double x) {
    if (isnan(x)) return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2); /* a in [2^(e2-1), 2^e2) */
    if (e2 - 1 < -14) {
        /* subnormal range: quantum 2^-24; nearbyint uses the default mode,
           round-to-nearest-even.  n == 1024 is the smallest normal. */
        double n = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)n);
    }
    /* normal: 11 significant bits, quantum 2^(e2-11) */
    double n = nearbyint(ldexp(a, 11 - e2)); /* in [1024, 2048] */
    int exp_field = e2 + 14;                 /* (e2-1) + 15 */
    if (n >= 2048.0) {
        n = 1024.0;
        exp_field += 1;
    }
    if (exp_field >= 31) return (uint16_t)(sign | 0x7c00); /* overflow -> inf */
    return (uint16_t)(sign | (uint16_t)(exp_field << 10) | (uint16_t)((int)n - 1024));
}

QO_API void qo_f16_to_f64_array(const uint16_t* h, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = qo_f16_to_f64(h[i]);
}

QO_API void qo_f64_to_f16_array(const double* x, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = qo_f64_to_f16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Signed int4 in the natural layout: byte [k][n/2]; even n in bits 0-3,    */
/* odd n in bits 4-7; two's complement, so nibble 8 is -8.                  */
/* ------------------------------------------------------------------------ */

QO_API int qo_int4_at(const uint8_t* w, int32_t N, int32_t k, int32_t n) {
    const uint8_t b = w[(int64_t)k * (N / 2) + n / 2];
    const int v = (n & 1) ? (b >> 4) : (b & 0x0f);
    return v >= 8 ? v - 16 : v;
}

QO_API void qo_int4_unpack(const uint8_t* w, int8_t* q, int32_t K, int32_t N) {
    for (int32_t k = 0; k < K; ++k)
        for (int32_t n = 0; n < N; ++n) q[(int64_t)k * N + n] = (int8_t)qo_int4_at(w, N, k, n);
}

/* ------------------------------------------------------------------------ */
/* W4A16 group-wise GEMM  [P3 class summary]                                */
/*   Y[m][n] = fp16( sum_k A[m][k] * q(k,n) * S[k/G][n] ),  k ascending      */
/* A fp16 [M][K] row-major; W natural int4 [K][N/2]; S fp16 [ceil(K/G)][N]   */
/* (the last group may be shorter than G);                                  */
/* Y fp16 [M][N].  Y64 (optional) receives the unrounded fp64 sums.          */
/* ------------------------------------------------------------------------ */

QO_API void qo_w4a16(const uint16_t* A, const uint8_t* W, const uint16_t* S, uint16_t* Y,
                     double* Y64, int32_t M, int32_t N, int32_t K, int32_t G) {
    for (int32_t m = 0; m < M; ++m) {
        double* acc = (double*)calloc((size_t)N, sizeof(double));
        /* each thread owns a fixed range of columns; every column sums k in
           ascending order */
#pragma omp parallel for schedule(static)
        for (int32_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int32_t k = 0; k < K; ++k) {
                const double a = qo_f16_to_f64(A[(int64_t)m * K + k]);
                const double w = (double)qo_int4_at(W, N, k, n) *
                                 qo_f16_to_f64(S[(int64_t)(k / G) * N + n]);
                s += a * w;
            }
            acc[n] = s;
        }
        for (int32_t n = 0; n < N; ++n) {
            if (Y) Y[(int64_t)m * N + n] = qo_f64_to_f16(acc[n]);
            if (Y64) Y64[(int64_t)m * N + n] = acc[n];
        }
        free(acc);
    }
}

/* Same definition, evaluated only at the listed (m, n) positions. */
QO_API void qo_w4a16_at(const uint16_t* A, const uint8_t* W, const uint16_t* S,
                        const int32_t* ms, const int32_t* ns, int64_t count, uint16_t* y,
                        double* y64, int32_t M, int32_t N, int32_t K, int32_t G) {
    (void)M;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < count; ++i) {
        const int32_t m = ms[i], n = ns[i];
        double s = 0.0;
        for (int32_t k = 0; k < K; ++k) {
            const double a = qo_f16_to_f64(A[(int64_t)m * K + k]);
            const double w = (double)qo_int4_at(W, N, k, n) *
                             qo_f16_to_f64(S[(int64_t)(k / G) * N + n]);
            s += a * w;
        }
        if (y) y[i] = qo_f64_to_f16(s);
        if (y64) y64[i] = s;
    }
}

/* ------------------------------------------------------------------------ */
/* Weight prepack: natural int4 [K][N/2] -> the library's fragment layout.  */
/* Written from the layout definition, independent of the GPU code:         */
/*   weight block (16 columns x 128 k, 1024 bytes): strip s = n/16,          */
/*     chunk c = k/128;                                                      */
/*   tile (128 columns x 128 k, 8192 bytes) = 8 consecutive strips;          */
/*   block offset = ((s/8) * (K/128) + c) * 8192 + (s%8) * 1024;             */
/*   inside a block, with r = k%128, column cl = n%16:                       */
/*     kk = r/32, q = (r%32)/8, j = r%8;                                     */
/*     32-bit word at byte (cl + 16*q)*16 + 4*kk;                            */
/*     nibble position pos = j/2 + 4*(j%2) (bits 4*pos .. 4*pos+3);          */
/*     stored value (v + 8) & 15 (offset binary).                            */
/* K and N that are not multiples of 128 are padded to whole tiles (the      */
/* page's fragment rows = ceil(N/128) * ceil(K/64) * 8): the layout has      */
/* ceil(K/128) chunks per strip and ceil(N/128) tiles, and every padding     */
/* position holds the offset-binary code of weight 0 (nibble 8).             */
/* ------------------------------------------------------------------------ */

QO_API int64_t qo_frag_nibble_index(int32_t K, int32_t k, int32_t n) {
    const int32_t s = n / 16, cl = n % 16, c = k / 128, r = k % 128;
    const int32_t kk = r / 32, q = (r % 32) / 8, j = r % 8;
    const int64_t kchunks = (K + 127) / 128;
    const int64_t block = ((int64_t)(s / 8) * kchunks + c) * 8192 + (int64_t)(s % 8) * 1024;
    const int64_t word = block + (int64_t)(cl + 16 * q) * 16 + 4 * kk;
    const int32_t pos = j / 2 + 4 * (j % 2);
    return word * 2 + pos; /* nibble index: byte = idx/2, high nibble if idx odd */
}

/* Bytes of the padded layout: ceil(K/128)*128 x ceil(N/128)*128 nibbles. */
QO_API int64_t qo_w4a16_packed_bytes(int32_t K, int32_t N) {
    return ((int64_t)(K + 127) / 128) * 128 * (((int64_t)N + 127) / 128) * 128 / 2;
}

QO_API void qo_w4a16_prepack(const uint8_t* W, uint8_t* F, int32_t K, int32_t N) {
    memset(F, 0x88, (size_t)qo_w4a16_packed_bytes(K, N));
    for (int32_t k = 0; k < K; ++k)
        for (int32_t n = 0; n < N; ++n) {
            const int v = qo_int4_at(W, N, k, n);
            const uint8_t u = (uint8_t)((v + 8) & 15);
            const int64_t idx = qo_frag_nibble_index(K, k, n);
            F[idx / 2] = (idx & 1) ? (uint8_t)((F[idx / 2] & 0x0f) | (u << 4))
                                   : (uint8_t)((F[idx / 2] & 0xf0) | u);
        }
}

/* ------------------------------------------------------------------------ */
/* W8A16 weight-only int8 GEMM  [P2 INT8 configurations: int8 weight-only    */
/* quantization with fp16 activations]                                      */
/*   Y[m][n] = fp16( sum_k A[m][k] * W[k][n] * S[k/G][n] ),  k ascending     */
/* A fp16 [M][K]; W int8 [K][N] (two's complement, row-major); S fp16        */
/* [K/G][N]; G == K is one scale per output column (per channel).  Y fp16    */
/* [M][N]; Y64 (optional) receives the unrounded fp64 sums.                 */
/* ------------------------------------------------------------------------ */

static double qo_w8a16_dot(const uint16_t* A, const int8_t* W, const uint16_t* S, int32_t N,
                           int32_t K, int32_t G, int32_t m, int32_t n) {
    double s = 0.0;
    for (int32_t k = 0; k < K; ++k) {
        const double a = qo_f16_to_f64(A[(int64_t)m * K + k]);
        const double w = (double)W[(int64_t)k * N + n] * qo_f16_to_f64(S[(int64_t)(k / G) * N + n]);
        s += a * w;
    }
    return s;
}

QO_API void qo_w8a16(const uint16_t* A, const int8_t* W, const uint16_t* S, uint16_t* Y,
                     double* Y64, int32_t M, int32_t N, int32_t K, int32_t G) {
#pragma omp parallel for schedule(static) collapse(2)
    for (int32_t m = 0; m < M; ++m)
        for (int32_t n = 0; n < N; ++n) {
            const double s = qo_w8a16_dot(A, W, S, N, K, G, m, n);
            if (Y) Y[(int64_t)m * N + n] = qo_f64_to_f16(s);
            if (Y64) Y64[(int64_t)m * N + n] = s;
        }
}

QO_API void qo_w8a16_at(const uint16_t* A, const int8_t* W, const uint16_t* S,
                        const int32_t* ms, const int32_t* ns, int64_t count, uint16_t* y,
                        double* y64, int32_t N, int32_t K, int32_t G) {
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < count; ++i) {
        const double s = qo_w8a16_dot(A, W, S, N, K, G, ms[i], ns[i]);
        if (y) y[i] = qo_f64_to_f16(s);
        if (y64) y64[i] = s;
    }
}

/* ------------------------------------------------------------------------ */
/* Int8 weight prepack: natural int8 [K][N] -> the library's int8 fragment   */
/* layout, written from its definition:                                      */
/*   weight block (16 columns x 128 k, 2048 bytes): strip s = n/16,          */
/*     chunk c = k/128;                                                      */
/*   tile (128 columns x 128 k, 16384 bytes) = 8 consecutive strips;         */
/*   block offset = ((s/8) * (K/128) + c) * 16384 + (s%8) * 2048;            */
/*   inside a block, with r = k%128, column cl = n%16:                       */
/*     kk = r/32, q = (r%32)/8, j = r%8;                                     */
/*     byte (kk/2)*1024 + (cl + 16*q)*16 + (kk%2)*8 + j;                     */
/*     stored value v + 128 (offset binary).                                 */
/* The k of each byte is that of the int4 layout's nibble with the same      */
/* (block, cl, q, kk, j).  K and N are padded to whole 128 x 128 tiles as    */
/* for int4; padding bytes hold the offset-binary code of 0 (128).           */
/* ------------------------------------------------------------------------ */

QO_API int64_t qo_frag8_byte_index(int32_t K, int32_t k, int32_t n) {
    const int32_t s = n / 16, cl = n % 16, c = k / 128, r = k % 128;
    const int32_t kk = r / 32, q = (r % 32) / 8, j = r % 8;
    const int64_t kchunks = (K + 127) / 128;
    const int64_t block = ((int64_t)(s / 8) * kchunks + c) * 16384 + (int64_t)(s % 8) * 2048;
    return block + (int64_t)(kk / 2) * 1024 + (int64_t)(cl + 16 * q) * 16 + (kk % 2) * 8 + j;
}

QO_API int64_t qo_w8a16_packed_bytes(int32_t K, int32_t N) {
    return ((int64_t)(K + 127) / 128) * 128 * (((int64_t)N + 127) / 128) * 128;
}

QO_API void qo_w8a16_prepack(const int8_t* W, uint8_t* F, int32_t K, int32_t N) {
    memset(F, 128, (size_t)qo_w8a16_packed_bytes(K, N));
    for (int32_t k = 0; k < K; ++k)
        for (int32_t n = 0; n < N; ++n)
            F[qo_frag8_byte_index(K, k, n)] = (uint8_t)((int)W[(int64_t)k * N + n] + 128);
}

/* ------------------------------------------------------------------------ */
/* Symmetric int8 quantization per row  [P1 answer step 1, knowledge 2 & 5; */
/* P4 quantize_symmetric]                                                    */
/*   amax = max |x|;  if amax == 0: s = 0, q = 0                             */
/*   else m = fl32(127 / amax); s = fl32(amax / 127);                        */
/*        q = clamp(rne(fl32(x * m)), -127, 127)                             */
/* X fp16 [rows][cols]; Q int8 [rows][cols]; S fp32 [rows] (dequant scale).  */
/* ------------------------------------------------------------------------ */

static float qo_f16_to_f32(uint16_t h) { return (float)qo_f16_to_f64(h); }

QO_API void qo_quant_sym_int8(const uint16_t* X, int8_t* Q, float* S, int64_t rows, int32_t cols) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* x = X + r * cols;
        float amax = 0.0f;
        for (int32_t c = 0; c < cols; ++c) {
            const float a = fabsf(qo_f16_to_f32(x[c]));
            if (a > amax) amax = a;
        }
        int8_t* q = Q + r * cols;
        if (amax == 0.0f) {
            S[r] = 0.0f;
            for (int32_t c = 0; c < cols; ++c) q[c] = 0;
            continue;
        }
        const float mult = 127.0f / amax;
        S[r] = amax / 127.0f;
        for (int32_t c = 0; c < cols; ++c) {
            const float t = qo_f16_to_f32(x[c]) * mult;
            float v = nearbyintf(t);
            if (v > 127.0f) v = 127.0f;
            if (v < -127.0f) v = -127.0f;
            q[c] = (int8_t)v;
        }
    }
}

/* Dequantization  [P4 dequantize_symmetric]:  x = fp16(fl32(float(q) * s)) */
QO_API void qo_dequant_sym_int8(const int8_t* Q, const float* S, uint16_t* X, int64_t rows,
                                int32_t cols) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t c = 0; c < cols; ++c) {
            const float p = (float)Q[r * cols + c] * S[r];
            X[r * cols + c] = qo_f64_to_f16((double)p);
        }
}

/* ------------------------------------------------------------------------ */
/* W8A8 int8 GEMM  [P1 knowledge point 1: INT8 operands, integer accumulate]*/
/*   acc[m][n] = sum_k qa[m][k] * qw[n][k]   (exact integer)                 */
/* qa int8 [M][K]; qw int8 [N][K] (one row per output channel).              */
/* ------------------------------------------------------------------------ */

static int32_t qo_dot_i8(const int8_t* a, const int8_t* w, int32_t K) {
    int64_t s = 0;
    for (int32_t k = 0; k < K; ++k) s += (int64_t)a[k] * (int64_t)w[k];
    return (int32_t)s; /* |s| <= K * 127^2 fits int32 for K <= 133143 */
}

QO_API void qo_w8a8_acc(const int8_t* A, const int8_t* W, int32_t* acc, int32_t M, int32_t N,
                        int32_t K) {
#pragma omp parallel for schedule(static)
    for (int32_t m = 0; m < M; ++m)
        for (int32_t n = 0; n < N; ++n)
            acc[(int64_t)m * N + n] = qo_dot_i8(A + (int64_t)m * K, W + (int64_t)n * K, K);
}

/* GELU, erf form g(y) = y/2 * (1 + erf(y/sqrt(2))), with erf evaluated by
   Abramowitz & Stegun formula 7.1.28 (|error| <= 3e-7 for x >= 0):
     erf(x) ~= 1 - (1 + a1 x + a2 x^2 + ... + a6 x^6)^-16,
   extended to x < 0 by oddness.  Fixed fp32 sequence (Horner by fma, four
   squarings, one correctly rounded division), so that every IEEE-conforming
   evaluator produces the same bits. */
QO_API float qo_gelu28(float y) {
    const float a1 = 0.0705230784f, a2 = 0.0422820123f, a3 = 0.0092705272f;
    const float a4 = 0.0001520143f, a5 = 0.0002765672f, a6 = 0.0000430638f;
    const float u = y * 0.70710678f;
    const float a = fabsf(u);
    float p = fmaf(a, a6, a5);
    p = fmaf(a, p, a4);
    p = fmaf(a, p, a3);
    p = fmaf(a, p, a2);
    p = fmaf(a, p, a1);
    p = fmaf(a, p, 1.0f);
    p = p * p; /* p^2 */
    p = p * p; /* p^4 */
    p = p * p; /* p^8 */
    p = p * p; /* p^16 */
    float e = 1.0f - 1.0f / p;
    e = copysignf(e, u);
    return (0.5f * y) * (1.0f + e);
}

#define QO_EPI_BIAS 1u
#define QO_EPI_GELU 2u

/* Epilogue  [P1 knowledge point 2: rescale + bias + GELU, then requantize]
     t = fl32(acc); t = t * sa; t = t * sw; t = t + bias (if BIAS);
     g = gelu28(t) (if GELU) else t;  q = clamp(rne(g * out_mult), -127, 127) */
QO_API int8_t qo_w8a8_requant(int32_t acc, float sa, float sw, uint16_t bias, float out_mult,
                              uint32_t flags) {
    float t = (float)acc;
    t = t * sa;
    t = t * sw;
    if (flags & QO_EPI_BIAS) t = t + qo_f16_to_f32(bias);
    const float g = (flags & QO_EPI_GELU) ? qo_gelu28(t) : t;
    float v = nearbyintf(g * out_mult);
    if (v > 127.0f) v = 127.0f;
    if (v < -127.0f) v = -127.0f;
    return (int8_t)v;
}

QO_API void qo_w8a8_epilogue(const int8_t* A, const int8_t* W, const float* sa, const float* sw,
                             const uint16_t* bias, float out_mult, uint32_t flags, int8_t* Y,
                             int32_t* acc_out, int32_t M, int32_t N, int32_t K) {
#pragma omp parallel for schedule(static)
    for (int32_t m = 0; m < M; ++m)
        for (int32_t n = 0; n < N; ++n) {
            const int32_t acc = qo_dot_i8(A + (int64_t)m * K, W + (int64_t)n * K, K);
            if (acc_out) acc_out[(int64_t)m * N + n] = acc;
            Y[(int64_t)m * N + n] =
                qo_w8a8_requant(acc, sa[m], sw[n], bias ? bias[n] : 0, out_mult, flags);
        }
}

QO_API void qo_w8a8_epilogue_at(const int8_t* A, const int8_t* W, const float* sa,
                                const float* sw, const uint16_t* bias, float out_mult,
                                uint32_t flags, const int32_t* ms, const int32_t* ns,
                                int64_t count, int8_t* y, int32_t* acc_out, int32_t K) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const int32_t m = ms[i], n = ns[i];
        const int32_t acc = qo_dot_i8(A + (int64_t)m * K, W + (int64_t)n * K, K);
        if (acc_out) acc_out[i] = acc;
        y[i] = qo_w8a8_requant(acc, sa[m], sw[n], bias ? bias[n] : 0, out_mult, flags);
    }
}

/* ------------------------------------------------------------------------ */
/* INT4 MoE  [P5 constructor: numExperts, topK, hiddenSize, moeInterSize,   */
/* activationType, quantizationGroupSize]                                    */
/* ------------------------------------------------------------------------ */

/* Routing: per token, top-k experts by (logit descending, index ascending);
   gate weights = softmax over the selected logits (fp64). */
QO_API void qo_moe_route(const uint16_t* logits, int32_t T, int32_t E, int32_t topK, int32_t* ids,
                         double* w) {
    for (int32_t t = 0; t < T; ++t) {
        const uint16_t* l = logits + (int64_t)t * E;
        int32_t* id = ids + (int64_t)t * topK;
        for (int32_t j = 0; j < topK; ++j) {
            int32_t best = -1;
            double bv = 0.0;
            for (int32_t e = 0; e < E; ++e) {
                int taken = 0;
                for (int32_t i = 0; i < j; ++i) taken |= (id[i] == e);
                if (taken) continue;
                const double v = qo_f16_to_f64(l[e]);
                if (best < 0 || v > bv) { /* strict: lower index wins ties */
                    best = e;
                    bv = v;
                }
            }
            id[j] = best;
        }
        const double lmax = qo_f16_to_f64(l[id[0]]);
        double sum = 0.0;
        for (int32_t j = 0; j < topK; ++j) sum += exp(qo_f16_to_f64(l[id[j]]) - lmax);
        for (int32_t j = 0; j < topK; ++j)
            w[(int64_t)t * topK + j] = exp(qo_f16_to_f64(l[id[j]]) - lmax) / sum;
    }
}

/* Permutation: pairs p = t*topK + j grouped by expert, ascending p inside a
   group; offsets[e] = first slot of expert e, offsets[E] = T*topK. */
QO_API void qo_moe_permute(const int32_t* ids, int32_t T, int32_t topK, int32_t E,
                           int32_t* offsets, int32_t* pairs) {
    int32_t pos = 0;
    for (int32_t e = 0; e < E; ++e) {
        offsets[e] = pos;
        for (int32_t p = 0; p < T * topK; ++p)
            if (ids[p] == e) pairs[pos++] = p;
    }
    offsets[E] = pos;
}

/* Gate activation of the gated FFN (MoE plugin page, constructor:
   activationType), in fp64:
     0 SiLU       z / (1 + exp(-z))
     1 GELU, erf form   z/2 * (1 + erf(z / sqrt(2)))
     2 GELU, tanh form  z/2 * (1 + tanh(sqrt(2/pi) * (z + 0.044715 z^3)))
     3 ReLU       max(z, 0) */
QO_API double qo_moe_act(double z, int32_t activation) {
    switch (activation) {
        case 1: return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));
        case 2: return 0.5 * z * (1.0 + tanh(sqrt(2.0 / M_PI) * (z + 0.044715 * z * z * z)));
        case 3: return z > 0.0 ? z : 0.0;
        default: return z / (1.0 + exp(-z));
    }
}

/* One token through one expert: gated FFN with W4A16 weights.
     g = x . Wg, u = x . Wu   (fp64 sums over H, ascending)
     h = fp16( act(g) * u )   (act: qo_moe_act)
     o = h . Wd               (fp64 sum over I, ascending)
   Wg, Wu natural int4 [H][I/2], scales [H/G][I]; Wd natural [I][H/2],
   scales [I/G][H]. */
static void qo_expert_ffn(const uint16_t* x, const uint8_t* Wg, const uint8_t* Wu,
                          const uint8_t* Wd, const uint16_t* Sg, const uint16_t* Su,
                          const uint16_t* Sd, double* o, double* hbuf, int32_t H, int32_t I,
                          int32_t G, int32_t activation) {
#pragma omp parallel for schedule(static)
    for (int32_t i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int32_t h = 0; h < H; ++h) {
            const double xv = qo_f16_to_f64(x[h]);
            g += xv * ((double)qo_int4_at(Wg, I, h, i) * qo_f16_to_f64(Sg[(int64_t)(h / G) * I + i]));
            u += xv * ((double)qo_int4_at(Wu, I, h, i) * qo_f16_to_f64(Su[(int64_t)(h / G) * I + i]));
        }
        hbuf[i] = qo_f16_to_f64(qo_f64_to_f16(qo_moe_act(g, activation) * u));
    }
#pragma omp parallel for schedule(static)
    for (int32_t n = 0; n < H; ++n) {
        double s = 0.0;
        for (int32_t i = 0; i < I; ++i)
            s += hbuf[i] * ((double)qo_int4_at(Wd, H, i, n) * qo_f16_to_f64(Sd[(int64_t)(i / G) * H + n]));
        o[n] = s;
    }
}

/* Full layer for the listed tokens (tokens == NULL: all T tokens).
   y[t] = fp16( sum_{j < topK} w[t][j] * o[t][j] ), j ascending.
   Weights for expert e start at e * (H*I/2) bytes (gate/up/down) and scales
   at e * (H/G)*I (gate/up) or e * (I/G)*H (down) elements.  activation
   selects the gate nonlinearity (qo_moe_act).  Y is [T][H]; only the rows
   of the listed tokens are written.  ids/w receive the routing of all T. */
QO_API void qo_moe(const uint16_t* X, const uint16_t* logits, const uint8_t* Wg,
                   const uint8_t* Wu, const uint8_t* Wd, const uint16_t* Sg, const uint16_t* Su,
                   const uint16_t* Sd, uint16_t* Y, double* Y64, int32_t* ids, double* w,
                   int32_t T, int32_t H, int32_t I, int32_t E, int32_t topK, int32_t G,
                   int32_t activation, const int32_t* tokens, int32_t ntok) {
    (void)E;
    qo_moe_route(logits, T, E, topK, ids, w);
    const int64_t wbytes = (int64_t)H * I / 2;
    const int64_t sgn = (int64_t)(H / G) * I, sdn = (int64_t)(I / G) * H;
    double* o = (double*)malloc(sizeof(double) * (size_t)H);
    double* hb = (double*)malloc(sizeof(double) * (size_t)I);
    double* acc = (double*)malloc(sizeof(double) * (size_t)H);
    const int32_t count = tokens ? ntok : T;
    for (int32_t i = 0; i < count; ++i) {
        const int32_t t = tokens ? tokens[i] : i;
        for (int32_t n = 0; n < H; ++n) acc[n] = 0.0;
        for (int32_t j = 0; j < topK; ++j) {
            const int32_t e = ids[(int64_t)t * topK + j];
            qo_expert_ffn(X + (int64_t)t * H, Wg + e * wbytes, Wu + e * wbytes, Wd + e * wbytes,
                          Sg + e * sgn, Su + e * sgn, Sd + e * sdn, o, hb, H, I, G, activation);
            const double wj = w[(int64_t)t * topK + j];
            for (int32_t n = 0; n < H; ++n) acc[n] += wj * o[n];
        }
        for (int32_t n = 0; n < H; ++n) {
            if (Y) Y[(int64_t)t * H + n] = qo_f64_to_f16(acc[n]);
            if (Y64) Y64[(int64_t)t * H + n] = acc[n];
        }
    }
    free(o);
    free(hb);
    free(acc);
}

/* ------------------------------------------------------------------------ */
/* FP8 E4M3  [P2: FP8 E4M3 GEMM with per-tensor scaling factors derived     */
/* from the activation A-max, and the FP8 KV cache]                          */
/* Format: OCP "E4M3FN" -- sign, 4 exponent bits (bias 7), 3 mantissa bits; */
/* no infinities; exponent and mantissa all ones is NaN; largest finite     */
/* 448, smallest normal 2^-6, subnormals m * 2^-9.                          */
/* ------------------------------------------------------------------------ */

/* code -> exact binary64 value (NaN for the two NaN codes) */
QO_API double qo_e4m3_to_f64(uint8_t b) {
    const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7) return NAN;
    const double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* binary64 -> code: round to nearest, ties to the even mantissa; |x| >= 448
   saturates to +-448 (the quantizer clamps first, so this only matters for
   direct calls).  NaN input is outside the contract. */
QO_API uint8_t qo_f64_to_e4m3(double x) {
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    const double a = fabs(x);
    if (a >= 448.0) return sign | 0x7e;
    if (a < ldexp(1.0, -6)) {
        /* subnormal binade: multiples of 2^-9; 8 * 2^-9 is the smallest normal (code 0x08) */
        return sign | (uint8_t)nearbyint(a * 512.0);
    }
    int e;
    frexp(a, &e);                                  /* a in [2^(e-1), 2^e) */
    double q = nearbyint(ldexp(a, 4 - e));         /* 8 + mantissa, in [8, 16] */
    int E = e + 6;                                 /* exponent field of 2^(e-1) */
    if (q == 16.0) { q = 8.0; E += 1; }
    return sign | (uint8_t)(E << 3) | (uint8_t)(q - 8.0);
}

QO_API void qo_e4m3_to_f64_array(const uint8_t* b, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = qo_e4m3_to_f64(b[i]);
}
QO_API void qo_f64_to_e4m3_array(const double* x, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = qo_f64_to_e4m3(x[i]);
}

/* Symmetric FP8 quantization, per row (per_row != 0: one scale per row, as
   the per-token KV cache) or per tensor (one scale for all rows):
     amax = max |x|;  if amax == 0: s = 0, codes 0
     else m = fl32(448 / amax); s = fl32(amax / 448);
          q = e4m3(clamp(fl32(x * m), -448, 448))
   S receives rows scales (per row) or one scale (per tensor). */
QO_API void qo_quant_fp8(const uint16_t* X, uint8_t* Q, float* S, int64_t rows, int32_t cols,
                         int32_t per_row) {
    const int64_t groups = per_row ? rows : 1;
    const int64_t grows = per_row ? 1 : rows;
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < groups; ++g) {
        const uint16_t* x = X + g * grows * cols;
        uint8_t* q = Q + g * grows * cols;
        const int64_t n = grows * cols;
        float amax = 0.0f;
        for (int64_t i = 0; i < n; ++i) {
            const float a = fabsf(qo_f16_to_f32(x[i]));
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) {
            S[g] = 0.0f;
            for (int64_t i = 0; i < n; ++i) q[i] = 0;
            continue;
        }
        const float mult = 448.0f / amax;
        S[g] = amax / 448.0f;
        for (int64_t i = 0; i < n; ++i) {
            float t = qo_f16_to_f32(x[i]) * mult;
            if (t > 448.0f) t = 448.0f;
            if (t < -448.0f) t = -448.0f;
            q[i] = qo_f64_to_e4m3((double)t);
        }
    }
}

/* Dequantization: x = fp16(fl32(e4m3 value * s)), s per row or one per tensor. */
QO_API void qo_dequant_fp8(const uint8_t* Q, const float* S, uint16_t* X, int64_t rows,
                           int32_t cols, int32_t per_row) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float s = S[per_row ? r : 0];
        for (int32_t c = 0; c < cols; ++c) {
            const float p = (float)qo_e4m3_to_f64(Q[r * cols + c]) * s;
            X[r * cols + c] = qo_f64_to_f16((double)p);
        }
    }
}

/* FP8 GEMM: A e4m3 [M][K], W e4m3 [N][K] (one row per output column);
     acc = sum_k A[m][k] * W[n][k]  (every product and partial sum exact in fp64)
     Y[m][n] = fp16(acc * sa[m or 0] * sw[n or 0])  (fp64 products, one rounding) */
static double qo_fp8_dot(const uint8_t* a, const uint8_t* w, int32_t K) {
    double acc = 0.0;
    for (int32_t k = 0; k < K; ++k) acc += qo_e4m3_to_f64(a[k]) * qo_e4m3_to_f64(w[k]);
    return acc;
}

QO_API void qo_fp8_gemm(const uint8_t* A, const uint8_t* W, const float* sa, int32_t sa_per_row,
                        const float* sw, int32_t sw_per_row, uint16_t* Y, double* Y64, int32_t M,
                        int32_t N, int32_t K) {
#pragma omp parallel for schedule(static)
    for (int32_t m = 0; m < M; ++m)
        for (int32_t n = 0; n < N; ++n) {
            const double acc = qo_fp8_dot(A + (int64_t)m * K, W + (int64_t)n * K, K);
            const double y = acc * (double)sa[sa_per_row ? m : 0] * (double)sw[sw_per_row ? n : 0];
            Y[(int64_t)m * N + n] = qo_f64_to_f16(y);
            if (Y64) Y64[(int64_t)m * N + n] = y;
        }
}

/* Same definition at the listed (m, n) positions. */
QO_API void qo_fp8_gemm_at(const uint8_t* A, const uint8_t* W, const float* sa, int32_t sa_per_row,
                           const float* sw, int32_t sw_per_row, int64_t count, const int32_t* ms,
                           const int32_t* ns, uint16_t* Y, int32_t K) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        const int32_t m = ms[i], n = ns[i];
        const double acc = qo_fp8_dot(A + (int64_t)m * K, W + (int64_t)n * K, K);
        Y[i] = qo_f64_to_f16(acc * (double)sa[sa_per_row ? m : 0] * (double)sw[sw_per_row ? n : 0]);
    }
}

/* ------------------------------------------------------------------------ */
/* INT8 multi-head attention chain  [P1 answer step 3 (enqueue core): int8   */
/* QK^T GEMM to int32 logits; online softmax from fp32 to int8              */
/* probabilities, the logits scaled by scale_q * scale_k; int8 P.V GEMM;    */
/* rescale, bias and requantization to int8.  P1 answer step 2: output      */
/* dimensions [batch, seq, heads, head_dim]; knowledge point 5: +-127]      */
/*                                                                          */
/* Q [B][Lq][H][D], K and V [B][Lk][H][D] int8; O [B][Lq][H][D] int8.        */
/* For head (b, h), query i, key j, channel c:                              */
/*   S_ij = sum_c Q[b,i,h,c] * K[b,j,h,c]                 exact integer      */
/*   x_ij = fl32(fl32(S_ij) * alpha)                      one fp32 multiply  */
/*   p_ij = exp(x_ij - max_j x) / sum_j exp(x_ij - max_j x)   in fp64        */
/*   P_ij = rne(127 * p_ij), in [0, 127] (probabilities carry scale 1/127)   */
/*   A_ic = sum_j P_ij * V[b,j,h,c]                       exact integer      */
/*   t = fl32(A_ic); t = t * pv_scale; t = t + bias[h*D + c] if flagged;     */
/*   O = clamp(rne(t * out_mult), -127, 127)              fp32 steps         */
/* Heads are listed as b*H + h; per-head arrays are [nheads][Lq][Lk].        */
/* ------------------------------------------------------------------------ */

static int64_t qo_mha_at(int32_t b, int32_t t, int32_t h, int32_t L, int32_t H, int32_t D) {
    return (((int64_t)b * L + t) * H + h) * D;
}

/* S (optional), P and R = 127 * p (optional) of the listed heads. */
QO_API void qo_mha_int8_probs(const int8_t* Q, const int8_t* K, const int32_t* heads, int64_t nheads,
                              int32_t H, int32_t Lq, int32_t Lk, int32_t D, float alpha, int32_t* S,
                              int8_t* P, double* R) {
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t hh = 0; hh < nheads; ++hh)
        for (int32_t i = 0; i < Lq; ++i) {
            const int32_t b = heads[hh] / H, h = heads[hh] % H;
            const int64_t row = (hh * Lq + i) * (int64_t)Lk;
            double* x = (double*)malloc(sizeof(double) * (size_t)Lk);
            double m = -INFINITY;
            for (int32_t j = 0; j < Lk; ++j) {
                const int8_t* q = Q + qo_mha_at(b, i, h, Lq, H, D);
                const int8_t* k = K + qo_mha_at(b, j, h, Lk, H, D);
                int64_t s = 0;
                for (int32_t c = 0; c < D; ++c) s += (int64_t)q[c] * (int64_t)k[c];
                if (S) S[row + j] = (int32_t)s;
                const float xs = (float)s;
                const float xf = xs * alpha;
                x[j] = (double)xf;
                if (x[j] > m) m = x[j];
            }
            double sum = 0.0;
            for (int32_t j = 0; j < Lk; ++j) sum += exp(x[j] - m);
            for (int32_t j = 0; j < Lk; ++j) {
                const double r = 127.0 * (exp(x[j] - m) / sum);
                P[row + j] = (int8_t)nearbyint(r);
                if (R) R[row + j] = r;
            }
            free(x);
        }
}

/* O of the listed heads from their probabilities P ([nheads][Lq][Lk]); the
   other heads' outputs are left untouched. */
QO_API void qo_mha_int8_out(const int8_t* P, const int8_t* V, const uint16_t* bias, const int32_t* heads,
                            int64_t nheads, int32_t H, int32_t Lq, int32_t Lk, int32_t D, float pv_scale,
                            float out_mult, uint32_t flags, int8_t* O) {
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t hh = 0; hh < nheads; ++hh)
        for (int32_t i = 0; i < Lq; ++i) {
            const int32_t b = heads[hh] / H, h = heads[hh] % H;
            const int8_t* p = P + (hh * Lq + i) * (int64_t)Lk;
            for (int32_t c = 0; c < D; ++c) {
                int64_t acc = 0;
                for (int32_t j = 0; j < Lk; ++j) acc += (int64_t)p[j] * (int64_t)V[qo_mha_at(b, j, h, Lk, H, D) + c];
                float t = (float)acc;
                t = t * pv_scale;
                if (flags & QO_EPI_BIAS) t = t + qo_f16_to_f32(bias[h * D + c]);
                float v = nearbyintf(t * out_mult);
                if (v > 127.0f) v = 127.0f;
                if (v < -127.0f) v = -127.0f;
                O[qo_mha_at(b, i, h, Lq, H, D) + c] = (int8_t)v;
            }
        }
}
