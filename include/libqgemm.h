/*
 * libqgemm -- quantized GEMM kernels for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * C ABI.  Every entry point is asynchronous on the caller's HIP stream and
 * returns an int32 status (0 = success), in the manner of the plugin
 * `enqueue` calls of the TensorRT-Edge-LLM "Int4 Groupwise GEMM Plugin V2"
 * and "Int4 Moe Plugin" pages (Public Functions: enqueue returns 0 on success,
 * non-zero on error).  No C++ exception crosses this boundary and the library
 * never prints or exits.
 *
 * Conventions for every function below:
 *   - All data pointers are DEVICE pointers owned by the caller; the library
 *     allocates no device memory, caches nothing and keeps no state between
 *     calls, so calls are re-entrant and thread-safe.
 *   - fp16 data is passed as uint16_t bit patterns (IEEE binary16).
 *   - All matrices are row-major and densely packed.
 *   - `stream` is a hipStream_t (NULL = the null stream).
 *   - Shapes, pointers, alignment and workspace are validated before any
 *     launch; on a validation error nothing is launched and no output is
 *     touched.  A launch failure returns QGEMM_HIP_ERROR.  Faults that happen
 *     while a kernel runs surface at the caller's next synchronization.
 *   - Every pointer must be 16-byte aligned (128-bit vector loads), except
 *     the per-row/per-column vectors (scales, bias, routing outputs), which
 *     need 4-byte alignment.
 *   - Results are deterministic: fixed reduction orders, no floating-point
 *     atomics (the one atomic, in per-tensor FP8 quantization, is an integer
 *     maximum); two calls with the same inputs give identical bits.
 */
#ifndef LIBQGEMM_H
#define LIBQGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define QGEMM_API __attribute__((visibility("default")))
#else
#define QGEMM_API
#endif

#define QGEMM_ABI_VERSION 1

/* Status codes. */
#define QGEMM_OK 0
#define QGEMM_NULL_PTR 1            /* a required pointer is NULL */
#define QGEMM_BAD_SHAPE 2           /* negative size, topK > E, G not dividing K, ... */
#define QGEMM_MISALIGNED 3          /* a pointer violates the alignment rule above */
#define QGEMM_WORKSPACE_TOO_SMALL 4 /* workspace_bytes below the *_workspace_bytes() query */
#define QGEMM_UNSUPPORTED 5         /* valid request outside what this version implements */
#define QGEMM_HIP_ERROR 6           /* a HIP launch or API call failed */

/* Returns QGEMM_ABI_VERSION. */
QGEMM_API int32_t qgemm_abi_version(void);

/* Static string naming a status code ("unknown status" for other values). */
QGEMM_API const char* qgemm_status_str(int32_t status);

/* ------------------------------------------------------------------------
 * W4A16 group-wise GEMM  (Int4 Groupwise GEMM Plugin V2 page, class summary
 * and constructor: fp16 activations [b,seq,K] x int4 weights with fp16
 * scales [ceil(K/G), N] -> fp16 [b,seq,N]; K = weight rows, N = weight
 * columns, G = quantization group size; weights are repacked offline into a
 * fragment layout, with no repack or cached weight buffer at run time).
 *
 *   Y[m][n] = fp16( sum_k A[m][k] * q(k,n) * S[k/G][n] )
 *
 * Natural weight format: uint8 [K][N/2]; column n of row k is the low nibble
 * (bits 0-3) of byte [k][n/2] for even n and the high nibble for odd n; each
 * nibble is a two's-complement int4 in [-8, 7].
 *
 * Supported in this version: K % 8 == 0 and N % 8 == 0 (rows of A and Y stay
 * 16-byte aligned), G in {32, 64, 128}; other shapes return
 * QGEMM_UNSUPPORTED.  K need not be a multiple of 128 or of G (the page's
 * ceil(K/G) scale rows: the last group covers the remaining K % G rows) and
 * N need not be a multiple of 128: the fragment layout is padded to whole
 * 128 x 128 tiles with weight 0 (the page's fragment rows
 * ceil(N/128) * ceil(K/64) * 8), and such shapes run the decode or the
 * 128x128 prefill kernel (tactics 1, 2 and 4).
 * ---------------------------------------------------------------------- */

/* Bytes of the fragment-layout weight buffer for a K x N int4 matrix,
   padded to whole 128 x 128 tiles: ceil(K/128)*128 * ceil(N/128)*128 / 2
   (= K*N/2 when both are multiples of 128); 0 if the shape is unsupported. */
QGEMM_API size_t qgemm_w4a16_packed_bytes(int32_t K, int32_t N);

/* Repack natural int4 weights into the library's gfx950 fragment layout.
   w_natural: uint8 [K][N/2] (input, not modified).
   w_frag:    uint8 [qgemm_w4a16_packed_bytes(K, N)] (output); must not
              overlap w_natural.
   Run once per weight matrix, offline; the layout is the library's own and
   is only consumed by qgemm_w4a16 and moe_w4a16. */
QGEMM_API int32_t qgemm_w4a16_prepack(const uint8_t* w_natural, uint8_t* w_frag, int32_t K, int32_t N,
                            void* stream);

/* Workspace bytes qgemm_w4a16 uses for this shape: for 16 < M <= 128 (and
   M*K < 2^31, K and N multiples of 128) the fp32 partial sums of its split-K
   path, S * M * N * 4 bytes with S = max(1, min(floor(512 / (N/128)), K/128, 16));
   0 for every other shape and for invalid arguments. */
QGEMM_API size_t qgemm_w4a16_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t G);

/* Y = A x dequant(w_frag, scales).
   A:      fp16 [M][K] activations (M = batch * sequence length).
   w_frag: prepacked weights from qgemm_w4a16_prepack(K, N).
   scales: fp16 [ceil(K/G)][N].
   Y:      fp16 [M][N] output; must not overlap the inputs.
   workspace: device memory of workspace_bytes bytes (16-byte aligned), or
   NULL / 0.  M == 0 is a successful no-op.  M <= 16 runs the memory-bound
   decode kernel; 16 < M <= 128 with at least qgemm_w4a16_workspace_bytes()
   of workspace runs the split-K kernel (fp32 partials in the workspace, then
   a reduction adding the K splits in a fixed order); other M, or a smaller
   workspace, run the MFMA prefill kernels.  All compute the same function
   (fp32 accumulation, one rounding to fp16 at the end) and are
   deterministic.  Calls sharing one workspace must not overlap. */
QGEMM_API int32_t qgemm_w4a16(const uint16_t* A, const uint8_t* w_frag, const uint16_t* scales, uint16_t* Y,
                    int32_t M, int32_t N, int32_t K, int32_t G, void* workspace,
                    size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * W4A16 tactics  (Int4 Groupwise GEMM Plugin V2 page: getNbTactics /
 * getValidTactics list the valid kernel variants for a shape as positive ids,
 * setTactic selects one, 0 being the default; configurePlugin's token count
 * steers the choice; the timing cache lets each shape be autotuned once).
 *
 * Ids of this library's W4A16 kernels (all compute qgemm_w4a16's function
 * with fp32 accumulation; results of different tactics agree within the
 * fp16 tolerance, not bit for bit; each tactic alone is deterministic):
 *   1 decode, one 16-column strip per workgroup      valid for M <= 2
 *   2 decode, balanced ranges of up to 3 strips      valid for M <= 16
 *   3 split-K with fp32 partials + ordered reduction valid for M <= 512,
 *     M*K < 2^31, K % 128 == 0 and N % 128 == 0; needs
 *     qgemm_w4a16_tactic_workspace_bytes() of workspace
 *   4 prefill, 128x128 tiles                         valid for every M
 *   5 prefill, 128x256 tiles (LDS DMA)               valid for N % 256 == 0
 *                                                    and K % 128 == 0
 * The library keeps no tactic state: a caller that autotunes keeps the
 * result per shape.
 * ---------------------------------------------------------------------- */
#define QGEMM_TACTIC_DEFAULT 0
#define QGEMM_W4A16_TACTIC_DECODE_NARROW 1
#define QGEMM_W4A16_TACTIC_DECODE_BALANCED 2
#define QGEMM_W4A16_TACTIC_SPLITK 3
#define QGEMM_W4A16_TACTIC_PREFILL 4
#define QGEMM_W4A16_TACTIC_PREFILL_LARGE 5

/* Number of tactics valid for the shape (0 if qgemm_w4a16 does not support
   the shape or M <= 0); the first min(count, capacity) ids, ascending, are
   written to tactics (may be NULL). */
QGEMM_API int32_t qgemm_w4a16_tactics(int32_t M, int32_t N, int32_t K, int32_t G, int32_t* tactics,
                                      int32_t capacity);

/* Workspace bytes a tactic needs (tactic 0: qgemm_w4a16_workspace_bytes;
   0 for tactics that need none and for invalid arguments). */
QGEMM_API size_t qgemm_w4a16_tactic_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t G, int32_t tactic);

/* qgemm_w4a16 with the kernel chosen by the caller: tactic 0 is exactly
   qgemm_w4a16; a tactic not valid for the shape returns QGEMM_UNSUPPORTED;
   tactic 3 without enough workspace returns QGEMM_WORKSPACE_TOO_SMALL.
   Arguments and errors otherwise as qgemm_w4a16. */
QGEMM_API int32_t qgemm_w4a16_tactic(const uint16_t* A, const uint8_t* w_frag, const uint16_t* scales, uint16_t* Y,
                                     int32_t M, int32_t N, int32_t K, int32_t G, int32_t tactic, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Times every valid tactic (tactic 3 only if the workspace suffices) on the
   given operands: two untimed launches, then `reps` launches between two HIP
   events on `stream`; writes the fastest id to *best_tactic and its mean
   microseconds per launch to *best_us (may be NULL).  Blocks the host until
   the timed launches finish; Y is overwritten; creates and destroys two HIP
   events, allocates no device memory.  M == 0 or reps <= 0 return
   QGEMM_BAD_SHAPE; other argument errors as qgemm_w4a16. */
QGEMM_API int32_t qgemm_w4a16_autotune(const uint16_t* A, const uint8_t* w_frag, const uint16_t* scales,
                                       uint16_t* Y, int32_t M, int32_t N, int32_t K, int32_t G, void* workspace,
                                       size_t workspace_bytes, int32_t reps, int32_t* best_tactic, float* best_us,
                                       void* stream);

/* ------------------------------------------------------------------------
 * W8A16 weight-only int8 GEMM  (FP8 vs INT8 low-precision inference in
 * TensorRT-LLM, itzkxy.com: weight-only int8 with fp16 activations is one of
 * the INT8 configurations compared; the page leaves the scale granularity
 * open, and this version takes group-wise or per-column fp16 scales).
 *
 *   Y[m][n] = fp16( sum_k A[m][k] * W[k][n] * S[k/G][n] )
 *
 * Natural weight format: int8 [K][N] (two's complement, full range
 * [-128, 127]).  G = K means one scale per column (S is fp16 [1][N]).
 *
 * Supported in this version: K % 8 == 0, N % 8 == 0, G in {32, 64, 128} or
 * G == K; other shapes return QGEMM_UNSUPPORTED.  As for W4A16, K and N need
 * not be multiples of 128 nor K of G (scales [ceil(K/G)][N], the layout
 * padded to whole 128 x 128 tiles with weight 0; such shapes run the decode
 * or the 128x128 prefill kernel).
 * ---------------------------------------------------------------------- */

/* Bytes of the int8 fragment-layout buffer for a K x N matrix, padded to
   whole 128 x 128 tiles: ceil(K/128)*128 * ceil(N/128)*128 (= K*N when both
   are multiples of 128); 0 if the shape is unsupported. */
QGEMM_API size_t qgemm_w8a16_packed_bytes(int32_t K, int32_t N);

/* Repack natural int8 weights into the library's int8 fragment layout.
   w_natural: int8 [K][N] (input, not modified).
   w_frag:    uint8 [qgemm_w8a16_packed_bytes(K, N)] (output); must not
              overlap w_natural.
   Run once per weight matrix; the layout is only consumed by qgemm_w8a16. */
QGEMM_API int32_t qgemm_w8a16_prepack(const int8_t* w_natural, uint8_t* w_frag, int32_t K, int32_t N,
                                      void* stream);

/* Workspace bytes qgemm_w8a16 uses for this shape: the same rule as
   qgemm_w4a16_workspace_bytes (split-K partials for 16 < M <= 128, else 0;
   0 for invalid arguments). */
QGEMM_API size_t qgemm_w8a16_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t G);

/* Y = A x (W * S).
   A:      fp16 [M][K] activations.
   w_frag: prepacked weights from qgemm_w8a16_prepack(K, N).
   scales: fp16 [ceil(K/G)][N] ([1][N] for G == K).
   Y:      fp16 [M][N] output; must not overlap the inputs.
   workspace: as for qgemm_w4a16.  M <= 16 runs the memory-bound decode
   kernel, 16 < M <= 128 with enough workspace the split-K kernel, every
   other M the MFMA prefill kernel; all compute the same function (fp32
   accumulation, one rounding to fp16) and are deterministic.  Calls sharing
   one workspace must not overlap. */
QGEMM_API int32_t qgemm_w8a16(const uint16_t* A, const uint8_t* w_frag, const uint16_t* scales, uint16_t* Y,
                              int32_t M, int32_t N, int32_t K, int32_t G, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Symmetric int8 quantization, one scale per row  (INT8 cross-modal MHA
 * TensorRT plugin interview page, answer step 1: scale = 127 / max|x| per
 * output channel of the weights and per token of the activations, and
 * knowledge point 5: codes limited to [-127, 127]; KV Cache INT8量化 page,
 * quantize_symmetric / dequantize_symmetric).
 *
 * Per row r of `cols` contiguous values:
 *   amax = max |x|;  amax == 0 -> scale 0 and all codes 0; otherwise
 *   mult = fl32(127 / amax);  scale = fl32(amax / 127);
 *   q = clamp(round_half_even(fl32(x * mult)), -127, 127)
 * (each fl32 is one IEEE single-precision operation).
 * Used for per-token activations, per-output-channel weights (rows of W
 * [N][K]) and KV-cache rows (one row per (head, token)).
 * ---------------------------------------------------------------------- */

/* X: fp16 [rows][cols] (input, finite values; a row holding an infinity or
   NaN gets unspecified codes); Q: int8 [rows][cols] (output);
   scales: fp32 [rows] (output, the dequantization scale amax/127).
   cols must be a multiple of 8 and at most 65536; rows == 0 is a no-op.
   Codes and scales are bit-exact functions of X. */
QGEMM_API int32_t quant_sym_int8(const uint16_t* X, int8_t* Q, float* scales, int32_t rows, int32_t cols,
                       void* stream);

/* X[r][c] = fp16( fl32( float(Q[r][c]) * scales[r] ) ), round to nearest even.
   Q: int8 [rows][cols]; scales: fp32 [rows]; X: fp16 [rows][cols] (output).
   cols must be a multiple of 8. */
QGEMM_API int32_t dequant_sym_int8(const int8_t* Q, const float* scales, uint16_t* X, int32_t rows,
                         int32_t cols, void* stream);

/* ------------------------------------------------------------------------
 * W8A8 int8 GEMM with fused epilogue  (INT8 cross-modal MHA TensorRT plugin
 * interview page, knowledge points 1-2: int8 operands with integer
 * accumulation, then rescale + bias + GELU and requantization to int8;
 * answer step 3: per-tensor output scale and fp16 bias).
 *
 *   acc[m][n] = sum_k A[m][k] * W[n][k]                       (exact int32)
 *   t = fl32(acc); t = t * a_scale[m]; t = t * w_scale[n];
 *   if (flags & QGEMM_EPI_BIAS) t = t + float(bias[n]);
 *   g = (flags & QGEMM_EPI_GELU) ? gelu(t) : t;
 *   Y[m][n] = clamp(round_half_even(g * out_mult), -127, 127)
 *
 * gelu(t) = t/2 * (1 + erf(t / sqrt 2)) with erf from Abramowitz & Stegun
 * formula 7.1.28, evaluated in a fixed fp32 sequence:
 *   u = t * 0.70710678f; a = |u|;
 *   p = fma(a, fma(a, fma(a, fma(a, fma(a, fma(a, a6, a5), a4), a3), a2), a1), 1);
 *   p = p^16 by four squarings; e = copysign(1 - 1/p, u);  g = (0.5f * t) * (1 + e)
 *   a1..a6 = 0.0705230784, 0.0422820123, 0.0092705272, 0.0001520143,
 *            0.0002765672, 0.0000430638.
 * ---------------------------------------------------------------------- */
#define QGEMM_EPI_BIAS 1u
#define QGEMM_EPI_GELU 2u

/* A: int8 [M][K] activation codes; W: int8 [N][K] weight codes (one row per
   output channel); a_scale: fp32 [M]; w_scale: fp32 [N]; bias: fp16 [N]
   (may be NULL when QGEMM_EPI_BIAS is clear); Y: int8 [M][N] (output);
   acc_out: int32 [M][N] raw accumulators (optional, NULL to skip).
   Supported: any M >= 0, N % 128 == 0, K % 128 == 0 and K <= 133120 (so
   |acc| <= K * 127^2 < 2^31).  Other shapes return QGEMM_UNSUPPORTED.
   M == 0 is a successful no-op. */
QGEMM_API int32_t qgemm_w8a8_epilogue(const int8_t* A, const int8_t* W, const float* a_scale,
                            const float* w_scale, const uint16_t* bias, float out_mult,
                            uint32_t flags, int8_t* Y, int32_t* acc_out, int32_t M, int32_t N,
                            int32_t K, void* stream);

/* ------------------------------------------------------------------------
 * INT4 mixture-of-experts layer  (Int4 Moe Plugin page, constructor:
 * numExperts, topK, hiddenSize, moeInterSize, activationType,
 * quantizationGroupSize; one output tensor).
 *
 * Routing: per token, the topK experts with the largest logits (the lower
 * expert index wins ties), in descending order; gate weights = softmax over
 * the selected logits (fp32).
 * Expert FFN (gated, act chosen by activation):  g = x Wg_e, u = x Wu_e (W4A16,
 * fp32 accumulation), h = fp16(act(g) * u), o = h Wd_e (W4A16).
 * Combine: Y[t] = fp16( sum_{j < topK} w[t][j] * o[t][j] ), j ascending.
 * ---------------------------------------------------------------------- */

/* Gate activation of the expert FFN, h = fp16(act(g) * u) (the constructor's
   activationType; the page does not list its values, so these are the
   library's): */
#define QGEMM_MOE_ACT_SILU 0      /* g / (1 + exp(-g)) */
#define QGEMM_MOE_ACT_GELU_ERF 1  /* g/2 * (1 + erf(g / sqrt(2))) */
#define QGEMM_MOE_ACT_GELU_TANH 2 /* g/2 * (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))) */
#define QGEMM_MOE_ACT_RELU 3      /* max(g, 0) */

/* Workspace bytes moe_w4a16 needs (T tokens, hidden H, intermediate I,
   E experts, topK).  Layout, in this order, each part 256-byte aligned:
     int32 offsets[E+1]      first slot of each expert in the sorted order
     int32 pairs[T*topK]     pair ids p = t*topK + j sorted by expert, then p
     int32 slot_of[T*topK]   inverse of pairs
     fp16  h[T*topK][I]      intermediate activations, sorted order
     fp32  o[S][T*topK][H]   partial expert outputs, sorted order, one slice
                             per split of the down projection's K; S starts
                             at 1 and doubles while S < 8, E*(H/128)*S < 512
                             and (I/128) % (2*S) == 0
   The first two parts are part of the documented result (tests read them). */
QGEMM_API size_t moe_w4a16_workspace_bytes(int32_t T, int32_t H, int32_t I, int32_t E, int32_t topK);

/* X: fp16 [T][H] hidden states; logits: fp16 [T][E] router logits.
   w_gate_frag, w_up_frag: E consecutive prepacked matrices of
     qgemm_w4a16_packed_bytes(H, I) bytes each (K = H rows, N = I columns).
   w_down_frag: E consecutive prepacked matrices of
     qgemm_w4a16_packed_bytes(I, H) bytes (K = I, N = H).
   s_gate, s_up: fp16 [E][H/G][I]; s_down: fp16 [E][I/G][H].
   Y: fp16 [T][H] (output); topk_ids: int32 [T][topK] (output);
   topk_w: fp32 [T][topK] (output).
   activation: one of QGEMM_MOE_ACT_*.
   Supported: H % 128 == 0, I % 128 == 0, G in {32, 64, 128}, 1 <= topK <= E
   <= 64, T*H < 2^31 and T*topK*I < 2^31.  T == 0 is a successful no-op. */
QGEMM_API int32_t moe_w4a16(const uint16_t* X, const uint16_t* logits, const uint8_t* w_gate_frag,
                  const uint8_t* w_up_frag, const uint8_t* w_down_frag, const uint16_t* s_gate,
                  const uint16_t* s_up, const uint16_t* s_down, uint16_t* Y, int32_t* topk_ids,
                  float* topk_w, int32_t T, int32_t H, int32_t I, int32_t E, int32_t topK,
                  int32_t G, int32_t activation, void* workspace, size_t workspace_bytes,
                  void* stream);

/* moe_w4a16 without a workspace argument, for callers that cannot allocate
   device memory (code under HIP graph capture, tight serving loops, harnesses
   that forbid hipMalloc).  Same arguments, limits, kernels and results as
   moe_w4a16; the workspace is a library-owned array of
   QGEMM_MOE_NO_ALLOC_SCRATCH_BYTES bytes per GPU, created with the library's
   code object on the first use on that GPU and held until the process ends.
   The call itself allocates nothing.
   Returns QGEMM_WORKSPACE_TOO_SMALL when moe_w4a16_workspace_bytes(T, H, I, E,
   topK) exceeds that size (the layer of 256 tokens, hidden 4096, intermediate
   14336, 8 experts, top-2 needs about 31.5 MB), QGEMM_UNSUPPORTED when a
   non-NULL stream belongs to another device than the current one.
   Every call on one GPU shares that GPU's array and leaves its contents
   behind (no part has to start at zero): calls that may overlap on one GPU
   (different streams, or host threads) race and must be serialized by the
   caller. */
#define QGEMM_MOE_NO_ALLOC_SCRATCH_BYTES ((size_t)64 << 20)
QGEMM_API int32_t moe_w4a16_no_alloc(const uint16_t* X, const uint16_t* logits,
                  const uint8_t* w_gate_frag, const uint8_t* w_up_frag,
                  const uint8_t* w_down_frag, const uint16_t* s_gate, const uint16_t* s_up,
                  const uint16_t* s_down, uint16_t* Y, int32_t* topk_ids, float* topk_w,
                  int32_t T, int32_t H, int32_t I, int32_t E, int32_t topK, int32_t G,
                  int32_t activation, void* stream);

/* ------------------------------------------------------------------------
 * FP8 E4M3  (FP8-vs-INT8 article for TensorRT-LLM: the E4M3 format for the
 * GEMMs and the KV cache, scaling factors from the activation A-max,
 * per-tensor scaling sufficing for FP8).
 *
 * Format: OCP E4M3 ("E4M3FN"): sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; no infinities; S.1111.111 is NaN; largest finite 448.  Codes are
 * passed as uint8_t.  NaN or infinite inputs are outside the contract.
 * ---------------------------------------------------------------------- */
#define QGEMM_FP8_PER_TENSOR 0 /* one scale for the whole [rows][cols] tensor */
#define QGEMM_FP8_PER_ROW 1    /* one scale per row (per token / per channel) */

/* Symmetric FP8 quantization of fp16 X [rows][cols] into codes Q [rows][cols]:
     amax = max |x| over a row (per row) or over the tensor (per tensor);
     if amax == 0: scale 0 and every code 0x00;
     else m = fl32(448 / amax); s = fl32(amax / 448);
          Q = e4m3_rne(clamp(fl32(x * m), -448, 448))   (ties to even)
   scales: fp32, [rows] per row or [1] per tensor (output: s).
   per_row: QGEMM_FP8_PER_ROW or QGEMM_FP8_PER_TENSOR.
   cols must be a multiple of 8 (per row also at most 4096); rows == 0 is a
   no-op.  Codes and scales are bit-exact functions of X.  Per tensor, three
   stream-ordered launches: per-block maxima of |x| are written into the
   first bytes of Q, the codes of the rest of Q follow, then the codes of
   those first bytes and scales[0]; Q and scales must not be read before the
   call has completed on the stream. */
QGEMM_API int32_t quant_fp8_e4m3(const uint16_t* X, uint8_t* Q, float* scales, int32_t rows,
                                 int32_t cols, int32_t per_row, void* stream);

/* X[r][c] = fp16( fl32( e4m3_value(Q[r][c]) * s ) ), round to nearest even,
   s = scales[r] (per row) or scales[0] (per tensor).  cols % 8 == 0. */
QGEMM_API int32_t dequant_fp8_e4m3(const uint8_t* Q, const float* scales, uint16_t* X, int32_t rows,
                                   int32_t cols, int32_t per_row, void* stream);

/* FP8 GEMM with fp16 output:
     acc[m][n] = sum_k e4m3(A[m][k]) * e4m3(W[n][k])     (fp32 accumulation)
     Y[m][n]   = fp16( fl32( fl32(acc * sa) * sw ) )
   with sa = a_scale[m] (a_per_row = 1) or a_scale[0] (0), and
   sw = w_scale[n] (w_per_row = 1) or w_scale[0] (0).
   A: E4M3 codes [M][K]; W: E4M3 codes [N][K] (one row per output column,
   both K-contiguous); Y: fp16 [M][N] (output).
   Supported: K % 128 == 0, M*K < 2^32, N*K < 2^32; any M, N >= 1 (M == 0
   or N == 0 is a no-op).  The accumulation order is fixed, so results are
   reproducible; they match the exact sum within fp32 rounding. */
QGEMM_API int32_t qgemm_fp8(const uint8_t* A, const uint8_t* W, const float* a_scale,
                            int32_t a_per_row, const float* w_scale, int32_t w_per_row, uint16_t* Y,
                            int32_t M, int32_t N, int32_t K, void* stream);

/* ------------------------------------------------------------------------
 * INT8 multi-head attention chain  (INT8 cross-modal MHA TensorRT plugin
 * interview page, answer step 3, enqueue core: int8 QK^T GEMM to int32
 * logits; online softmax from fp32 to int8 probabilities with the factor
 * scale_q * scale_k; int8 P.V GEMM; requantization with the output scale and
 * an fp16 bias.  Answer step 2: output [batch, seq, heads, head_dim].
 * Knowledge point 5: int8 codes within [-127, 127]).
 *
 * For batch b, head h, query i, key j, channel c (D = head_dim):
 *   S_ij = sum_c Q[b][i][h][c] * K[b][j][h][c]                (int32, exact)
 *   x_ij = fl32(fl32(S_ij) * alpha)
 *   P_ij = rne(127 * softmax_j(x)_ij)  in [0, 127]    (probability scale 1/127)
 *   A_ic = sum_j P_ij * V[b][j][h][c]                         (int32, exact)
 *   O[b][i][h][c] = clamp(rne(fl32(fl32(fl32(A_ic) * pv_scale) + bias[h*D + c])
 *                              * out_mult), -127, 127)
 * (the bias term only with QGEMM_EPI_BIAS).  alpha is the logit factor the
 * caller forms from its per-tensor dequant scales, scale_q * scale_k, with
 * any 1/sqrt(D) folded in; pv_scale = (1/127) * scale_v.
 *
 * The softmax runs in fp32 (exp2 of the max-shifted logits, an online sum
 * over key blocks, then code = rne(e * fl32(127 / sum))), so a probability
 * code may differ by one from the exactly rounded 127 * p where that value
 * lies within the fp32 error of a rounding boundary; everything else is
 * integer or a fixed fp32 sequence.
 *
 *   Q: int8 [B][Lq][H][D]; K, V: int8 [B][Lk][H][D]; O: int8 [B][Lq][H][D].
 *   bias: fp16 [H*D] (read only with QGEMM_EPI_BIAS).
 *   s_out: optional int32 [B][H][Lq][Lk] logits S; p_out: optional int8
 *   [B][H][Lq][Lk] probability codes P (NULL skips them; for tests).
 *   Supported: D in {64, 128}, 1 <= Lk <= 133143, B and H <= 65535, flags in
 *   {0, QGEMM_EPI_BIAS}.  B, H or Lq == 0 is a successful no-op; Lk == 0 is
 *   QGEMM_BAD_SHAPE.
 * ---------------------------------------------------------------------- */
QGEMM_API int32_t mha_int8(const int8_t* Q, const int8_t* K, const int8_t* V, const uint16_t* bias, int8_t* O,
                           int32_t* s_out, int8_t* p_out, int32_t B, int32_t H, int32_t Lq, int32_t Lk,
                           int32_t D, float alpha, float pv_scale, float out_mult, uint32_t flags,
                           void* stream);

/* ------------------------------------------------------------------------
 * Measurement aid (not a step of the method): reads `bytes` bytes of device
 * memory at `buf` with one 16-byte non-temporal load per lane and address,
 * eight per lane in flight, and discards them (a store to sink[0] that depends
 * on the data keeps the loads; it happens only if the data XOR to one fixed
 * value).  Its rate over a working set is the achievable read bandwidth that
 * the memory-bound kernels are compared with.  bytes must be a multiple of 16,
 * buf 16-byte and sink 4-byte aligned; bytes == 0 is a no-op.
 * ---------------------------------------------------------------------- */
QGEMM_API int32_t qgemm_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* ------------------------------------------------------------------------
 * Measurement aid (not a step of the method): reads src_bytes of device
 * memory at src and writes dst_bytes at dst, in the traffic shapes of the
 * int8 quantizer (dst_bytes == src_bytes / 2: 16 bytes read, 8 written per
 * lane step) and dequantizer (dst_bytes == 2 * src_bytes: 8 read, 16
 * written).  dst receives words derived from src: with s the 32-bit words of
 * src, dst word i = s[2i] ^ s[2i+1] (halving), or dst words 4j .. 4j+3 =
 * s[2j], s[2j+1], s[2j] + 1, s[2j+1] + 1 (doubling).  Its rate is the
 * achievable read+write bandwidth for those shapes.  Both sizes
 * multiples of 16, both pointers 16-byte aligned, the buffers disjoint; any
 * other size ratio is QGEMM_BAD_SHAPE; both sizes 0 is a no-op.
 * ---------------------------------------------------------------------- */
QGEMM_API int32_t qgemm_stream_copy(const void* src, size_t src_bytes, void* dst, size_t dst_bytes,
                                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBQGEMM_H */
