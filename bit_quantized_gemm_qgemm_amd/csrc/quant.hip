// Per-row symmetric int8 quantization and dequantization.
//
// INT8 cross-modal MHA TensorRT plugin interview page: answer step 1 (one
// scale = 127 / max|x| per weight output channel and per activation token),
// extension point 1 (the per-token max found online by a wave reduction),
// knowledge point 5 (codes limited to [-127, 127]).  KV Cache INT8量化 page:
// quantize_symmetric (scale = max|x| / 127) and dequantize_symmetric
// (x = q * scale), applied here with one scale per (head, token) row.
//
// Each row is reduced by one group of lanes (16 lanes for rows of at most
// 256 values, one or two 16-byte chunks each; a whole wave otherwise) with no cross-workgroup traffic; the
// codes are written from the registers that held the inputs, so the input is
// read from HBM once.  The arithmetic is the bit-exact sequence
//   mult = 127 / amax; scale = amax / 127; q = clamp(rne(x * mult), +-127)
// (correctly rounded fp32 division, no contraction).
#include "common.hpp"

namespace {

using qg::uintx2;
using qg::uintx4;

__device__ __forceinline__ uint32_t quant4(uint32_t h01, uint32_t h23, float mult) {
    // four fp16 values (two words) -> four int8 codes in one word.
    // m = fl32(x * mult) as fma(x, mult, +0): one rounding of the same product,
    // and the fp16 operand is read in place (v_fma_mix_f32, no conversion
    // instruction); the two can differ only in the sign of a zero product,
    // which gives code 0 either way.  No clamp to [-127, 127] is needed: with
    // |x| <= amax and mult = fl32(127 / amax) <= (127 / amax)(1 + 2^-24), the
    // product is at most 127 (1 + 2^-24) in magnitude and rounds to at most
    // 127 (inputs are finite).  Rounding to an integer: m + 1.5 * 2^23 lies in
    // [2^23, 2^24), where the fp32 spacing is 1, so the addition rounds m to
    // nearest, ties to even, and the sum's low mantissa bits hold that integer
    // (0x4B400000 + rne(m)); its low byte is the two's-complement code.  Four
    // low bytes are gathered by byte permutes.
    const float x[4] = {qg::h2f(h01 & 0xffffu), qg::h2f(h01 >> 16), qg::h2f(h23 & 0xffffu),
                        qg::h2f(h23 >> 16)};
    uint32_t f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __builtin_bit_cast(uint32_t, __builtin_fmaf(x[i], mult, 0.0f) + 12582912.0f);
    const uint32_t lo = __builtin_amdgcn_perm(f[1], f[0], 0x0c0c0400u);  // bytes: f0.b0, f1.b0, 0, 0
    const uint32_t hi = __builtin_amdgcn_perm(f[3], f[2], 0x04000c0cu);  // bytes: 0, 0, f2.b0, f3.b0
    return lo | hi;
}

// mult = 127 / a and scale = a / 127, correctly rounded, for a = max |x| of
// fp16 values (so a is 0, +inf or a positive finite fp16 value): v_rcp_f32
// with one fused correction of the quotient gives the correctly rounded
// result for every positive finite fp16 a (checked on gfx950 over all 31743
// of them against the IEEE divisions), in four operations instead of the
// division's ten; a = 0 gives 0 and 0, a = +inf gives 0 and +inf, as the
// divisions (and the zero-row rule) do.
__device__ __forceinline__ void int8_scales(float a, float& mult, float& scale) {
    const float r = __builtin_amdgcn_rcpf(a);
    const float q = 127.0f * r;
    const float m = __builtin_fmaf(__builtin_fmaf(-a, q, 127.0f), r, q);
    constexpr float r127 = 1.0f / 127.0f;
    const float s0 = a * r127;
    const float sc = __builtin_fmaf(__builtin_fmaf(-s0, 127.0f, a), r127, s0);
    const bool fin = a < __builtin_inff();
    mult = a > 0.0f ? (fin ? m : 0.0f) : 0.0f;
    scale = a > 0.0f ? (fin ? sc : a) : 0.0f;
}

// Rows held in registers: each of LPR lanes holds CPL chunks of 8 values;
// FULL: cols == LPR * CPL * 8, so every chunk is in the row.  A lane group
// takes NR rows (rows g + r * RPB of its block's RPB * NR), all their loads
// issued before the first reduction.
template <int LPR, int CPL, bool FULL, int NR = 1>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ X,
                                                         int8_t* __restrict__ Q,
                                                         float* __restrict__ S, int rows,
                                                         int cols) {
    constexpr int RPB = 256 / LPR;  // rows per block and pass
    const int lane = threadIdx.x % LPR;
    const int nchunk = cols / 8;
    // Every load is unconditional (a chunk past the row end reads chunk 0 and
    // is then zeroed; a row past the last reads row 0 and stores nothing): a
    // load under a branch makes the compiler wait for all outstanding loads
    // at the join, serializing the lane's loads.
    int row[NR];
    uintx4 v[NR][CPL];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        row[r] = (blockIdx.x * NR + r) * RPB + threadIdx.x / LPR;
        const uint16_t* x = X + (size_t)(row[r] < rows ? row[r] : 0) * cols;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + i * LPR;
            v[r][i] = qg::ldg_nt(reinterpret_cast<const uintx4*>(x) + (FULL || c < nchunk ? c : 0));
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            if (!FULL && lane + i * LPR >= nchunk) v[r][i] = uintx4{0, 0, 0, 0};
            amax = fmaxf(amax, qg::absmax8(v[r][i]));
        }
        amax = qg::group_max<LPR>(amax);
        if (row[r] >= rows) continue;  // (uniform over the lane group)
        float mult, scale;
        int8_scales(amax, mult, scale);
        if (lane == 0) S[row[r]] = scale;
        int8_t* q = Q + (size_t)row[r] * cols;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + i * LPR;
            if (FULL || c < nchunk) {
                const uint32_t lo = quant4(v[r][i].x, v[r][i].y, mult);
                const uint32_t hi = quant4(v[r][i].z, v[r][i].w, mult);
                reinterpret_cast<uintx2*>(q)[c] = uintx2{lo, hi};
            }
        }
    }
}

// Long rows: one wave per row, two passes over the row (max, then codes).
__global__ __launch_bounds__(256) void quant_rows_long_kernel(const uint16_t* __restrict__ X,
                                                              int8_t* __restrict__ Q,
                                                              float* __restrict__ S, int rows,
                                                              int cols) {
    const int lane = threadIdx.x % 64;
    const int row = blockIdx.x * 4 + threadIdx.x / 64;
    if (row >= rows) return;
    const int nchunk = cols / 8;
    const uintx4* x = reinterpret_cast<const uintx4*>(X + (size_t)row * cols);
    float amax = 0.0f;
    for (int c = lane; c < nchunk; c += 64) amax = fmaxf(amax, qg::absmax8(x[c]));
    amax = qg::group_max<64>(amax);
    float mult, scale;
    int8_scales(amax, mult, scale);
    if (lane == 0) S[row] = scale;
    uintx2* q = reinterpret_cast<uintx2*>(Q + (size_t)row * cols);
    for (int c = lane; c < nchunk; c += 64) {
        const uintx4 v = x[c];
        q[c] = uintx2{quant4(v.x, v.y, mult), quant4(v.z, v.w, mult)};
    }
}

// Dequantization: a lane turns chunks of 8 codes of one row into fp16
// (cols % 8 == 0, so a chunk never straddles rows); grid-stride over chunks,
// DQ_U chunks per lane per step, all their loads issued first.  At the
// KV-cache size (1 M chunks, 1024 blocks: one step) 6.18 -> 5.50 us against
// one chunk per lane over 4096 blocks; eight chunks over 512 blocks 5.48, two
// over 2048 blocks 5.70, four or two over half the blocks (two steps) 6.2 to
// 6.3 (one box).
// IDX: the chunk index type (32 bits whenever the indexes fit, which turns
// the row index's 64-bit division into a 32-bit one); row_shift >= 0: chunks
// per row = 1 << row_shift, and the row index is a shift.
constexpr int DQ_U = 4, DQ_BLOCKS = 1024;

__device__ __forceinline__ uintx4 dequant8(uintx2 q, float s) {
    const uint32_t w[2] = {q.x, q.y};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t a = qg::f2h_of_product((float)(int8_t)((w[i] >> (16 * j)) & 0xffu), s);
            const uint32_t b = qg::f2h_of_product((float)(int8_t)((w[i] >> (16 * j + 8)) & 0xffu), s);
            o[2 * i + j] = a | (b << 16);
        }
    }
    return uintx4{o[0], o[1], o[2], o[3]};
}

template <typename IDX>
__global__ __launch_bounds__(256) void dequant_kernel(const int8_t* __restrict__ Q,
                                                      const float* __restrict__ S,
                                                      uint16_t* __restrict__ X, IDX nchunk,
                                                      int chunks_per_row, int row_shift) {
    const IDX stride = (IDX)gridDim.x * blockDim.x;
    const uintx2* q2 = reinterpret_cast<const uintx2*>(Q);
    uintx4* x4 = reinterpret_cast<uintx4*>(X);
    auto row = [&](IDX c) { return row_shift >= 0 ? c >> row_shift : c / (IDX)chunks_per_row; };
    IDX c = (IDX)blockIdx.x * blockDim.x + threadIdx.x;
    // non-temporal stores: 6.62 -> 6.24 us for the KV cache with one chunk
    // per lane (plain stores were faster for the quantizers' 8-byte codes)
    for (; c + (DQ_U - 1) * stride < nchunk; c += DQ_U * stride) {
        uintx2 q[DQ_U];
        float s[DQ_U];
#pragma unroll
        for (int i = 0; i < DQ_U; ++i) q[i] = qg::ldg_nt(q2 + c + i * stride);
#pragma unroll
        for (int i = 0; i < DQ_U; ++i) s[i] = S[row(c + i * stride)];
#pragma unroll
        for (int i = 0; i < DQ_U; ++i) __builtin_nontemporal_store(dequant8(q[i], s[i]), x4 + c + i * stride);
    }
    for (; c < nchunk; c += stride) __builtin_nontemporal_store(dequant8(qg::ldg_nt(q2 + c), S[row(c)]), x4 + c);
}

}  // namespace

extern "C" int32_t quant_sym_int8(const uint16_t* X, int8_t* Q, float* scales, int32_t rows,
                                  int32_t cols, void* stream) {
    if (!X || !Q || !scales) return QGEMM_NULL_PTR;
    if (rows < 0 || cols < 0) return QGEMM_BAD_SHAPE;
    if (rows == 0) return QGEMM_OK;
    if (cols == 0 || cols % 8 != 0 || cols > 65536) return QGEMM_UNSUPPORTED;
    if (!qgh::aligned(X, 16) || !qgh::aligned(Q, 8) || !qgh::aligned(scales, 4))
        return QGEMM_MISALIGNED;
    hipStream_t st = (hipStream_t)stream;
    // rows of up to 128 values (the KV cache's head_dim): 8 lanes of two
    // 16-byte chunks per row (7.34 us for 65,536 rows of 128 with 16 lanes of
    // two chunks, 6.83 with 16 lanes of one, 6.46 with 8 of two, 6.90 with 4
    // of four; 6.12 once quant4 took the fma-mix product and dropped the clamp)
    // (two rows per lane group for rows of 128 values: 6.17 -> 6.08 us at
    // 65,536 rows, four loads per lane in flight; four rows 6.66, and
    // non-temporal code stores 6.41)
    auto launch = [&](auto kern, int lpr, int nr) {
        const int rpb = 256 / lpr * nr;
        hipLaunchKernelGGL(kern, dim3((rows + rpb - 1) / rpb), dim3(256), 0, st, X, Q, scales, (int)rows,
                           (int)cols);
    };
    if (cols == 8 * 8 * 2) {
        launch(quant_rows_kernel<8, 2, true, 2>, 8, 2);
    } else if (cols < 8 * 8 * 2) {
        launch(quant_rows_kernel<8, 2, false>, 8, 1);
    } else if (cols <= 16 * 8 * 2) {
        launch(quant_rows_kernel<16, 2, false>, 16, 1);
    } else if (cols == 64 * 8 * 8) {
        launch(quant_rows_kernel<64, 8, true>, 64, 1);
    } else if (cols <= 64 * 8 * 8) {
        launch(quant_rows_kernel<64, 8, false>, 64, 1);
    } else {
        hipLaunchKernelGGL(quant_rows_long_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, X, Q,
                           scales, (int)rows, (int)cols);
    }
    return qgh::launch_status();
}

extern "C" int32_t dequant_sym_int8(const int8_t* Q, const float* scales, uint16_t* X,
                                    int32_t rows, int32_t cols, void* stream) {
    if (!X || !Q || !scales) return QGEMM_NULL_PTR;
    if (rows < 0 || cols < 0) return QGEMM_BAD_SHAPE;
    if (rows == 0) return QGEMM_OK;
    if (cols == 0 || cols % 8 != 0) return QGEMM_UNSUPPORTED;
    if (!qgh::aligned(X, 16) || !qgh::aligned(Q, 8) || !qgh::aligned(scales, 4))
        return QGEMM_MISALIGNED;
    const size_t nchunk = (size_t)rows * cols / 8;
    const size_t want = (nchunk + 256 * DQ_U - 1) / (256 * DQ_U);
    const int blocks = (int)(want < DQ_BLOCKS ? want : DQ_BLOCKS);
    const int cpr = cols / 8, shift = (cpr & (cpr - 1)) == 0 ? __builtin_ctz((unsigned)cpr) : -1;
    if (nchunk + (size_t)blocks * 256 * DQ_U < ((size_t)1 << 32))
        hipLaunchKernelGGL(dequant_kernel<uint32_t>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, Q, scales,
                           X, (uint32_t)nchunk, cpr, shift);
    else
        hipLaunchKernelGGL(dequant_kernel<size_t>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, Q, scales,
                           X, nchunk, cpr, shift);
    return qgh::launch_status();
}
