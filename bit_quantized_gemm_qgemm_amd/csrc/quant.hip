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
// 256 values, a whole wave otherwise) with no cross-workgroup traffic; the
// codes are written from the registers that held the inputs, so the input is
// read from HBM once.  The arithmetic is the bit-exact sequence
//   mult = 127 / amax; scale = amax / 127; q = clamp(rne(x * mult), +-127)
// (correctly rounded fp32 division, no contraction).
#include "common.hpp"

namespace {

using qg::uintx2;
using qg::uintx4;

__device__ __forceinline__ uint32_t quant4(uint32_t h01, uint32_t h23, float mult) {
    // four fp16 values (two words) -> four int8 codes in one word
    const float x[4] = {qg::h2f(h01 & 0xffffu), qg::h2f(h01 >> 16), qg::h2f(h23 & 0xffffu),
                        qg::h2f(h23 >> 16)};
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v = __builtin_rintf(x[i] * mult);
        v = fminf(fmaxf(v, -127.0f), 127.0f);
        out |= ((uint32_t)(int32_t)v & 0xffu) << (8 * i);
    }
    return out;
}

// Rows held in registers: each of LPR lanes holds CPL chunks of 8 values.
template <int LPR, int CPL>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ X,
                                                         int8_t* __restrict__ Q,
                                                         float* __restrict__ S, int rows,
                                                         int cols) {
    constexpr int RPB = 256 / LPR;  // rows per block
    const int lane = threadIdx.x % LPR;
    const int row = blockIdx.x * RPB + threadIdx.x / LPR;
    const bool live = row < rows;
    const int nchunk = cols / 8;
    const uint16_t* x = X + (size_t)(live ? row : 0) * cols;
    // Every load is unconditional (a chunk past the row end reads chunk 0 and
    // is then zeroed): a load under a branch makes the compiler wait for all
    // outstanding loads at the join, serializing the lane's loads.
    uintx4 v[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + i * LPR;
        v[i] = qg::ldg_nt(reinterpret_cast<const uintx4*>(x) + (c < nchunk ? c : 0));
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        if (lane + i * LPR >= nchunk) v[i] = uintx4{0, 0, 0, 0};
        amax = fmaxf(amax, qg::absmax8(v[i]));
    }
    amax = qg::group_max<LPR>(amax);
    if (!live) return;
    const float mult = amax > 0.0f ? 127.0f / amax : 0.0f;
    if (lane == 0) S[row] = amax > 0.0f ? amax / 127.0f : 0.0f;
    int8_t* q = Q + (size_t)row * cols;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + i * LPR;
        if (c < nchunk) {
            const uint32_t lo = quant4(v[i].x, v[i].y, mult);
            const uint32_t hi = quant4(v[i].z, v[i].w, mult);
            reinterpret_cast<uintx2*>(q)[c] = uintx2{lo, hi};
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
    const float mult = amax > 0.0f ? 127.0f / amax : 0.0f;
    if (lane == 0) S[row] = amax > 0.0f ? amax / 127.0f : 0.0f;
    uintx2* q = reinterpret_cast<uintx2*>(Q + (size_t)row * cols);
    for (int c = lane; c < nchunk; c += 64) {
        const uintx4 v = x[c];
        q[c] = uintx2{quant4(v.x, v.y, mult), quant4(v.z, v.w, mult)};
    }
}

// Dequantization: each lane turns a chunk of 8 codes of one row into fp16
// (cols % 8 == 0, so a chunk never straddles rows); grid-stride over chunks.
__global__ __launch_bounds__(256) void dequant_kernel(const int8_t* __restrict__ Q,
                                                      const float* __restrict__ S,
                                                      uint16_t* __restrict__ X, size_t nchunk,
                                                      int chunks_per_row) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunk; c += stride) {
        const uintx2 q = qg::ldg_nt(reinterpret_cast<const uintx2*>(Q) + c);
        const float s = S[c / chunks_per_row];
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
        reinterpret_cast<uintx4*>(X)[c] = uintx4{o[0], o[1], o[2], o[3]};
    }
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
    if (cols <= 16 * 8 * 2) {
        const int rpb = 256 / 16;
        hipLaunchKernelGGL((quant_rows_kernel<16, 2>), dim3((rows + rpb - 1) / rpb), dim3(256), 0,
                           st, X, Q, scales, (int)rows, (int)cols);
    } else if (cols <= 64 * 8 * 8) {
        const int rpb = 256 / 64;
        hipLaunchKernelGGL((quant_rows_kernel<64, 8>), dim3((rows + rpb - 1) / rpb), dim3(256), 0,
                           st, X, Q, scales, (int)rows, (int)cols);
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
    const size_t want = (nchunk + 255) / 256;
    const int blocks = (int)(want < 8192 ? want : 8192);
    hipLaunchKernelGGL(dequant_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, Q, scales,
                       X, nchunk, (int)(cols / 8));
    return qgh::launch_status();
}
