// Offline weight repack: natural int4 [K][N/2] -> gfx950 fragment layout.
//
// The Int4 Groupwise GEMM Plugin V2 page (class summary) consumes weights
// already in a fragment layout, repacked at export time with the N tile
// pinned at 128; there is no repack at run time.  Here the tile is
// 128 columns x 128 k (8 KB): eight 1 KB blocks of 16 columns, each block
// exactly what one wave64 loads with one 16-byte load per lane and feeds to
// v_mfma_f32_16x16x32_f16 as four B fragments (one 128-k scale group).
#include "common.hpp"

namespace {

// One workgroup per 128 x 128 tile: stage the natural bytes (128 rows x 64 B)
// in LDS with coalesced loads, then write the 8 KB fragment tile with
// coalesced 16-byte stores.
__global__ __launch_bounds__(256) void prepack_kernel(const uint8_t* __restrict__ wn,
                                                      uint8_t* __restrict__ wf, int K, int N) {
    __shared__ uint32_t tile[128][17];  // 64 bytes per row + pad
    const int n_tile = blockIdx.x;      // 128-column tile
    const int c = blockIdx.y;           // 128-k chunk
    const int t = threadIdx.x;
    const int row_bytes = N / 2;
    // 128 rows x 16 words: 2048 words, 8 per thread; words past K or N (a
    // ragged shape's last tile) are weight 0, nibbles 0
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int w = t + 256 * i;
        const int r = w >> 4, cw = w & 15;
        const int k = c * 128 + r, byte = n_tile * 64 + cw * 4;
        tile[r][cw] = (k < K && byte < row_bytes)
                          ? *reinterpret_cast<const uint32_t*>(wn + (size_t)k * row_bytes + byte)
                          : 0u;
    }
    __syncthreads();
    // thread t writes words 8t .. 8t+7 of the tile
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int wi = 8 * t + i;
        const int b = wi >> 8;           // block (strip inside tile)
        const int p = (wi & 255) >> 2;   // lane position
        const int kk = wi & 3;
        const int cl = p & 15, q = p >> 4;
        const int n_local = b * 16 + cl;
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k_local = kk * 32 + q * 8 + j;
            const uint32_t byte = (tile[k_local][n_local >> 3] >> (8 * ((n_local >> 1) & 3))) & 0xffu;
            const uint32_t nib = ((n_local & 1) ? (byte >> 4) : byte) & 0xfu;
            const int pos = (j >> 1) + 4 * (j & 1);
            word |= (nib ^ 8u) << (4 * pos);
        }
        out[i] = word;
    }
    const int kchunks = (K + 127) / 128;
    uint8_t* dst = wf + ((size_t)n_tile * kchunks + c) * 8192u + (size_t)t * 32u;
    reinterpret_cast<qg::uintx4*>(dst)[0] = qg::uintx4{out[0], out[1], out[2], out[3]};
    reinterpret_cast<qg::uintx4*>(dst)[1] = qg::uintx4{out[4], out[5], out[6], out[7]};
}

}  // namespace

// K and N are padded to whole 128 x 128 tiles (weight 0 in the padding).
extern "C" size_t qgemm_w4a16_packed_bytes(int32_t K, int32_t N) {
    if (K <= 0 || N <= 0 || K % 8 != 0 || N % 8 != 0) return 0;
    return (size_t)((K + 127) / 128) * 128 * (size_t)((N + 127) / 128) * 128 / 2;
}

extern "C" int32_t qgemm_w4a16_prepack(const uint8_t* w_natural, uint8_t* w_frag, int32_t K,
                                       int32_t N, void* stream) {
    if (!w_natural || !w_frag) return QGEMM_NULL_PTR;
    if (K < 0 || N < 0) return QGEMM_BAD_SHAPE;
    if (K == 0 || N == 0) return QGEMM_OK;
    if (K % 8 != 0 || N % 8 != 0) return QGEMM_UNSUPPORTED;
    if (!qgh::aligned(w_natural, 16) || !qgh::aligned(w_frag, 16)) return QGEMM_MISALIGNED;
    const size_t in_bytes = (size_t)K * N / 2, out_bytes = qgemm_w4a16_packed_bytes(K, N);
    const uintptr_t a = (uintptr_t)w_natural, b = (uintptr_t)w_frag;
    if (a < b + out_bytes && b < a + in_bytes) return QGEMM_BAD_SHAPE;  // overlapping buffers
    dim3 grid((N + 127) / 128, (K + 127) / 128);
    hipLaunchKernelGGL(prepack_kernel, grid, dim3(256), 0, (hipStream_t)stream, w_natural, w_frag,
                       (int)K, (int)N);
    return qgh::launch_status();
}
