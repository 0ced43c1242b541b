// W8A16 weight-only int8 GEMM: Y[M,N] = A[M,K] (fp16) x (q (int8) * S (fp16,
// one per (K-group, column), or one per column)), fp32 accumulation, fp16
// output.
//
// FP8 vs INT8 low-precision inference in TensorRT-LLM (itzkxy.com): among
// the INT8 configurations compared there is weight-only int8 with fp16
// activations.  The kernels are the weight-only ones of wq_gemm.hpp with the
// int8 fragment layout (2 KB blocks of 16 columns x 128 k, stored v + 128):
// decode for M <= 16 (twice the weight bytes of W4A16 per column, so the
// kernel is HBM-bound on a 2x larger stream), mid-M split-K with a
// workspace, and the 128x128 or (with enough tiles) 128x256 MFMA prefill
// kernels for every other M.
#include "common.hpp"
#include "wq_gemm.hpp"

namespace {

using namespace qg;

// One workgroup per 128 x 128 tile: stage the natural bytes (128 rows x
// 128 B) in LDS with coalesced 16-byte loads, then write the 16 KB fragment
// tile with coalesced 16-byte stores.  Piece i of the tile (16 bytes) is
// block i / 128, half (i / 64) % 2, lane position p = i % 64 (column
// p % 16 of the block, q = p / 16); its byte b holds k-step
// kk = 2 * half + b / 8, j = b % 8, i.e. k = 32 kk + 8 q + j of the chunk.
constexpr int P8_PITCH = 144;  // LDS bytes per staged row (128 + 16 pad)

__global__ __launch_bounds__(256) void prepack8_kernel(const int8_t* __restrict__ wn,
                                                       uint8_t* __restrict__ wf, int K, int N) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[128 * P8_PITCH];
    const int n_tile = blockIdx.x, c = blockIdx.y, t = threadIdx.x;
    // 8-byte pieces (rows of N % 8 == 0 bytes are 8-byte aligned); pieces past
    // K or N (a ragged shape's last tile) are weight 0
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int idx = t + 256 * i, r = idx >> 4, col = idx & 15;
        const int k = c * 128 + r, n = n_tile * 128 + col * 8;
        *reinterpret_cast<uintx2*>(&tile[r * P8_PITCH + col * 8]) =
            (k < K && n < N) ? *reinterpret_cast<const uintx2*>(wn + (size_t)k * N + n) : uintx2{0u, 0u};
    }
    __syncthreads();
    const int kchunks = (K + 127) / 128;
    uint8_t* dst = wf + ((size_t)n_tile * kchunks + c) * 16384u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int pi = t + 256 * i;
        const int blk = pi >> 7, half = (pi >> 6) & 1, p = pi & 63;
        const int n_local = blk * 16 + (p & 15), q = p >> 4;
        uint32_t w[4];
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
            uint32_t word = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int byte = 4 * wi + b;
                const int k_local = (2 * half + (byte >> 3)) * 32 + q * 8 + (byte & 7);
                word |= (uint32_t)(tile[k_local * P8_PITCH + n_local] ^ 0x80u) << (8 * b);
            }
            w[wi] = word;
        }
        *reinterpret_cast<uintx4*>(dst + (size_t)pi * 16) = uintx4{w[0], w[1], w[2], w[3]};
    }
}

template <int G>
int32_t launch_w8a16(const uint16_t* A, const uint8_t* wf, const uint16_t* S, int ldS, uint16_t* Y, int M,
                     int N, int K, float* part, hipStream_t st) {
    if (M <= 16) {
        launch_wq_decode<8, G>(A, wf, S, ldS, Y, M, N, K, st);
    } else if (part) {
        launch_wq_mid<8, G>(A, wf, S, ldS, Y, M, N, K, part, st);
    } else if (ragged(N, K) || N % PL_BN != 0 || (long)(N / PL_BN) * ((M + PL_BM - 1) / PL_BM) < 160) {
        launch_wq_prefill<8, G>(A, wf, S, ldS, Y, M, N, K, st);
    } else {
        // the 128x256 kernel once it has enough tiles for the chip (the W4A16 rule)
        dim3 grid((N / PL_BN) * ((M + PL_BM - 1) / PL_BM));
        hipLaunchKernelGGL((wq_prefill_large_kernel<8, G>), grid, dim3(256), 0, st, A, wf, S, ldS, Y, M, N, K);
    }
    return qgh::launch_status();
}

bool w8a16_group_ok(int G, int K) { return G == 32 || G == 64 || G == 128 || G == K; }

}  // namespace

// K and N are padded to whole 128 x 128 tiles (weight 0 in the padding).
extern "C" size_t qgemm_w8a16_packed_bytes(int32_t K, int32_t N) {
    if (K <= 0 || N <= 0 || K % 8 != 0 || N % 8 != 0) return 0;
    return (size_t)((K + 127) / 128) * 128 * (size_t)((N + 127) / 128) * 128;
}

extern "C" int32_t qgemm_w8a16_prepack(const int8_t* w_natural, uint8_t* w_frag, int32_t K, int32_t N,
                                       void* stream) {
    if (!w_natural || !w_frag) return QGEMM_NULL_PTR;
    if (K < 0 || N < 0) return QGEMM_BAD_SHAPE;
    if (K == 0 || N == 0) return QGEMM_OK;
    if (K % 8 != 0 || N % 8 != 0) return QGEMM_UNSUPPORTED;
    if (!qgh::aligned(w_natural, 16) || !qgh::aligned(w_frag, 16)) return QGEMM_MISALIGNED;
    const size_t in_bytes = (size_t)K * N, out_bytes = qgemm_w8a16_packed_bytes(K, N);
    const uintptr_t a = (uintptr_t)w_natural, b = (uintptr_t)w_frag;
    if (a < b + out_bytes && b < a + in_bytes) return QGEMM_BAD_SHAPE;  // overlapping buffers
    hipLaunchKernelGGL(prepack8_kernel, dim3((N + 127) / 128, (K + 127) / 128), dim3(256), 0, (hipStream_t)stream,
                       w_natural, w_frag, (int)K, (int)N);
    return qgh::launch_status();
}

extern "C" size_t qgemm_w8a16_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t G) {
    if (M <= 0 || N <= 0 || K <= 0 || G <= 0 || N % 8 != 0 || K % 8 != 0 || ragged(N, K)) return 0;
    if (!w8a16_group_ok(G, K)) return 0;
    return mid_path(M, K) ? mid_workspace_bytes(M, N, K) : 0;
}

extern "C" int32_t qgemm_w8a16(const uint16_t* A, const uint8_t* w_frag, const uint16_t* scales, uint16_t* Y,
                               int32_t M, int32_t N, int32_t K, int32_t G, void* workspace,
                               size_t workspace_bytes, void* stream) {
    if (M < 0 || N < 0 || K < 0 || G <= 0) return QGEMM_BAD_SHAPE;
    if (M == 0) return QGEMM_OK;
    if (!A || !w_frag || !scales || !Y) return QGEMM_NULL_PTR;
    if (N == 0 || K == 0 || N % 8 != 0 || K % 8 != 0) return QGEMM_UNSUPPORTED;
    if (!w8a16_group_ok(G, K)) return QGEMM_UNSUPPORTED;
    if (!qgh::aligned(A, 16) || !qgh::aligned(w_frag, 16) || !qgh::aligned(scales, 4) ||
        !qgh::aligned(Y, 16))
        return QGEMM_MISALIGNED;
    hipStream_t st = (hipStream_t)stream;
    float* part = nullptr;
    if (!ragged(N, K) && mid_path(M, K) && workspace && qgh::aligned(workspace, 16) &&
        workspace_bytes >= mid_workspace_bytes(M, N, K))
        part = static_cast<float*>(workspace);
    // one scale per column (G == K > 128): 128-k groups that all read scale row 0
    const int ldS = G > 128 ? 0 : N;
    switch (G) {
        case 32: return launch_w8a16<32>(A, w_frag, scales, ldS, Y, M, N, K, part, st);
        case 64: return launch_w8a16<64>(A, w_frag, scales, ldS, Y, M, N, K, part, st);
        default: return launch_w8a16<128>(A, w_frag, scales, ldS, Y, M, N, K, part, st);
    }
}
