// W4A16 group-wise GEMM: Y[M,N] = A[M,K] (fp16) x (q (int4) * S (fp16, one
// per (K-group, column))), fp32 accumulation, fp16 output.
//
// Int4 Groupwise GEMM Plugin V2 page (class summary: inputs, output and the
// fragment-layout weights; configurePlugin: the token count M steers the
// kernel choice).  Two regimes, chosen by M:
//   decode  (M <= 16): HBM-bound weight stream.  One workgroup per 16-column
//       strip, four waves splitting K; every lane issues its 16-byte weight
//       loads for the whole K slice up front, dequantizes in registers to
//       exact fp16 integers, and v_mfma_f32_16x16x32_f16 forms per-group
//       partial sums (rows >= M are zero) that are scaled in fp32.  The four
//       K partials are added in LDS in a fixed order.
//   prefill (M > 16): MFMA-bound.  128x128 output tiles, four waves of 64x64;
//       A tiles double-buffered through LDS, B fragments straight from the
//       fragment layout into registers, dequantized with the group scale
//       folded in, v_mfma_f32_32x32x16_f16.
#include "common.hpp"
#include "w4_tile.hpp"

namespace {

using namespace qg;

// ------------------------------------------------------------------ decode

__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int G>
__global__ __launch_bounds__(256) void w4a16_decode_kernel(const uint16_t* __restrict__ A,
                                                           const uint8_t* __restrict__ wf,
                                                           const uint16_t* __restrict__ S,
                                                           uint16_t* __restrict__ Y, int M, int N,
                                                           int K) {
    constexpr int BATCH = 8;  // chunks per wave in flight
    const int strip = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int cl = lane & 15, q = lane >> 4;
    const int kchunks = K / 128;
    const int n = strip * 16 + cl;
    const bool arow_ok = cl < M;  // A-fragment row of this lane is cl
    const uint16_t* arow = A + (size_t)(arow_ok ? cl : 0) * K + q * 8;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};

    for (int c0 = wave; c0 < kchunks; c0 += 4 * BATCH) {
        uintx4 raw[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const int c = c0 + 4 * i;
            raw[i] = c < kchunks ? ldg_nt(reinterpret_cast<const uintx4*>(
                                       wf + frag_block_offset(strip, c, kchunks) + lane * 16))
                                 : uintx4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const int c = c0 + 4 * i;
            if (c >= kchunks) break;
            half8 a[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                a[kk] = arow_ok ? *reinterpret_cast<const half8*>(arow + c * 128 + kk * 32)
                                : half8{0, 0, 0, 0, 0, 0, 0, 0};
            }
            const uint32_t d[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
            constexpr int KK_PER_G = G / 32;  // MFMA k-steps per scale group
#pragma unroll
            for (int g0 = 0; g0 < 4; g0 += KK_PER_G) {
                floatx4 tmp = mfma16(a[g0], dequant8(d[g0]), zero);
#pragma unroll
                for (int kk = g0 + 1; kk < g0 + KK_PER_G; ++kk) tmp = mfma16(a[kk], dequant8(d[kk]), tmp);
                const float s = h2f(S[(size_t)((c * 128 + g0 * 32) / G) * N + n]);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = __builtin_fmaf(tmp[j], s, acc[j]);
            }
        }
    }

    __shared__ floatx4 red[4][64];
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        floatx4 s = red[0][lane];
        s += red[1][lane];
        s += red[2][lane];
        s += red[3][lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 4 * q + j;  // accumulator layout: rows 4*(l/16)+j, column l%16
            if (row < M) Y[(size_t)row * N + n] = f2h(s[j]);
        }
    }
}

// ------------------------------------------------------------------ prefill

constexpr int PF_BM = 128, PF_BN = 128, PF_LDA = 136;  // LDS row: 128 halfs + 8 pad

template <int G>
__global__ __launch_bounds__(256, 2) void w4a16_prefill_kernel(const uint16_t* __restrict__ A,
                                                               const uint8_t* __restrict__ wf,
                                                               const uint16_t* __restrict__ S,
                                                               uint16_t* __restrict__ Y, int M,
                                                               int N, int K) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][PF_BM * PF_LDA];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * PF_BM, n0 = blockIdx.x * PF_BN;
    const int kchunks = K / 128;
    const int h = lane >> 5, c32 = lane & 31;
    const int ncol0 = n0 + wn * 64;

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[i][t][j] = 0.f;

    // A staging: 128 rows x 256 bytes = 2048 pieces of 16 bytes, 8 per thread.
    uintx4 areg[8];
    auto load_a = [&](int c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = tid + 256 * i, row = idx >> 4, col = idx & 15;
            const int gm = m0 + row;
            areg[i] = gm < M ? *reinterpret_cast<const uintx4*>(A + (size_t)gm * K + c * 128 + col * 8)
                             : uintx4{0, 0, 0, 0};
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = tid + 256 * i, row = idx >> 4, col = idx & 15;
            *reinterpret_cast<uintx4*>(&sA[buf][row * PF_LDA + col * 8]) = areg[i];
        }
    };

    BChunk<2, G> bcur, bnext;
    load_a(0);
    load_b_chunk<2, G>(bcur, wf, S, N, kchunks, 0, ncol0, lane);
    store_a(0);
    __syncthreads();

    for (int c = 0; c < kchunks; ++c) {
        const int buf = c & 1;
        const bool more = c + 1 < kchunks;
        if (more) {
            load_a(c + 1);
            load_b_chunk<2, G>(bnext, wf, S, N, kchunks, c + 1, ncol0, lane);
        }
        const uint16_t* sa = sA[buf];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int kg = kgroup_of_step(s, h);
            half8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const half8*>(&sa[(wm * 64 + i * 32 + c32) * PF_LDA + kg * 8]);
#pragma unroll
            for (int t = 0; t < 2; ++t) b[t] = b_frag<2, G>(bcur, t, s);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int t = 0; t < 2; ++t) acc[i][t] = mfma32(a[i], b[t], acc[i][t]);
        }
        if (more) {
            store_a(buf ^ 1);
            bcur = bnext;
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int col = ncol0 + t * 32 + c32;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int row = m0 + wm * 64 + i * 32 + acc_row(j, lane);
                if (row < M) Y[(size_t)row * N + col] = f2h(acc[i][t][j]);
            }
        }
}

template <int G>
int32_t launch_w4a16(const uint16_t* A, const uint8_t* wf, const uint16_t* S, uint16_t* Y, int M,
                     int N, int K, hipStream_t st) {
    if (M <= 16) {
        hipLaunchKernelGGL(w4a16_decode_kernel<G>, dim3(N / 16), dim3(256), 0, st, A, wf, S, Y, M,
                           N, K);
    } else {
        dim3 grid(N / PF_BN, (M + PF_BM - 1) / PF_BM);
        hipLaunchKernelGGL(w4a16_prefill_kernel<G>, grid, dim3(256), 0, st, A, wf, S, Y, M, N, K);
    }
    return qgh::launch_status();
}

}  // namespace

extern "C" size_t qgemm_w4a16_workspace_bytes(int32_t, int32_t, int32_t, int32_t) { return 0; }

extern "C" int32_t qgemm_w4a16(const uint16_t* A, const uint8_t* w_frag, const uint16_t* scales,
                               uint16_t* Y, int32_t M, int32_t N, int32_t K, int32_t G,
                               void* workspace, size_t workspace_bytes, void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    if (M < 0 || N < 0 || K < 0 || G <= 0) return QGEMM_BAD_SHAPE;
    if (K % G != 0) return QGEMM_BAD_SHAPE;
    if (M == 0) return QGEMM_OK;
    if (!A || !w_frag || !scales || !Y) return QGEMM_NULL_PTR;
    if (N == 0 || K == 0 || N % 128 != 0 || K % 128 != 0) return QGEMM_UNSUPPORTED;
    if (G != 32 && G != 64 && G != 128) return QGEMM_UNSUPPORTED;
    if (!qgh::aligned(A, 16) || !qgh::aligned(w_frag, 16) || !qgh::aligned(scales, 4) ||
        !qgh::aligned(Y, 16))
        return QGEMM_MISALIGNED;
    hipStream_t st = (hipStream_t)stream;
    switch (G) {
        case 32: return launch_w4a16<32>(A, w_frag, scales, Y, M, N, K, st);
        case 64: return launch_w4a16<64>(A, w_frag, scales, Y, M, N, K, st);
        default: return launch_w4a16<128>(A, w_frag, scales, Y, M, N, K, st);
    }
}
