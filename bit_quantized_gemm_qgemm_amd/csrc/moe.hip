// INT4 mixture-of-experts layer (Int4 Moe Plugin page, constructor:
// numExperts, topK, hiddenSize, moeInterSize, activationType,
// quantizationGroupSize; one output).  Five stream-ordered launches:
//   1. route:   per token, top-k experts by logit (lower index wins ties) and
//               softmax over the selected logits (fp32);
//   2. permute: one workgroup groups the (token, j) pairs by expert, keeping
//               ascending pair order inside an expert (wave ballots, no
//               atomics on the result order), and records each pair's slot;
//   3. gate/up: per expert, a W4A16 MFMA GEMM over that expert's gathered
//               token rows with both the gate and the up matrix, fused with
//               h = fp16(silu(g) * u);
//   4. down:    per expert, W4A16 MFMA GEMM of h with the down matrix, fp32
//               results per slot;
//   5. combine: y[t] = fp16(sum_j w[t][j] * o[slot(t, j)]), j ascending.
// Every reduction has a fixed order, so the layer is deterministic.
#include "common.hpp"
#include "w4_tile.hpp"

namespace {

using namespace qg;

constexpr int MBM = 64, MBN = 128, MLDA = 136;

struct Work {
    int32_t* offsets;
    int32_t* pairs;
    int32_t* slot_of;
    uint16_t* h;
    float* o;
};

__host__ __device__ inline void workspace_layout(int T, int H, int I, int E, int topK, size_t* off) {
    const size_t P = (size_t)T * topK;
    size_t x = 0;
    off[0] = x;
    x = (x + sizeof(int32_t) * (E + 1) + 255) & ~(size_t)255;
    off[1] = x;
    x = (x + sizeof(int32_t) * P + 255) & ~(size_t)255;
    off[2] = x;
    x = (x + sizeof(int32_t) * P + 255) & ~(size_t)255;
    off[3] = x;
    x = (x + sizeof(uint16_t) * P * I + 255) & ~(size_t)255;
    off[4] = x;
    x = (x + sizeof(float) * P * H + 255) & ~(size_t)255;
    off[5] = x;
}

// ------------------------------------------------------------------ route

__global__ __launch_bounds__(256) void moe_route_kernel(const uint16_t* __restrict__ logits,
                                                        int32_t* __restrict__ ids,
                                                        float* __restrict__ w, int T, int E,
                                                        int topK) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    const uint16_t* l = logits + (size_t)t * E;
    uint64_t taken = 0;
    float vals[64];
    int sel[64];
    for (int j = 0; j < topK; ++j) {
        int best = -1;
        float bv = 0.0f;
        for (int e = 0; e < E; ++e) {
            if ((taken >> e) & 1ull) continue;
            const float v = h2f(l[e]);
            if (best < 0 || v > bv) {
                best = e;
                bv = v;
            }
        }
        taken |= 1ull << best;
        sel[j] = best;
        vals[j] = bv;
    }
    const float lmax = vals[0];
    float sum = 0.0f;
    for (int j = 0; j < topK; ++j) {
        vals[j] = expf(vals[j] - lmax);
        sum += vals[j];
    }
    for (int j = 0; j < topK; ++j) {
        ids[(size_t)t * topK + j] = sel[j];
        w[(size_t)t * topK + j] = vals[j] / sum;
    }
}

// ------------------------------------------------------------------ permute

__global__ __launch_bounds__(1024) void moe_permute_kernel(const int32_t* __restrict__ ids, int P,
                                                           int E, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ pairs,
                                                           int32_t* __restrict__ slot_of) {
    __shared__ int cnt[64];
    __shared__ int base[64];
    __shared__ int wave_cnt[16][64];
    __shared__ int wave_off[16][64];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (tid < 64) cnt[tid] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += 1024) atomicAdd(&cnt[ids[p]], 1);
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int e = 0; e < E; ++e) {
            base[e] = run;
            offsets[e] = run;
            run += cnt[e];
        }
        offsets[E] = run;
    }
    __syncthreads();
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int b0 = 0; b0 < P; b0 += 1024) {
        const int p = b0 + tid;
        const int e = p < P ? ids[p] : -1;
        int rank = 0;
        for (int x = 0; x < E; ++x) {
            const uint64_t m = __ballot(e == x);
            if (e == x) rank = __popcll(m & below);
            if (lane == 0) wave_cnt[wave][x] = __popcll(m);
        }
        __syncthreads();
        if (tid < E) {
            int run = base[tid];
            for (int wv = 0; wv < 16; ++wv) {
                wave_off[wv][tid] = run;
                run += wave_cnt[wv][tid];
            }
            base[tid] = run;
        }
        __syncthreads();
        if (e >= 0) {
            const int pos = wave_off[wave][e] + rank;
            pairs[pos] = p;
            slot_of[p] = pos;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ grouped GEMMs

// Shared main loop: 64 x 128 output tile of one expert; four waves of 32 x 64
// (one 32-row MFMA tile, two 32-column tiles); NB = number of weight
// matrices sharing the A rows (2 for gate/up, 1 for down).
template <int G, int NB>
struct GroupedTile {
    floatx16 acc[NB][2];
};

template <int G, int NB, typename RowSrc>
__device__ __forceinline__ void grouped_mainloop(GroupedTile<G, NB>& tile, uint16_t* sA,
                                                 RowSrc row_src, const uint8_t* const* wf,
                                                 const uint16_t* const* S, int N, int K,
                                                 int ncol0) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1;
    const int h = lane >> 5, c32 = lane & 31;
    const int kchunks = K / 128;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 16; ++j) tile.acc[b][t][j] = 0.f;

    // A staging: 64 rows x 256 bytes = 1024 pieces, 4 per thread
    // rows past the expert's last one repeat row 0 (unconditional loads; those
    // accumulator rows are not stored)
    const uint16_t* src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i, row = idx >> 4, col = idx & 15;
        const uint16_t* r = row_src(row);
        src[i] = (r ? r : row_src(0)) + col * 8;
    }
    uintx4 areg[4];
    auto load_a = [&](int c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) areg[i] = *reinterpret_cast<const uintx4*>(src[i] + c * 128);
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i, row = idx >> 4, col = idx & 15;
            *reinterpret_cast<uintx4*>(&sA[buf * MBM * MLDA + row * MLDA + col * 8]) = areg[i];
        }
    };

    BChunk<2, G> bcur[NB], bnext[NB];
    load_a(0);
#pragma unroll
    for (int b = 0; b < NB; ++b) load_b_chunk<2, G>(bcur[b], wf[b], S[b], N, kchunks, 0, ncol0, lane);
    store_a(0);
    __syncthreads();
    for (int c = 0; c < kchunks; ++c) {
        const int buf = c & 1;
        const bool more = c + 1 < kchunks;
        if (more) {
            load_a(c + 1);
#pragma unroll
            for (int b = 0; b < NB; ++b)
                load_b_chunk<2, G>(bnext[b], wf[b], S[b], N, kchunks, c + 1, ncol0, lane);
        }
        const uint16_t* sa = sA + buf * MBM * MLDA;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int kg = kgroup_of_step(s, h);
            const half8 a = *reinterpret_cast<const half8*>(&sa[(wm * 32 + c32) * MLDA + kg * 8]);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    tile.acc[b][t] = mfma32(a, b_frag<2, G>(bcur[b], t, s), tile.acc[b][t]);
        }
        if (more) {
            store_a(buf ^ 1);
#pragma unroll
            for (int b = 0; b < NB; ++b) bcur[b] = bnext[b];
        }
        __syncthreads();
    }
}

template <int G>
__global__ __launch_bounds__(256, 2) void moe_gateup_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
    const uint16_t* __restrict__ sg, const uint16_t* __restrict__ su, Work wk, int T, int H, int I,
    int topK, int mtiles) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2 * MBM * MLDA];
    const int e = blockIdx.y / mtiles, mt = blockIdx.y % mtiles;
    const int off = wk.offsets[e], me = wk.offsets[e + 1] - off;
    const int r0 = mt * MBM;
    if (r0 >= me) return;
    const int rows = me - r0 < MBM ? me - r0 : MBM;
    const int slot0 = off + r0;
    auto row_src = [&](int row) -> const uint16_t* {
        if (row >= rows) return nullptr;
        const int token = wk.pairs[slot0 + row] / topK;
        return X + (size_t)token * H;
    };
    const size_t wbytes = (size_t)H * I / 2;
    const size_t sn = (size_t)(H / G) * I;
    const uint8_t* wf[2] = {wg + e * wbytes, wu + e * wbytes};
    const uint16_t* S[2] = {sg + e * sn, su + e * sn};
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ncol0 = blockIdx.x * MBN + (wave & 1) * 64;
    GroupedTile<G, 2> tile;
    grouped_mainloop<G, 2>(tile, sA, row_src, wf, S, I, H, ncol0);
    const int wm = wave >> 1;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int col = ncol0 + t * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int row = wm * 32 + acc_row(j, lane);
            if (row < rows) {
                const float g = tile.acc[0][t][j], u = tile.acc[1][t][j];
                const float silu = g / (1.0f + expf(-g));
                wk.h[(size_t)(slot0 + row) * I + col] = f2h(silu * u);
            }
        }
    }
}

template <int G>
__global__ __launch_bounds__(256, 2) void moe_down_kernel(const uint8_t* __restrict__ wd,
                                                          const uint16_t* __restrict__ sd, Work wk,
                                                          int H, int I, int mtiles) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2 * MBM * MLDA];
    const int e = blockIdx.y / mtiles, mt = blockIdx.y % mtiles;
    const int off = wk.offsets[e], me = wk.offsets[e + 1] - off;
    const int r0 = mt * MBM;
    if (r0 >= me) return;
    const int rows = me - r0 < MBM ? me - r0 : MBM;
    const int slot0 = off + r0;
    const uint16_t* hb = wk.h;
    auto row_src = [&](int row) -> const uint16_t* {
        return row < rows ? hb + (size_t)(slot0 + row) * I : nullptr;
    };
    const uint8_t* wf[1] = {wd + e * ((size_t)I * H / 2)};
    const uint16_t* S[1] = {sd + e * ((size_t)(I / G) * H)};
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ncol0 = blockIdx.x * MBN + (wave & 1) * 64;
    GroupedTile<G, 1> tile;
    grouped_mainloop<G, 1>(tile, sA, row_src, wf, S, H, I, ncol0);
    const int wm = wave >> 1;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int col = ncol0 + t * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int row = wm * 32 + acc_row(j, lane);
            if (row < rows) wk.o[(size_t)(slot0 + row) * H + col] = tile.acc[0][t][j];
        }
    }
}

// ------------------------------------------------------------------ combine

__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ w, Work wk,
                                                          uint16_t* __restrict__ Y, int T, int H,
                                                          int topK) {
    const int per_row = H / 8;
    const size_t total = (size_t)T * per_row;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += stride) {
        const int t = (int)(c / per_row), c8 = (int)(c % per_row);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < topK; ++j) {
            const int p = t * topK + j;
            const float wj = w[p];
            const float* o = wk.o + (size_t)wk.slot_of[p] * H + c8 * 8;
            const floatx4 lo = *reinterpret_cast<const floatx4*>(o);
            const floatx4 hi = *reinterpret_cast<const floatx4*>(o + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[i] = __builtin_fmaf(wj, lo[i], acc[i]);
                acc[4 + i] = __builtin_fmaf(wj, hi[i], acc[4 + i]);
            }
        }
        const uintx4 out = {(uint32_t)f2h(acc[0]) | ((uint32_t)f2h(acc[1]) << 16),
                            (uint32_t)f2h(acc[2]) | ((uint32_t)f2h(acc[3]) << 16),
                            (uint32_t)f2h(acc[4]) | ((uint32_t)f2h(acc[5]) << 16),
                            (uint32_t)f2h(acc[6]) | ((uint32_t)f2h(acc[7]) << 16)};
        *reinterpret_cast<uintx4*>(Y + (size_t)t * H + c8 * 8) = out;
    }
}

template <int G>
int32_t launch_moe(const uint16_t* X, const uint16_t* logits, const uint8_t* wg, const uint8_t* wu,
                   const uint8_t* wd, const uint16_t* sg, const uint16_t* su, const uint16_t* sd,
                   uint16_t* Y, int32_t* ids, float* w, int T, int H, int I, int E, int topK,
                   const Work& wk, hipStream_t st) {
    const int P = T * topK;
    hipLaunchKernelGGL(moe_route_kernel, dim3((T + 255) / 256), dim3(256), 0, st, logits, ids, w, T,
                       E, topK);
    hipLaunchKernelGGL(moe_permute_kernel, dim3(1), dim3(1024), 0, st, ids, P, E, wk.offsets,
                       wk.pairs, wk.slot_of);
    const int mtiles = (T + MBM - 1) / MBM;  // an expert sees each token at most once
    hipLaunchKernelGGL(moe_gateup_kernel<G>, dim3(I / MBN, E * mtiles), dim3(256), 0, st, X, wg, wu,
                       sg, su, wk, T, H, I, topK, mtiles);
    hipLaunchKernelGGL(moe_down_kernel<G>, dim3(H / MBN, E * mtiles), dim3(256), 0, st, wd, sd, wk,
                       H, I, mtiles);
    const size_t chunks = (size_t)T * H / 8;
    const size_t want = (chunks + 255) / 256;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((int)(want < 4096 ? want : 4096)), dim3(256), 0, st,
                       w, wk, Y, T, H, topK);
    return qgh::launch_status();
}

}  // namespace

extern "C" size_t moe_w4a16_workspace_bytes(int32_t T, int32_t H, int32_t I, int32_t E,
                                            int32_t topK) {
    if (T < 0 || H < 0 || I < 0 || E <= 0 || topK <= 0) return 0;
    size_t off[6];
    workspace_layout(T, H, I, E, topK, off);
    return off[5];
}

extern "C" int32_t moe_w4a16(const uint16_t* X, const uint16_t* logits, const uint8_t* w_gate_frag,
                             const uint8_t* w_up_frag, const uint8_t* w_down_frag,
                             const uint16_t* s_gate, const uint16_t* s_up, const uint16_t* s_down,
                             uint16_t* Y, int32_t* topk_ids, float* topk_w, int32_t T, int32_t H,
                             int32_t I, int32_t E, int32_t topK, int32_t G, int32_t activation,
                             void* workspace, size_t workspace_bytes, void* stream) {
    if (T < 0 || H < 0 || I < 0 || E <= 0 || topK <= 0 || topK > E || G <= 0) return QGEMM_BAD_SHAPE;
    if (H % G != 0 || I % G != 0) return QGEMM_BAD_SHAPE;
    if (T == 0) return QGEMM_OK;
    if (!X || !logits || !w_gate_frag || !w_up_frag || !w_down_frag || !s_gate || !s_up || !s_down ||
        !Y || !topk_ids || !topk_w || !workspace)
        return QGEMM_NULL_PTR;
    if (activation != 0 || E > 64 || H == 0 || I == 0 || H % 128 != 0 || I % 128 != 0 ||
        (G != 32 && G != 64 && G != 128) || (size_t)T * topK > (size_t)1 << 30)
        return QGEMM_UNSUPPORTED;
    if (!qgh::aligned(X, 16) || !qgh::aligned(logits, 2) || !qgh::aligned(w_gate_frag, 16) ||
        !qgh::aligned(w_up_frag, 16) || !qgh::aligned(w_down_frag, 16) || !qgh::aligned(s_gate, 4) ||
        !qgh::aligned(s_up, 4) || !qgh::aligned(s_down, 4) || !qgh::aligned(Y, 16) ||
        !qgh::aligned(topk_ids, 4) || !qgh::aligned(topk_w, 4) || !qgh::aligned(workspace, 256))
        return QGEMM_MISALIGNED;
    size_t off[6];
    workspace_layout(T, H, I, E, topK, off);
    if (workspace_bytes < off[5]) return QGEMM_WORKSPACE_TOO_SMALL;
    char* base = static_cast<char*>(workspace);
    Work wk;
    wk.offsets = reinterpret_cast<int32_t*>(base + off[0]);
    wk.pairs = reinterpret_cast<int32_t*>(base + off[1]);
    wk.slot_of = reinterpret_cast<int32_t*>(base + off[2]);
    wk.h = reinterpret_cast<uint16_t*>(base + off[3]);
    wk.o = reinterpret_cast<float*>(base + off[4]);
    hipStream_t st = (hipStream_t)stream;
    switch (G) {
        case 32:
            return launch_moe<32>(X, logits, w_gate_frag, w_up_frag, w_down_frag, s_gate, s_up,
                                  s_down, Y, topk_ids, topk_w, T, H, I, E, topK, wk, st);
        case 64:
            return launch_moe<64>(X, logits, w_gate_frag, w_up_frag, w_down_frag, s_gate, s_up,
                                  s_down, Y, topk_ids, topk_w, T, H, I, E, topK, wk, st);
        default:
            return launch_moe<128>(X, logits, w_gate_frag, w_up_frag, w_down_frag, s_gate, s_up,
                                   s_down, Y, topk_ids, topk_w, T, H, I, E, topK, wk, st);
    }
}
