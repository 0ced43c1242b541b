// INT4 mixture-of-experts layer (Int4 Moe Plugin page, constructor:
// numExperts, topK, hiddenSize, moeInterSize, activationType,
// quantizationGroupSize; one output).  Four stream-ordered launches:
//   1. route + permute, one workgroup: per token, top-k experts by logit
//               (lower index wins ties) and softmax over the selected logits
//               (fp32); then the (token, j) pairs grouped by expert, keeping
//               ascending pair order inside an expert (wave ballots, no
//               atomics on the result order), and each pair's slot recorded;
//   2. gate/up: per expert, a W4A16 MFMA GEMM over that expert's gathered
//               token rows with both the gate and the up matrix, fused with
//               h = fp16(act(g) * u) (act: the constructor's activation
//               type, SiLU by default);
//   3. down:    per expert, W4A16 MFMA GEMM of h with the down matrix, K
//               split over workgroups, fp32 partial results per slot;
//   4. combine: y[t] = fp16(sum_j w[t][j] * o[slot(t, j)]), j ascending,
//               o being the K-split partials added in split order.
// Every reduction has a fixed order, so the layer is deterministic.
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "wq_pass.hpp"

namespace {

using namespace qg;

struct Work {
    int32_t* offsets;
    int32_t* pairs;
    int32_t* slot_of;
    uint16_t* h;
    float* o;
};

// K splits of the down projection: double until the workgroups cover the
// chip about twice (two per CU are resident), keeping whole 128-k chunks per
// split.  At H = 4096, E = 8 that is two splits: on one box the layer took
// 268.3 us against 273.8 with four (more partials for the combine to read),
// on another 253.5 us against 271 with one.
__host__ __device__ inline int down_splits(int H, int I, int E) {
    const int tiles = E * (H / 128), kc = I / 128;
    int ks = 1;
    while (ks < 8 && tiles * ks < 512 && kc % (2 * ks) == 0) ks *= 2;
    return ks;
}

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
    x = (x + sizeof(float) * down_splits(H, I, E) * P * H + 255) & ~(size_t)255;
    off[5] = x;
}

// ------------------------------------------------------------------ route + permute

// One workgroup.  Route: thread t takes tokens t, t + 1024, ...; per token
// the top-k experts by logit (lower index wins ties) and the softmax over the
// selected logits (fp32).  With eight experts (and 16-byte aligned logit
// rows, topK <= 8) a token's logits arrive in one 16-byte load and the
// selection runs on registers (arrays indexed by unrolled constants only);
// otherwise each logit is read from memory as it is compared and the
// selected logits wait in the output weights until the sum is known (no
// per-thread arrays, so no scratch memory either way).  The expert ids also
// go to LDS when the pairs fit (P <= MOE_LDS_PAIRS), so the permute below
// reads them from there rather than back from global memory.
// Permute: groups the (token, j) pairs by expert, keeping ascending pair
// order inside an expert (wave ballots, no atomics on the result order), and
// records each pair's slot.  One launch for both: the routing of a few
// hundred tokens is far below a launch's cost.
constexpr int MOE_LDS_PAIRS = 8192;

__global__ __launch_bounds__(1024) void moe_route_permute_kernel(const uint16_t* __restrict__ logits,
                                                                 int32_t* __restrict__ ids,
                                                                 float* __restrict__ w, int T, int E,
                                                                 int topK, int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ pairs,
                                                                 int32_t* __restrict__ slot_of) {
    __shared__ int sid[MOE_LDS_PAIRS];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int P = T * topK;
    const bool in_lds = P <= MOE_LDS_PAIRS;
    if (E == 8 && topK <= 8 && ((uintptr_t)logits & 15) == 0) {
        for (int t = tid; t < T; t += 1024) {
            const uintx4 raw = *reinterpret_cast<const uintx4*>(logits + (size_t)t * 8);
            float lv[8], vals[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lv[2 * i] = h2f((uint16_t)(raw[i] & 0xffffu));
                lv[2 * i + 1] = h2f((uint16_t)(raw[i] >> 16));
            }
            uint32_t taken = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j >= topK) break;
                int best = -1;
                float bv = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if ((taken >> e) & 1u) continue;
                    if (best < 0 || lv[e] > bv) {
                        best = e;
                        bv = lv[e];
                    }
                }
                taken |= 1u << best;
                ids[(size_t)t * topK + j] = best;
                if (in_lds) sid[t * topK + j] = best;
                vals[j] = bv;
            }
            const float lmax = vals[0];
            float sum = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j >= topK) break;
                vals[j] = expf(vals[j] - lmax);
                sum += vals[j];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j >= topK) break;
                w[(size_t)t * topK + j] = vals[j] / sum;
            }
        }
    } else {
        for (int t = tid; t < T; t += 1024) {
            const uint16_t* l = logits + (size_t)t * E;
            int32_t* it = ids + (size_t)t * topK;
            float* wt = w + (size_t)t * topK;
            uint64_t taken = 0;
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
                it[j] = best;
                if (in_lds) sid[t * topK + j] = best;
                wt[j] = bv;
            }
            const float lmax = wt[0];
            float sum = 0.0f;
            for (int j = 0; j < topK; ++j) {
                const float v = expf(wt[j] - lmax);
                wt[j] = v;
                sum += v;
            }
            for (int j = 0; j < topK; ++j) wt[j] = wt[j] / sum;
        }
    }
    __syncthreads();  // the expert ids written above are read by every thread below

    __shared__ int cnt[64];
    __shared__ int base[64];
    __shared__ int wave_cnt[16][64];
    __shared__ int wave_off[16][64];
    if (tid < 64) cnt[tid] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += 1024) atomicAdd(&cnt[in_lds ? sid[p] : ids[p]], 1);
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
        const int e = p < P ? (in_lds ? sid[p] : ids[p]) : -1;
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

// One kernel for both projections.  A workgroup owns one expert and one
// 128-column tile of its weight matrices (NB = 2: gate and up, which share
// the A rows; NB = 1: down) and runs every row of that expert through it, in
// passes of up to 128 rows, so each weight byte is read from HBM once per
// pass (one pass unless an expert holds more than 96 rows for gate/up, 128
// for down: the gate/up pass keeps 2 x 3 accumulator tiles in registers).  Wave w owns
// columns 32w .. 32w + 31 of the tile for all rows: it dequantizes its B
// fragments once per k-step and feeds them to the NRB 32-row MFMA blocks.
// A rows (gathered tokens for gate/up, contiguous h rows for down) go
// buffer -> LDS by DMA, double-buffered, with the XOR swizzle of the prefill
// kernel; B fragments are prefetched one 128-k chunk ahead in registers.
// The down projection splits K over KS workgroups (fp32 partials, added in
// split order by the combine) so that it has enough workgroups.

// Workgroup L: expert L % E, then column tile, then K split.  Workgroups are
// dealt to the eight XCDs by id, so with eight experts each XCD runs one
// expert and keeps that expert's gathered A rows in its L2 (every workgroup
// re-reads them per chunk).  Ordering the ids by expert instead (the experts
// with the most rows first) measured 328 against 282 us for the layer with
// 256 tokens, hidden 4096, intermediate 14336, top-2 of 8: A then misses in
// every XCD's L2.  The gate/up pass with eight experts pairs them instead
// (below), two experts per XCD.
template <int G, int MODE>
__global__ __launch_bounds__(256, 2) void moe_expert_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ w0, const uint8_t* __restrict__ w1,
    const uint16_t* __restrict__ s0, const uint16_t* __restrict__ s1, Work wk, int T, int H, int I,
    int E, int topK, int splits, int act) {
    constexpr int NB = MODE == 0 ? 2 : 1;
    __shared__ __attribute__((aligned(1024))) uint16_t sA[2 * XP_SLAB];
    const int L = blockIdx.x;
    const int N = MODE == 0 ? I : H, K = MODE == 0 ? H : I;
    const int ntiles = N / 128;
    int e = L % E, ct = (L / E) % ntiles;
    const int ks = (L / E) / ntiles;
    if (MODE == 0 && E == 8 && ntiles % 2 == 0) {
        // Balanced pairs: rank the experts by 32-row MFMA blocks (most first,
        // lower index on ties) and give XCDs 2p and 2p + 1 the experts ranked
        // p and 7 - p, one half of the column tiles of each, the heavier
        // expert's tiles first in dispatch order.  So every XCD carries half
        // of a heavy and half of a light expert instead of one whole expert
        // (the layer's time is that of its slowest XCD) and still reads the A
        // rows of only two experts.  Every (expert, tile) is still one
        // workgroup; results do not depend on the mapping.
        const int x = L % 8, i = L / 8, half = ntiles / 2;
        const int p = x >> 1, want = i < half ? p : 7 - p;
        int nb[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) nb[q] = (wk.offsets[q + 1] - wk.offsets[q] + 31) >> 5;
        e = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            int rank = 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) rank += (nb[u] > nb[q]) || (nb[u] == nb[q] && u < q);
            if (rank == want) e = q;
        }
        ct = (x & 1) * half + (i < half ? i : i - half);
    }
    const int off = wk.offsets[e], me = wk.offsets[e + 1] - off;
    if (me == 0) return;
    const int kchunks = K / 128, per = kchunks / splits;
    const int c0 = ks * per, c1 = c0 + per;
    const size_t wbytes = (size_t)K * N / 2, sn = (size_t)(K / G) * N;
    const uint8_t* wf[NB];
    const uint16_t* S[NB];
    wf[0] = w0 + e * wbytes;
    S[0] = s0 + e * sn;
    if constexpr (NB == 2) {
        wf[1] = w1 + e * wbytes;
        S[1] = s1 + e * sn;
    }
    const int ncol0 = ct * 128 + (threadIdx.x >> 6) * 32;
    void* out = MODE == 0 ? static_cast<void*>(wk.h)
                          : static_cast<void*>(wk.o + (size_t)ks * T * topK * H);
    constexpr int PASS = MODE == 0 ? 96 : 128;  // rows per pass
    const uint16_t* abase = MODE == 0 ? X : wk.h;
    for (int r0 = 0; r0 < me; r0 += PASS) {
        const int R = me - r0 < PASS ? me - r0 : PASS;
        const int slot0 = off + r0;
        // A row r of this pass: its pair index (gate/up, gathered tokens) or
        // its slot (down), and from that its element offset (rows < 2^31 / H
        // elements)
        auto row_key = [&](int r) -> uint32_t {
            if constexpr (MODE == 0) return (uint32_t)wk.pairs[slot0 + r];
            else return (uint32_t)(slot0 + r);
        };
        auto key_off = [&](uint32_t k) -> uint32_t {
            if constexpr (MODE == 0) return (k / (uint32_t)topK) * (uint32_t)H;
            else return k * (uint32_t)I;
        };
        switch ((R + 31) / 32) {
            case 1: expert_pass<G, NB, 1, MODE, 4>(sA, abase, row_key, key_off, R, wf, S, N, N, kchunks, c0, c1, ncol0, slot0, out, act); break;
            case 2: expert_pass<G, NB, 2, MODE, 4>(sA, abase, row_key, key_off, R, wf, S, N, N, kchunks, c0, c1, ncol0, slot0, out, act); break;
            case 3: expert_pass<G, NB, 3, MODE, 4>(sA, abase, row_key, key_off, R, wf, S, N, N, kchunks, c0, c1, ncol0, slot0, out, act); break;
            default:
                if constexpr (PASS == 128)
                    expert_pass<G, NB, 4, MODE, 4>(sA, abase, row_key, key_off, R, wf, S, N, N, kchunks, c0, c1, ncol0, slot0, out, act);
                break;
        }
        __syncthreads();  // the next pass refills both LDS buffers
    }
}

// ------------------------------------------------------------------ combine

// y[t] = fp16(sum_j w[t][j] * o[slot(t, j)]), j ascending; o = the K-split
// partials added in split order.
// IDX: the chunk index type (32 bits whenever the indexes fit); row_shift >=
// 0: H / 8 = 1 << row_shift, and the token of a chunk is a shift (the first
// loads of a chunk wait for that index: a 64-bit division there sat on the
// critical path).
template <typename IDX>
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ w, Work wk,
                                                          uint16_t* __restrict__ Y, int T, int H,
                                                          int topK, int splits, int row_shift) {
    const int per_row = H / 8;
    const IDX total = (IDX)T * per_row;
    const IDX stride = (IDX)gridDim.x * blockDim.x;
    const size_t split_stride = (size_t)T * topK * H;
    for (IDX c = (IDX)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += stride) {
        const int t = (int)(row_shift >= 0 ? c >> row_shift : c / (IDX)per_row);
        const int c8 = (int)(c - (IDX)t * per_row);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < topK; ++j) {
            const int p = t * topK + j;
            const float wj = w[p];
            const float* o = wk.o + (size_t)wk.slot_of[p] * H + c8 * 8;
            floatx4 lo = *reinterpret_cast<const floatx4*>(o);
            floatx4 hi = *reinterpret_cast<const floatx4*>(o + 4);
            for (int k = 1; k < splits; ++k) {
                lo += *reinterpret_cast<const floatx4*>(o + k * split_stride);
                hi += *reinterpret_cast<const floatx4*>(o + k * split_stride + 4);
            }
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
                   int act, const Work& wk, hipStream_t st) {
    hipLaunchKernelGGL(moe_route_permute_kernel, dim3(1), dim3(1024), 0, st, logits, ids, w, T, E, topK,
                       wk.offsets, wk.pairs, wk.slot_of);
    const int splits = down_splits(H, I, E);
    hipLaunchKernelGGL((moe_expert_kernel<G, 0>), dim3(E * (I / 128)), dim3(256), 0, st, X, wg, wu,
                       sg, su, wk, T, H, I, E, topK, 1, act);
    hipLaunchKernelGGL((moe_expert_kernel<G, 1>), dim3(E * (H / 128) * splits), dim3(256), 0, st, X,
                       wd, wd, sd, sd, wk, T, H, I, E, topK, splits, 0);
    const size_t chunks = (size_t)T * H / 8;
    const size_t want = (chunks + 255) / 256;
    const int cblocks = (int)(want < 4096 ? want : 4096), per_row = H / 8;
    const int shift = (per_row & (per_row - 1)) == 0 ? __builtin_ctz((unsigned)per_row) : -1;
    if (chunks + (size_t)cblocks * 256 < ((size_t)1 << 32))
        hipLaunchKernelGGL(moe_combine_kernel<uint32_t>, dim3(cblocks), dim3(256), 0, st, w, wk, Y, T, H, topK,
                           splits, shift);
    else
        hipLaunchKernelGGL(moe_combine_kernel<size_t>, dim3(cblocks), dim3(256), 0, st, w, wk, Y, T, H, topK,
                           splits, shift);
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

// Validation and launch shared by both entry points (workspace given by the
// caller, or this file's scratch array).
static int32_t moe_run(const uint16_t* X, const uint16_t* logits, const uint8_t* w_gate_frag,
                       const uint8_t* w_up_frag, const uint8_t* w_down_frag, const uint16_t* s_gate,
                       const uint16_t* s_up, const uint16_t* s_down, uint16_t* Y, int32_t* topk_ids,
                       float* topk_w, int32_t T, int32_t H, int32_t I, int32_t E, int32_t topK,
                       int32_t G, int32_t activation, void* workspace, size_t workspace_bytes,
                       void* stream) {
    if (!workspace) return QGEMM_NULL_PTR;
    if (!qgh::aligned(workspace, 256)) return QGEMM_MISALIGNED;
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
                                  s_down, Y, topk_ids, topk_w, T, H, I, E, topK, activation, wk, st);
        case 64:
            return launch_moe<64>(X, logits, w_gate_frag, w_up_frag, w_down_frag, s_gate, s_up,
                                  s_down, Y, topk_ids, topk_w, T, H, I, E, topK, activation, wk, st);
        default:
            return launch_moe<128>(X, logits, w_gate_frag, w_up_frag, w_down_frag, s_gate, s_up,
                                   s_down, Y, topk_ids, topk_w, T, H, I, E, topK, activation, wk, st);
    }
}

// Argument checks common to both entry points, except the workspace.
static int32_t moe_check(const uint16_t* X, const uint16_t* logits, const uint8_t* w_gate_frag,
                         const uint8_t* w_up_frag, const uint8_t* w_down_frag,
                         const uint16_t* s_gate, const uint16_t* s_up, const uint16_t* s_down,
                         const uint16_t* Y, const int32_t* topk_ids, const float* topk_w, int32_t T,
                         int32_t H, int32_t I, int32_t E, int32_t topK, int32_t G,
                         int32_t activation) {
    if (!X || !logits || !w_gate_frag || !w_up_frag || !w_down_frag || !s_gate || !s_up || !s_down ||
        !Y || !topk_ids || !topk_w)
        return QGEMM_NULL_PTR;
    if (activation < QGEMM_MOE_ACT_SILU || activation > QGEMM_MOE_ACT_RELU || E > 64 || H == 0 || I == 0 ||
        H % 128 != 0 || I % 128 != 0 ||
        (G != 32 && G != 64 && G != 128) || (size_t)T * topK > (size_t)1 << 30 ||
        (size_t)T * H >= (size_t)1 << 31 || (size_t)T * topK * I >= (size_t)1 << 31)
        return QGEMM_UNSUPPORTED;
    if (!qgh::aligned(X, 16) || !qgh::aligned(logits, 2) || !qgh::aligned(w_gate_frag, 16) ||
        !qgh::aligned(w_up_frag, 16) || !qgh::aligned(w_down_frag, 16) || !qgh::aligned(s_gate, 4) ||
        !qgh::aligned(s_up, 4) || !qgh::aligned(s_down, 4) || !qgh::aligned(Y, 16) ||
        !qgh::aligned(topk_ids, 4) || !qgh::aligned(topk_w, 4))
        return QGEMM_MISALIGNED;
    return QGEMM_OK;
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
    const int32_t c = moe_check(X, logits, w_gate_frag, w_up_frag, w_down_frag, s_gate, s_up, s_down,
                                Y, topk_ids, topk_w, T, H, I, E, topK, G, activation);
    if (c != QGEMM_OK) return c;
    return moe_run(X, logits, w_gate_frag, w_up_frag, w_down_frag, s_gate, s_up, s_down, Y,
                   topk_ids, topk_w, T, H, I, E, topK, G, activation, workspace, workspace_bytes,
                   stream);
}

// ------------------------------------------------------------------ no-allocation variant

// Workspace of moe_w4a16_no_alloc: one array per GPU, created with the code
// object when the library is first used on that GPU and held until the
// process ends.  Host code never passes `scratch` itself (in host code it
// names a host-side shadow, not device memory): it looks up the device
// address once per GPU and passes that.
static __device__ __align__(256) unsigned char scratch[QGEMM_MOE_NO_ALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up on the first
// call on each device, with that device current).
int32_t scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return QGEMM_HIP_ERROR;
    }
    if (dev < 0 || dev >= kMaxDevices) return QGEMM_UNSUPPORTED;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
                (void)hipGetLastError();
                return QGEMM_HIP_ERROR;
            }
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return QGEMM_OK;
}

}  // namespace

extern "C" int32_t moe_w4a16_no_alloc(const uint16_t* X, const uint16_t* logits,
                                      const uint8_t* w_gate_frag, const uint8_t* w_up_frag,
                                      const uint8_t* w_down_frag, const uint16_t* s_gate,
                                      const uint16_t* s_up, const uint16_t* s_down, uint16_t* Y,
                                      int32_t* topk_ids, float* topk_w, int32_t T, int32_t H,
                                      int32_t I, int32_t E, int32_t topK, int32_t G,
                                      int32_t activation, void* stream) {
    if (T < 0 || H < 0 || I < 0 || E <= 0 || topK <= 0 || topK > E || G <= 0) return QGEMM_BAD_SHAPE;
    if (H % G != 0 || I % G != 0) return QGEMM_BAD_SHAPE;
    if (T == 0) return QGEMM_OK;
    const int32_t c = moe_check(X, logits, w_gate_frag, w_up_frag, w_down_frag, s_gate, s_up, s_down,
                                Y, topk_ids, topk_w, T, H, I, E, topK, G, activation);
    if (c != QGEMM_OK) return c;
    size_t off[6];
    workspace_layout(T, H, I, E, topK, off);
    if (off[5] > QGEMM_MOE_NO_ALLOC_SCRATCH_BYTES) return QGEMM_WORKSPACE_TOO_SMALL;
    if (stream) {
        int cur = -1, sdev = -1;
        if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) {
            (void)hipGetLastError();
            return QGEMM_HIP_ERROR;
        }
        if (cur != sdev) return QGEMM_UNSUPPORTED;
    }
    void* ws = nullptr;
    const int32_t s = scratch_address(&ws);
    if (s != QGEMM_OK) return s;
    return moe_run(X, logits, w_gate_frag, w_up_frag, w_down_frag, s_gate, s_up, s_down, Y,
                   topk_ids, topk_w, T, H, I, E, topK, G, activation, ws,
                   QGEMM_MOE_NO_ALLOC_SCRATCH_BYTES, stream);
}
