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
//   4. down:    per expert, W4A16 MFMA GEMM of h with the down matrix, K
//               split over workgroups, fp32 partial results per slot;
//   5. combine: y[t] = fp16(sum_j w[t][j] * o[slot(t, j)]), j ascending,
//               o being the K-split partials added in split order.
// Every reduction has a fixed order, so the layer is deterministic.
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

// Workgroup L: expert L % E, then column tile, then K split.
template <int G, int MODE>
__global__ __launch_bounds__(256, 2) void moe_expert_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ w0, const uint8_t* __restrict__ w1,
    const uint16_t* __restrict__ s0, const uint16_t* __restrict__ s1, Work wk, int T, int H, int I,
    int E, int topK, int splits) {
    constexpr int NB = MODE == 0 ? 2 : 1;
    __shared__ __attribute__((aligned(1024))) uint16_t sA[2 * XP_SLAB];
    const int L = blockIdx.x;
    const int e = L % E, rest = L / E;
    const int N = MODE == 0 ? I : H, K = MODE == 0 ? H : I;
    const int ntiles = N / 128;
    const int ct = rest % ntiles, ks = rest / ntiles;
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
        // element offset of A row r of this pass (rows < 2^31 / H elements)
        auto row_off = [&](int r) -> uint32_t {
            if constexpr (MODE == 0) return (uint32_t)(wk.pairs[slot0 + r] / topK) * (uint32_t)H;
            else return (uint32_t)(slot0 + r) * (uint32_t)I;
        };
        switch ((R + 31) / 32) {
            case 1: expert_pass<G, NB, 1, MODE, 4>(sA, abase, row_off, R, wf, S, N, N, kchunks, c0, c1, ncol0, slot0, out); break;
            case 2: expert_pass<G, NB, 2, MODE, 4>(sA, abase, row_off, R, wf, S, N, N, kchunks, c0, c1, ncol0, slot0, out); break;
            case 3: expert_pass<G, NB, 3, MODE, 4>(sA, abase, row_off, R, wf, S, N, N, kchunks, c0, c1, ncol0, slot0, out); break;
            default:
                if constexpr (PASS == 128)
                    expert_pass<G, NB, 4, MODE, 4>(sA, abase, row_off, R, wf, S, N, N, kchunks, c0, c1, ncol0, slot0, out);
                break;
        }
        __syncthreads();  // the next pass refills both LDS buffers
    }
}

// ------------------------------------------------------------------ combine

// y[t] = fp16(sum_j w[t][j] * o[slot(t, j)]), j ascending; o = the K-split
// partials added in split order.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ w, Work wk,
                                                          uint16_t* __restrict__ Y, int T, int H,
                                                          int topK, int splits) {
    const int per_row = H / 8;
    const size_t total = (size_t)T * per_row;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t split_stride = (size_t)T * topK * H;
    for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += stride) {
        const int t = (int)(c / per_row), c8 = (int)(c % per_row);
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
                   const Work& wk, hipStream_t st) {
    const int P = T * topK;
    hipLaunchKernelGGL(moe_route_kernel, dim3((T + 255) / 256), dim3(256), 0, st, logits, ids, w, T,
                       E, topK);
    hipLaunchKernelGGL(moe_permute_kernel, dim3(1), dim3(1024), 0, st, ids, P, E, wk.offsets,
                       wk.pairs, wk.slot_of);
    const int splits = down_splits(H, I, E);
    hipLaunchKernelGGL((moe_expert_kernel<G, 0>), dim3(E * (I / 128)), dim3(256), 0, st, X, wg, wu,
                       sg, su, wk, T, H, I, E, topK, 1);
    hipLaunchKernelGGL((moe_expert_kernel<G, 1>), dim3(E * (H / 128) * splits), dim3(256), 0, st, X,
                       wd, wd, sd, sd, wk, T, H, I, E, topK, splits);
    const size_t chunks = (size_t)T * H / 8;
    const size_t want = (chunks + 255) / 256;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((int)(want < 4096 ? want : 4096)), dim3(256), 0, st,
                       w, wk, Y, T, H, topK, splits);
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
        (G != 32 && G != 64 && G != 128) || (size_t)T * topK > (size_t)1 << 30 ||
        (size_t)T * H >= (size_t)1 << 31 || (size_t)T * topK * I >= (size_t)1 << 31)
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
