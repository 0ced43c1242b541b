// Weight-only GEMM kernels shared by the int4 (W4A16) and int8 (W8A16)
// entry points: Y[M,N] = A[M,K] (fp16) x (q * s), q the WB-bit weights of a
// fragment layout (wq_tile.hpp), s fp16 scales, fp32 accumulation, fp16
// output.  Three regimes, chosen by M:
//   decode  (M <= 16): HBM-bound weight stream.  Each wave owns up to NSW
//       16-column strips and KCW 128-k chunks; it issues every weight, A and
//       scale load of its slice before its first wait, stages A and scales in
//       its own LDS slice (no workgroup barrier before the main loop) and runs
//       v_mfma_f32_16x16x32_f16 on the raw fp16 values 1024 + u; per-group
//       fp32 partials are corrected and scaled, and the K partials of the
//       workgroup's waves are added in LDS in a fixed order.
//   mid (16 < M <= 128, with a workspace): split-K.  A workgroup owns 128
//       columns and a K range and runs all M rows through them (the
//       B-stationary pass of the MoE GEMMs), writing fp32 partials; a second
//       launch adds the splits in a fixed order and rounds to fp16.  A single
//       pass over K with 128-column tiles would leave most CUs idle (86
//       workgroups for N = 11008).
//   prefill (other M > 16): 128x128 output tiles, four waves of 64x64, A
//       tiles double-buffered through LDS via registers, B fragments read
//       straight from the fragment layout into registers and dequantized with
//       the group scale folded in, v_mfma_f32_32x32x16_f16.  The workgroup
//       index runs column-major over tiles, so the workgroups resident on one
//       XCD share weight columns in its L2.
// Scales: row (k / G) of S at element offset (k / G) * ldS; ldS = 0 gives
// every group row 0, i.e. one scale per column.
#pragma once

#include "wq_pass.hpp"

namespace {

using namespace qg;

// ------------------------------------------------------------------ decode

__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// v plus the value of lane l' of the same 16-lane row, l' given by a DPP
// control (quad permutation or row mirror).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                     0xf, 0xf, false));
}

// Sum of v over each aligned group of N adjacent lanes (N = 4, 8 or 16),
// delivered to every lane of the group: lane ^ 1 and lane ^ 2 (quad
// permutations) give quad sums, the half-row mirror (lane 7 - i within 8)
// adds the other quad and the row mirror (lane 15 - i within 16) the other
// half.  Register moves only, no LDS round trips.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
    v = dpp_add<0xB1>(v);                          // quad_perm [1, 0, 3, 2]
    v = dpp_add<0x4E>(v);                          // quad_perm [2, 3, 0, 1]
    if constexpr (N >= 8) v = dpp_add<0x141>(v);   // row_half_mirror
    if constexpr (N >= 16) v = dpp_add<0x140>(v);  // row_mirror
    return v;
}

// Decode kernel for WB-bit weights.  MT = rows of the MFMA A tile that may be
// non-zero (M <= MT <= 16); each wave owns up to NSW 16-column strips and KCW
// 128-k chunks (NSW * KCW * P 16-byte weight loads per lane, P = 1 for int4
// and 2 for int8); WK = 32 / KCW waves cover
// 4096 k, so a workgroup of WK waves holds its strips over a whole 4096-k
// block and reduces its K partials in LDS in a fixed order.  With BAL the
// grid is sized to the chip and each workgroup takes a contiguous range of
// strips (NSW at most).
//
// Everything a wave needs is staged by that wave alone, in its own slice of
// LDS, so there is no barrier before the main loop: it issues the loads of
// its A slice (rows < M), of its group scales and then all eight weight
// loads; while the weights stream in it writes A and the scales to LDS and
// forms the per-(row, group) constant C = sum_k bias_k * a_k (bias_k = raw
// value - weight at k: 1032 or 72 by position for int4, 1152 for int8).  The
// MFMAs work on the raw fp16 values (five VALU ops per eight int4 weights,
// four per eight int8 weights); each group's fp32 partial T becomes
// acc += s * (T - C).  One A fragment read from
// LDS feeds the MFMAs of all NSW strips.
// Workgroups of a decode launch over N columns: one per 16-column strip, or
// (balanced) at least one per CU where there are enough strips, each over a
// contiguous range of at most three strips.  The kernel derives its grid size
// from N with this same function instead of reading gridDim, whose value sits
// in the hidden kernel arguments: that load, the only one left once the
// explicit arguments are preloaded into scalar registers, would delay every
// wave's first weight load by a memory round trip.
__host__ __device__ inline int decode_grid(int N, bool bal) {
    const int nstrips = (N + 15) / 16;
    if (!bal) return nstrips;
    const int nwg = nstrips < 256 ? nstrips : 256;
    return nwg < (nstrips + 2) / 3 ? (nstrips + 2) / 3 : nwg;
}

template <int WB, int MT, int NSW, int KCW, int G, bool BAL>
__global__ __launch_bounds__(64 * (32 / KCW)) void wq_decode_kernel(
    const uint16_t* __restrict__ A, const uint8_t* __restrict__ wf, const uint16_t* __restrict__ Sc,
    int ldS, uint16_t* __restrict__ Y, int M, int N, int K) {
    constexpr int P = WFormat<WB>::kPieces;
    constexpr float B0 = WFormat<WB>::kBias0, B1 = WFormat<WB>::kBias1;
    constexpr int WK = 32 / KCW;                 // waves per workgroup (one 4096-k block)
    constexpr int KW = KCW * 128;                // k per wave
    constexpr int LDA = KW + 8;                  // halfs per staged A row (+16 B pad)
    constexpr int APIECES = MT * KW / 8;         // 16-byte A pieces per wave
    constexpr int APL = APIECES < 64 ? 1 : APIECES / 64;  // per lane
    constexpr int NG = 128 / G, KKPG = G / 32;   // groups per chunk, k-steps per group
    constexpr int GW = KCW * NG;                 // groups per wave
    constexpr int GP = G / 8;                    // A pieces per group and row
    constexpr int SPL = GW * NSW * 2;            // 16-byte scale pieces per wave (<= 64)
    static_assert(APIECES < 64 || APL * 64 == APIECES, "A staging must tile the wave's slice");
    static_assert(SPL <= 64, "one scale piece per lane");
    // C = sum_k bias_k a_k per (row, group): by VALU during staging, except
    // for 16-row tiles over several strips, where an extra MFMA per k-step
    // against a constant bias operand (shared by the strips) is cheaper than
    // sixteen rows of sums and shuffles (measured: M = 16 8.8 us instead of
    // 9.6; for M <= 8 the VALU sums are faster)
    constexpr bool CM = NSW >= 2 && MT >= 16;
    struct WaveLds {
        _Float16 a[MT * LDA];
        float c[GW][16];
        uint16_t s[GW][NSW * 16];
    };
    constexpr size_t RED = sizeof(floatx4) * WK * NSW * 64;  // K-partials for the reduction
    constexpr size_t STAGE = sizeof(WaveLds) * WK;
    // The partials get LDS of their own when both fit in 128 KB (then a wave
    // writes its partials as soon as its loop ends, with no barrier before;
    // the 16-wave shapes run one workgroup per CU whatever their LDS size);
    // otherwise they reuse the staging area once every wave is done with it.
    constexpr bool OWN_RED = STAGE + RED <= 128 * 1024;
    constexpr size_t LDS_BYTES = OWN_RED ? STAGE + RED : (STAGE > RED ? STAGE : RED);
    __shared__ __attribute__((aligned(16))) char lds_raw[LDS_BYTES];
    WaveLds* lds = reinterpret_cast<WaveLds*>(lds_raw);

    // (the wave index as a scalar: the slice bounds and their branches are uniform)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    WaveLds& L = lds[wave];
    // BAL: the workgroups share the N / 16 strips in contiguous ranges of
    // NSW - 1 or NSW strips (every CU busy when N / 16 is not a multiple of
    // NSW x 256); a slot past the range repeats its last strip and is not stored
    int strip0, nst;
    const int nwg = decode_grid(N, BAL);
    if constexpr (BAL) {
        const int wg = xcd_contiguous(blockIdx.x, nwg), nstrips = (N + 15) / 16;
        strip0 = (int)((long)wg * nstrips / nwg);
        nst = (int)((long)(wg + 1) * nstrips / nwg) - strip0;
    } else {
        strip0 = xcd_contiguous(blockIdx.x, nwg) * NSW;
        nst = NSW;
    }
    const int cl = lane & 15, q = lane >> 4;
    const int kchunks = (K + 127) / 128;  // of the (padded) fragment layout
    const int arow = cl & (MT - 1);  // rows >= MT of the MFMA tile are never stored
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    floatx4 acc[NSW];
#pragma unroll
    for (int s = 0; s < NSW; ++s) acc[s] = zero;

    for (int kb0 = 0; kb0 < K; kb0 += 4096) {
        const int kw0 = kb0 + wave * KW;             // first k of this wave
        const int kwl = K - kw0 < KW ? K - kw0 : KW;  // k of this wave in this block (may be <= 0)
        // Loads, in the order they are needed: A, scales, weights.  Every load
        // is unconditional (out-of-range requests are clamped to valid data
        // that is never used): a load under a branch makes the compiler wait
        // for all outstanding loads at the join, which would serialize the
        // weight stream behind the staging.  Rows >= M repeat row M-1; they
        // only feed accumulator rows that are never stored.
        uintx4 ast[APL];
#pragma unroll
        for (int p = 0; p < APL; ++p) {
            const int idx = lane + 64 * p;
            const int row = idx / (KW / 8) < M ? idx / (KW / 8) : M - 1;
            const int c8 = (idx < APIECES && (idx % (KW / 8)) * 8 < kwl) ? idx % (KW / 8) : 0;
            ast[p] = *reinterpret_cast<const uintx4*>(A + (size_t)row * K + kw0 * (kwl > 0) + c8 * 8);
        }
        const int sp_g = lane / (NSW * 2), sp_r = lane % (NSW * 2);  // group, 8-column piece
        const bool sp_ok = lane < SPL && sp_g * G < kwl && sp_r < 2 * nst && strip0 * 16 + sp_r * 8 < N;
        const uintx4 sreg = *reinterpret_cast<const uintx4*>(
            Sc + (sp_ok ? (size_t)(kw0 / G + sp_g) * ldS + strip0 * 16 + sp_r * 8 : 0));
        uintx4 braw[KCW][NSW][P];
#pragma unroll
        for (int i = 0; i < KCW; ++i)
#pragma unroll
            for (int s = 0; s < NSW; ++s) {
                const int c = i * 128 < kwl ? kw0 / 128 + i : 0;
                const uint8_t* blk = wf + wblock_offset<WB>(strip0 + (s < nst ? s : nst - 1), c, kchunks);
#pragma unroll
                for (int p = 0; p < P; ++p)
                    braw[i][s][p] = ldg_nt(reinterpret_cast<const uintx4*>(blk + p * 1024 + lane * 16));
            }
        // keep every load above ahead of the first use of any of them
        __builtin_amdgcn_sched_barrier(0);
        // stage A and C; rows < MT only, pieces of a (row, group) sit in GP adjacent lanes
#pragma unroll
        for (int p = 0; p < APL; ++p) {
            const int idx = lane + 64 * p, row = idx / (KW / 8), c8 = idx % (KW / 8);
            // (Whole-vector bit casts only: a bit cast of one element of a
            // u32x4 was miscompiled by this toolchain into element 0.)  A
            // piece at or past K (a ragged K's last chunk) stages as zeros, so
            // that it adds nothing to the raw products or to C.
            const bool kin = idx < APIECES && c8 * 8 < kwl;
            const half8 h = __builtin_bit_cast(half8, kin ? ast[p] : uintx4{0u, 0u, 0u, 0u});
            if constexpr (CM) {
                if (idx < APIECES) *reinterpret_cast<half8*>(&L.a[row * LDA + c8 * 8]) = h;
            } else {
                float part;
                if constexpr (B0 == B1) {
                    part = 0.f;
#pragma unroll
                    for (int j = 0; j < 8; ++j) part += (float)h[j];
                    part = group_sum<GP>(part) * B0;
                } else {
                    // elements j % 4 < 2 against bias B0, the others against B1
                    const float p0 = ((float)h[0] + (float)h[1]) + ((float)h[4] + (float)h[5]);
                    const float p1 = ((float)h[2] + (float)h[3]) + ((float)h[6] + (float)h[7]);
                    part = group_sum<GP>(p0 * B0 + p1 * B1);
                }
                if (idx < APIECES) {
                    *reinterpret_cast<half8*>(&L.a[row * LDA + c8 * 8]) = h;
                    if (c8 % GP == 0) L.c[c8 / GP][row] = part;
                }
            }
        }
        if (lane < SPL) *reinterpret_cast<uintx4*>(&L.s[sp_g][sp_r * 8]) = sreg;
        __builtin_amdgcn_wave_barrier();
        auto chunk = [&](int i) __attribute__((always_inline)) {
            const _Float16* ap = L.a + arow * LDA + i * 128 + q * 8;
            half8 a[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) a[kk] = *reinterpret_cast<const half8*>(ap + kk * 32);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int gl = i * NG + g;
                floatx4 cc;
                if constexpr (CM) {
                    const _Float16 k0 = (_Float16)B0, k1 = (_Float16)B1;
                    const half8 cb = {k0, k0, k1, k1, k0, k0, k1, k1};
                    cc = zero;
#pragma unroll
                    for (int kk = g * KKPG; kk < (g + 1) * KKPG; ++kk) cc = mfma16(a[kk], cb, cc);
                } else {
                    cc = *reinterpret_cast<const floatx4*>(&L.c[gl][4 * q]);
                }
#pragma unroll
                for (int s = 0; s < NSW; ++s) {
                    floatx4 tmp = zero;
#pragma unroll
                    for (int kk = g * KKPG; kk < (g + 1) * KKPG; ++kk)
                        tmp = mfma16(a[kk], raw_kstep<WB>(braw[i][s], kk), tmp);
                    const float sv = h2f(L.s[gl][s * 16 + cl]);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[s][j] = __builtin_fmaf(tmp[j] - cc[j], sv, acc[s][j]);
                }
            }
        };
        // A whole slice (every wave but one past a ragged K) runs as one block
        // of straight-line code, so the LDS reads of a chunk can go out before
        // the wait for its weights (int4 only: with the int8 weights' twice as
        // many registers the hoisted reads make the 16-wave shapes spill)
        if (P == 1 && kwl >= KW) {
#pragma unroll
            for (int i = 0; i < KCW; ++i) chunk(i);
        } else {
#pragma unroll
            for (int i = 0; i < KCW; ++i) {
                if (i * 128 >= kwl) break;
                chunk(i);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }

    // K partials of the workgroup's strips, added in wave order
    if constexpr (!OWN_RED) __syncthreads();
    floatx4* red = reinterpret_cast<floatx4*>(lds_raw + (OWN_RED ? STAGE : 0));
#pragma unroll
    for (int s = 0; s < NSW; ++s) red[(wave * NSW + s) * 64 + lane] = acc[s];
    __syncthreads();
    // wave w < NSW finalizes strip w: the partials are read RB at a time
    // before they are added (a chain of read, wait, add per partial is WK LDS
    // round trips); int8 weights leave fewer free registers, so four at a
    // time there
    if (wave < nst) {
        constexpr int RB = P == 1 ? WK : (WK < 4 ? WK : 4);
        floatx4 t;
#pragma unroll
        for (int w0 = 0; w0 < WK; w0 += RB) {
            floatx4 pw[RB];
#pragma unroll
            for (int w = 0; w < RB; ++w) pw[w] = red[((w0 + w) * NSW + wave) * 64 + lane];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int w = 0; w < RB; ++w) t = (w0 + w == 0) ? pw[0] : t + pw[w];
        }
        const int n = (strip0 + wave) * 16 + cl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 4 * q + j;  // accumulator layout: rows 4*(l/16)+j, column l%16
            if (row < M && n < N) Y[(size_t)row * N + n] = f2h(t[j]);
        }
    }
}

// ------------------------------------------------------------------ prefill

constexpr int PF_BM = 128, PF_BN = 128, PF_LDA = 136;  // LDS row: 128 halfs + 8 pad

template <int WB, int G>
__global__ __launch_bounds__(256, 2) void wq_prefill_kernel(const uint16_t* __restrict__ A,
                                                            const uint8_t* __restrict__ wf,
                                                            const uint16_t* __restrict__ S, int ldS,
                                                            uint16_t* __restrict__ Y, int M, int N,
                                                            int K) {
    typedef BChunk<2, G, WB> Chunk;
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][PF_BM * PF_LDA];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    // tile (x, y) of workgroup id L: y = L % (row tiles), see the large kernel
    const int mtiles = (M + PF_BM - 1) / PF_BM;
    const int L = blockIdx.x;
    const int m0 = (L % mtiles) * PF_BM, n0 = (L / mtiles) * PF_BN;
    const int kchunks = (K + 127) / 128;  // of the (padded) fragment layout
    const int gmax = (K + (G < 128 ? G : 128) - 1) / (G < 128 ? G : 128) - 1;  // last scale row
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
            // rows >= M repeat row M-1 (unconditional load; those rows are not
            // stored); pieces at or past K (ragged K) read the row's first
            // piece and become zeros
            const int k8 = c * 128 + col * 8;
            const uintx4 v = *reinterpret_cast<const uintx4*>(A + (size_t)(gm < M ? gm : M - 1) * K + (k8 < K ? k8 : 0));
            areg[i] = k8 < K ? v : uintx4{0u, 0u, 0u, 0u};
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = tid + 256 * i, row = idx >> 4, col = idx & 15;
            *reinterpret_cast<uintx4*>(&sA[buf][row * PF_LDA + col * 8]) = areg[i];
        }
    };

    auto compute = [&](const uint16_t* sa, const Chunk& b) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int kg = kgroup_of_step(s, h);
            half8 a[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const half8*>(&sa[(wm * 64 + i * 32 + c32) * PF_LDA + kg * 8]);
#pragma unroll
            for (int t = 0; t < 2; ++t) bf[t] = b_frag<2, G, WB>(b, t, s);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int t = 0; t < 2; ++t) acc[i][t] = mfma32(a[i], bf[t], acc[i][t]);
        }
    };

    // Two B register sets used alternately (no copies), two chunks per trip
    // and no branch inside a trip: a load under a branch, a load issued
    // before a branch but used only after it, or a register copy of in-flight
    // data makes the compiler wait for the prefetch before computing.  The
    // scheduling barriers keep the prefetch loads ahead of the compute.  The
    // last trip reloads its second chunk when the count is even; an odd count
    // leaves one staged chunk for the tail.
    Chunk b0, b1;
    load_a(0);
    load_b_chunk<2, G, WB>(b0, wf, S, ldS, kchunks, 0, ncol0, lane, gmax, N - 1);
    store_a(0);
    __syncthreads();
    int c = 0;
    for (; c + 1 < kchunks; c += 2) {
        load_a(c + 1);
        load_b_chunk<2, G, WB>(b1, wf, S, ldS, kchunks, c + 1, ncol0, lane, gmax, N - 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(sA[0], b0);
        __builtin_amdgcn_sched_barrier(0);
        store_a(1);
        __syncthreads();
        const int c2 = c + 2 < kchunks ? c + 2 : c + 1;
        load_a(c2);
        load_b_chunk<2, G, WB>(b0, wf, S, ldS, kchunks, c2, ncol0, lane, gmax, N - 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(sA[1], b1);
        __builtin_amdgcn_sched_barrier(0);
        store_a(0);
        __syncthreads();
    }
    if (c < kchunks) compute(sA[0], b0);

    // Epilogue through an LDS tile (128 rows x 320 bytes) so that Y is
    // written in 16-byte row pieces: a quad transpose gives each lane four
    // adjacent columns of one row.  The barrier waits for every wave's last
    // reads of the A buffers.
    __syncthreads();
    constexpr int EPW = 80;  // tile pitch in dwords (256 bytes + 64)
    uint32_t* stile = reinterpret_cast<uint32_t*>(&sA[0][0]);
    const int q = lane & 3;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int r0 = wm * 64 + i * 32 + 8 * g + 4 * h;  // tile row of register 4g
                const uint32_t v0 = f2h(acc[i][t][4 * g]), v1 = f2h(acc[i][t][4 * g + 1]);
                const uint32_t v2 = f2h(acc[i][t][4 * g + 2]), v3 = f2h(acc[i][t][4 * g + 3]);
                uint32_t e0, e1;
                quad_rows_u16(v0 | (v1 << 16), v2 | (v3 << 16), lane, e0, e1);
                *reinterpret_cast<uintx2*>(&stile[(r0 + q) * EPW + wn * 32 + t * 16 + 2 * (c32 >> 2)]) =
                    uintx2{e0, e1};
            }
    __syncthreads();
    // 128 rows x 16 pieces of 8 outputs (N % 8 == 0: a piece is all inside
    // or all past N)
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int idx = tid + 256 * p, row = idx >> 4, piece = idx & 15;
        if (m0 + row < M && n0 + piece * 8 < N)
            __builtin_nontemporal_store(*reinterpret_cast<const uintx4*>(&stile[row * EPW + piece * 4]),
                                        reinterpret_cast<uintx4*>(Y + (size_t)(m0 + row) * N + n0 + piece * 8));
    }
}

// Large-M prefill: 128x256 output tiles, four waves side by side, each
// 128 rows x 64 columns (4 x 2 v_mfma_f32_32x32x16_f16 tiles, accumulators in
// the unified VGPR/AGPR file); one workgroup per CU at M = 2048.  A tile that
// is wide in N suits weight-only GEMMs: per 128-k chunk a workgroup streams
// 32 KB of fp16 A and 16 KB (int4) or 32 KB (int8) of B (a 256 x 128 tile
// would need 64 KB + 8 or 16 KB for the same MFMA work), and each wave owns
// its columns, so every B element is dequantized once per workgroup.
//
// Every load in the main loop is a buffer -> LDS DMA (no VGPR destinations,
// no VALU).  This kernel takes int8 weights: two A buffers and two B stages
// (fragment blocks plus scale rows), its B stages being twice the int4
// size; int4 weights take the producer-wave kernel below, whose A and B have
// three buffers each.  A wave's A-DMA instruction
// fills 1 KB of LDS in lane order (four 256-byte rows); the lane that fills
// position pos of row r fetches piece pos ^ (r & 15) of that row, so the MFMA
// fragment reads, 16 rows at one k-group, hit 16 distinct 16-byte bank
// groups.  The loop waits for the DMA it needs with an explicit counter wait
// and a bare barrier: __syncthreads() would also wait for the B prefetch
// still in flight.
constexpr int PL_BM = 128, PL_BN = 256;

template <int WB, int G>
__global__ __launch_bounds__(256, 1) void wq_prefill_large_kernel(const uint16_t* __restrict__ A,
                                                                   const uint8_t* __restrict__ wf,
                                                                   const uint16_t* __restrict__ S, int ldS,
                                                                   uint16_t* __restrict__ Y, int M, int N,
                                                                   int K) {
    constexpr int NG = 128 / G;
    constexpr int KBLK = WFormat<WB>::kBlock;  // bytes per 16-column x 128-k block
    constexpr int P = WFormat<WB>::kPieces;
    static_assert(WB == 8, "int8 weights; int4 takes wq_prefill_large_pc_kernel");
    // two of each: chunk c + 2's B copies are spread over the k-steps of
    // trip c, the A copies wait for the boundary
    constexpr int NBST = 2;   // B stages
    constexpr int NABUF = 2;  // A buffers
    constexpr int SLAB = PL_BM * 128;          // halfs per A buffer (32 KB)
    constexpr int BST = 16 * KBLK + 512 * NG;  // bytes per B stage: 16 fragment blocks + NG scale rows
    constexpr int BDMA = 4 * P + 2 * NG;       // DMA instructions per wave for one B stage
    // One LDS array for A and B: the compiler tells DMA targets from the
    // buffers being read by their offsets within one array, but not across
    // two arrays (it would then wait for every DMA before each LDS read).
    // (One size for every instantiation, the largest: B stages with G = 32.
    // An array whose size depends on the template parameters, passed to the
    // DMA builtin, made the host compiler drop the kernel's launch stub
    // without a diagnostic.)
    __shared__ __attribute__((aligned(1024))) uint16_t sA[(2 * PL_BM * 128 * 2 + 2 * (32768 + 512 * 4)) / 2];
    static_assert(NABUF * PL_BM * 128 * 2 + NBST * BST <= (int)sizeof(sA), "A buffers and B stages fit the LDS array");
    uint8_t* const sB = reinterpret_cast<uint8_t*>(sA + NABUF * SLAB);
    // (the wave index as a scalar: every DMA's LDS destination and source
    // base are then scalar arithmetic)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Workgroups are dealt to the 8 XCDs round-robin by id.  Tile (x, y) of
    // id L has y = L % (row tiles), so the workgroups on one XCD share their
    // A row tiles in that XCD's L2 and stream distinct B tiles.  (Grouping
    // each XCD's tiles into a 4 x 8 block, xcd_tile, cuts the L2 misses but
    // measured 0.3 us slower at M = 2048, N = K = 4096.)
    const int mtiles = (M + PL_BM - 1) / PL_BM;
    const int L = blockIdx.x;
    const int m0 = (L % mtiles) * PL_BM, n0 = (L / mtiles) * PL_BN;
    const int kchunks = K / 128, last = kchunks - 1;
    const int h = lane >> 5, c32 = lane & 31;

    floatx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[i][t][j] = 0.f;

    // A: this lane's source for wave instruction j is row 4 * (8 * wave + j) + lane / 16,
    // piece (lane % 16) ^ (row & 15).  Rows >= M repeat row M - 1 (never stored).
    // Every DMA is a buffer load: a wave-uniform descriptor (A rows from m0,
    // the weight tile, the scale columns from n0), a loop-invariant 32-bit
    // byte offset per lane and a scalar offset per copy, so issuing a copy
    // takes no vector instructions.  Offsets stay below 2^31: the A tile
    // spans 128 rows of K halfs, the weight tile two 128-column strips of K.
    const int rsub = lane >> 4, pos = lane & 15;
    uint32_t aoff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = 4 * (8 * wave + j) + rsub;
        const int gr = m0 + r < M ? r : M - 1 - m0;
        aoff[j] = ((uint32_t)gr * (uint32_t)K + (uint32_t)((pos ^ (r & 15)) * 8)) * 2u;
    }
    const int arows = M - m0 < PL_BM ? M - m0 : PL_BM;
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(A + (size_t)m0 * K, (uint32_t)arows * (uint32_t)K * 2u);
    auto dma_a = [&](int c, int buf) {
#pragma unroll
        for (int j = 0; j < 8; ++j) buffer_load_lds<16>(ra, sA + buf * SLAB + (8 * wave + j) * 512, aoff[j], c * 256);
    };
    // B: the tile's 256 columns are strips n0/16 .. n0/16 + 15, two 8-block
    // fragment tiles per chunk (stored one after the other in a stage);
    // wave w copies strips 4w .. 4w + 3, 1 KB per DMA instruction.  Each
    // wave also copies every scale row of the chunk (512 bytes each; the four
    // copies write identical bytes), which keeps the per-wave DMA count equal.
    const uint32_t sb_stride = (uint32_t)kchunks * (8 * KBLK);  // between the two fragment tiles
    const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(wf + (size_t)(n0 >> 7) * sb_stride, 2u * sb_stride);
    const uint32_t srows = ldS == 0 ? 1u : (uint32_t)(K / G);
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(S + n0, ((srows - 1u) * (uint32_t)ldS + (uint32_t)PL_BN) * 2u);
    const uint32_t boff = (uint32_t)lane * 16u, soff = (uint32_t)lane * 4u;
    auto dma_b = [&](int c, int stage) {
        uint8_t* dst = sB + stage * BST;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int strip = 4 * wave + j;
#pragma unroll
            for (int p = 0; p < P; ++p)
                buffer_load_lds<16>(rb, dst + strip * KBLK + p * 1024, boff,
                                    (uint32_t)c * (8 * KBLK) + (strip >> 3) * sb_stride + (strip & 7) * KBLK + p * 1024);
        }
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                buffer_load_lds<4>(rs, dst + 16 * KBLK + g * 512 + hh * 256, soff,
                                   ((uint32_t)(c * NG + g) * (uint32_t)ldS + 128u * hh) * 2u);
    };
    // DMA instruction i of chunk c (i < 8: A; then the B blocks, then the
    // scale rows), for issuing a chunk's copies a few at a time
    auto dma_one = [&](int c, int buf, int stage, int i) __attribute__((always_inline)) {
        if (i < 8) {
            buffer_load_lds<16>(ra, sA + buf * SLAB + (8 * wave + i) * 512, aoff[i], c * 256);
        } else if (i < 8 + 4 * P) {
            const int strip = 4 * wave + (i - 8) / P, p = (i - 8) % P;
            buffer_load_lds<16>(rb, sB + stage * BST + strip * KBLK + p * 1024, boff,
                                (uint32_t)c * (8 * KBLK) + (strip >> 3) * sb_stride + (strip & 7) * KBLK + p * 1024);
        } else {
            const int g = (i - 8 - 4 * P) / 2, hh = (i - 8 - 4 * P) % 2;
            buffer_load_lds<4>(rs, sB + stage * BST + 16 * KBLK + g * 512 + hh * 256, soff,
                               ((uint32_t)(c * NG + g) * (uint32_t)ldS + 128u * hh) * 2u);
        }
    };
    // this lane's B fragment pieces inside a stage: tile t, k-group parity h,
    // pieces q = h and q = h + 2 of the strip holding column 64 wave + 32 t + c32
    typedef BChunk<2, G, WB> Chunk;
    auto read_b = [&](const uint8_t* sb, Chunk& b) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int colt = wave * 64 + t * 32 + c32;  // column inside the tile
            const uint8_t* blk = sb + (colt >> 4) * KBLK + (colt & 15) * 16;
#pragma unroll
            for (int qi = 0; qi < 2; ++qi)
#pragma unroll
                for (int p = 0; p < P; ++p)
                    b.raw[t][qi * P + p] = *reinterpret_cast<const uintx4*>(blk + p * 1024 + 16 * 16 * (h + 2 * qi));
#pragma unroll
            for (int g = 0; g < NG; ++g)
                b.sc[t][g] = reinterpret_cast<const uint16_t*>(sb + 16 * KBLK)[g * 256 + colt];
        }
    };
    // Software-pipelined k-steps: the LDS reads and the dequant of step s + 1
    // are interleaved with the eight MFMAs of step s (one MFMA, then at most
    // one LDS read and four VALU ops), so the in-order wave keeps the MFMA
    // unit busy while it prepares the next operands.  The pipeline runs
    // across chunks too: the chunk boundary (counter wait and barrier) comes
    // before the last k-step, whose MFMAs then cover the next chunk's B
    // register reads, its first operands and the DMA issue.
    auto a_frags = [&](const uint16_t* sa, int s, half8 (&a)[4]) {
        const int kg = kgroup_of_step(s, h);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = i * 32 + c32;
            a[i] = *reinterpret_cast<const half8*>(&sa[r * 128 + ((kg ^ (r & 15)) * 8)]);
        }
    };
    auto operands = [&](const uint16_t* sa, const Chunk& b, int s, half8 (&a)[4], half8 (&bf)[2]) {
        a_frags(sa, s, a);
#pragma unroll
        for (int t = 0; t < 2; ++t) bf[t] = b_frag<2, G, WB>(b, t, s);
    };
    auto mfmas = [&](const half8 (&a)[4], const half8 (&bf)[2]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < 2; ++t) acc[i][t] = mfma32(a[i], bf[t], acc[i][t]);
    };
    // Pipeline state between trips: chunk c's B registers and the operands of
    // its first k-step.
    Chunk b;
    half8 a[4], bf[2];
    // One trip = k-steps 0..6 of chunk c with chunk c + 2's B copies (into
    // chunk c's stage, whose registers were read one trip earlier), the
    // boundary, then k-step 7 with chunk c + 1's set-up and chunk c + 2's A
    // copies (into the buffer chunk c was read from).  Every LDS offset a DMA
    // writes is a compile-time constant in each trip (buf and stage are
    // literals at every call; after inlining they fold): with a run-time
    // index the compiler cannot tell the DMA target from the buffer being
    // read and waits for the DMA before every LDS read.  The DMA indexes
    // clamp to the last chunk: the copies past the end are never read.
    auto trip = [&](int c, int buf, int stage) __attribute__((always_inline)) {
        const uint16_t* sa = sA + buf * SLAB;
        // chunk c + 2's B copies go out two or three per k-step: issued as
        // one burst, the four waves' copies queue up in the address unit and
        // each wave stalls at issue while the matrix unit runs dry
        const int cd = c + 2 < last ? c + 2 : last;
#pragma unroll
        for (int s = 0; s < 7; ++s) {
            half8 an[4], bn[2];
            operands(sa, b, s + 1, an, bn);
#pragma unroll
            for (int i = 8 + s * BDMA / 7; i < 8 + (s + 1) * BDMA / 7; ++i) dma_one(cd, buf, stage, i);
            mfmas(a, bf);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                if (q < 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                if (q == 1 || q == 3 || q == 5) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // one copy
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = an[i];
#pragma unroll
            for (int t = 0; t < 2; ++t) bf[t] = bn[t];
        }
        // chunk c + 1's A and B have landed (chunk c + 2's B copies, issued
        // this trip, may still be in flight); every wave's reads of chunk c's
        // A buffer are done
        wait_vmcnt<BDMA>();
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const int nbuf = buf + 1 < NABUF ? buf + 1 : 0, nstage = stage + 1 < NBST ? stage + 1 : 0;
        // first half: the LDS reads, then the A DMAs, under four MFMAs
        read_b(sB + nstage * BST, b);
        half8 an[4], bn[2];
        a_frags(sA + nbuf * SLAB, 0, an);
        dma_a(c + NABUF < last ? c + NABUF : last, buf);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            acc[0][t] = mfma32(a[0], bf[t], acc[0][t]);
            acc[1][t] = mfma32(a[1], bf[t], acc[1][t]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            if (q < 2) __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);  // LDS reads
            else __builtin_amdgcn_sched_group_barrier(0x010, 4, 0);   // DMA issue
        }
        // (a barrier to the scheduler: every A DMA is issued before the B DMAs,
        // which the counter wait above relies on)
        __builtin_amdgcn_sched_barrier(0);
        // second half: the dequant of chunk c + 1's first step
#pragma unroll
        for (int t = 0; t < 2; ++t) bn[t] = b_frag<2, G, WB>(b, t, 0);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            acc[2][t] = mfma32(a[2], bf[t], acc[2][t]);
            acc[3][t] = mfma32(a[3], bf[t], acc[3][t]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            if (q < 2) __builtin_amdgcn_sched_group_barrier(0x010, 4, 0);  // DMA issue
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = an[i];
#pragma unroll
        for (int t = 0; t < 2; ++t) bf[t] = bn[t];
    };

    // chunks 0 and 1
#pragma unroll
    for (int ab = 0; ab < NABUF; ++ab) dma_a(ab < last ? ab : last, ab);
#pragma unroll
    for (int st = 0; st < NBST; ++st) dma_b(st < last ? st : last, st);
    wait_vmcnt<0>();
    __syncthreads();
    read_b(sB, b);
    operands(sA, b, 0, a, bf);
    for (int c = 0; c < kchunks; c += 2) {
        trip(c, 0, 0);
        if (c + 1 < kchunks) trip(c + 1, 1, 1);
    }
    // ---- epilogue: Y through an LDS tile in 16-byte row pieces.  A quad
    // transpose gives each lane four adjacent columns of one row (8 bytes of
    // fp16), stored into a row-major tile of pitch 576 bytes; then every
    // thread writes whole 16-byte pieces, non-temporal (Y is not read again
    // here; at one tile per CU the write burst at the end is exposed, and the
    // streaming stores took 62.5 -> 61.3 us at M = 2048, K = N = 4096).  Each wave first drains its last
    // (unused) prefetches, and the barrier makes sure no DMA still writes LDS.
    wait_vmcnt<0>();
    __syncthreads();
    constexpr int EPW = 144;  // tile pitch in dwords (512 bytes + 64)
    uint32_t* stile = reinterpret_cast<uint32_t*>(sA);
    const int q = lane & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int r0 = i * 32 + 8 * g + 4 * h;  // tile row of register 4g
                const uint32_t v0 = f2h(acc[i][t][4 * g]), v1 = f2h(acc[i][t][4 * g + 1]);
                const uint32_t v2 = f2h(acc[i][t][4 * g + 2]), v3 = f2h(acc[i][t][4 * g + 3]);
                uint32_t e0, e1;
                quad_rows_u16(v0 | (v1 << 16), v2 | (v3 << 16), lane, e0, e1);
                *reinterpret_cast<uintx2*>(&stile[(r0 + q) * EPW + wave * 32 + t * 16 + 2 * (c32 >> 2)]) =
                    uintx2{e0, e1};
            }
    __syncthreads();
    // 128 rows x 32 pieces of 8 outputs (N % 256 == 0: every piece is whole and aligned)
    const int tid = threadIdx.x;
#pragma unroll 4
    for (int p = 0; p < 16; ++p) {
        const int idx = tid + 256 * p, row = idx >> 5, piece = idx & 31;
        if (m0 + row < M)
            __builtin_nontemporal_store(*reinterpret_cast<const uintx4*>(&stile[row * EPW + piece * 4]),
                                        reinterpret_cast<uintx4*>(Y + (size_t)(m0 + row) * N + n0 + piece * 8));
    }
}

// Large-M prefill for int4 weights: the tile, k-step pipeline and epilogue
// of the kernel above, with three A buffers and three B stages, and a fifth
// wave that issues every DMA copy.  Waves 0..3 compute and issue no memory
// instruction in the main loop; wave 4 copies chunk c + 2 (32 A rows of
// 1 KB, 16 fragment blocks, the scale rows once) during trip c into the
// buffers chunk c - 1 used, waits for chunk c + 1 and meets the computing
// waves at the barrier of their trip c.  Against the same kernel with each
// computing wave issuing its share of the copies, spread over its k-steps:
// 58.1 against 59.0 us and 61.9 against 62.9 us (two boxes, M = 2048,
// K = N = 4096), bit-identical outputs; the copies themselves still cost
// (issued with pauses between groups of eight they arrive late: 66.7 us).
// The computing waves fit 256 registers (two waves share one SIMD).
template <int G>
__global__ __launch_bounds__(320, 1) void wq_prefill_large_pc_kernel(const uint16_t* __restrict__ A,
                                                               const uint8_t* __restrict__ wf,
                                                               const uint16_t* __restrict__ S, int ldS,
                                                               uint16_t* __restrict__ Y, int M, int N, int K) {
    constexpr int WB = 4;
    constexpr int NG = 128 / G;
    constexpr int KBLK = WFormat<WB>::kBlock;
    constexpr int P = WFormat<WB>::kPieces;
    constexpr int SLAB = PL_BM * 128;
    constexpr int BST = 16 * KBLK + 512 * NG;
    constexpr int NCP = 32 + 16 * P + 2 * NG;  // copies per chunk
    static_assert(NCP < 64, "one chunk's copies fit the counter");
    __shared__ __attribute__((aligned(1024))) uint16_t sA[(3 * PL_BM * 128 * 2 + 3 * (16384 + 512 * 4)) / 2];
    uint8_t* const sB = reinterpret_cast<uint8_t*>(sA + 3 * SLAB);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int mtiles = (M + PL_BM - 1) / PL_BM;
    const int L = blockIdx.x;
    const int m0 = (L % mtiles) * PL_BM, n0 = (L / mtiles) * PL_BN;
    const int kchunks = K / 128, last = kchunks - 1;

    if (wave == 4) {
        const int rsub = lane >> 4, pos = lane & 15;
        uint32_t aoff[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const int r = 4 * j + rsub;
            const int gr = m0 + r < M ? r : M - 1 - m0;
            aoff[j] = ((uint32_t)gr * (uint32_t)K + (uint32_t)((pos ^ (r & 15)) * 8)) * 2u;
        }
        const int arows = M - m0 < PL_BM ? M - m0 : PL_BM;
        const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(A + (size_t)m0 * K, (uint32_t)arows * (uint32_t)K * 2u);
        const uint32_t sb_stride = (uint32_t)kchunks * (8 * KBLK);
        const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(wf + (size_t)(n0 >> 7) * sb_stride, 2u * sb_stride);
        const uint32_t srows = ldS == 0 ? 1u : (uint32_t)(K / G);
        const __amdgpu_buffer_rsrc_t rs =
            buffer_rsrc(S + n0, ((srows - 1u) * (uint32_t)ldS + (uint32_t)PL_BN) * 2u);
        const uint32_t boff = (uint32_t)lane * 16u, soff = (uint32_t)lane * 4u;
        auto copy = [&](int c, int buf, int i) __attribute__((always_inline)) {
            if (i < 32) {
                buffer_load_lds<16>(ra, sA + buf * SLAB + i * 512, aoff[i], c * 256);
            } else if (i < 32 + 16 * P) {
                const int strip = (i - 32) / P, p = (i - 32) % P;
                buffer_load_lds<16>(rb, sB + buf * BST + strip * KBLK + p * 1024, boff,
                                    (uint32_t)c * (8 * KBLK) + (strip >> 3) * sb_stride + (strip & 7) * KBLK + p * 1024);
            } else {
                const int g = (i - 32 - 16 * P) / 2, hh = (i - 32 - 16 * P) % 2;
                buffer_load_lds<4>(rs, sB + buf * BST + 16 * KBLK + g * 512 + hh * 256, soff,
                                   ((uint32_t)(c * NG + g) * (uint32_t)ldS + 128u * hh) * 2u);
            }
        };
        // groups of eight, at most 63 copies outstanding
        auto issue = [&](int c, int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int i0 = 0; i0 < NCP; i0 += 8) {
                wait_vmcnt<55>();
#pragma unroll
                for (int i = i0; i < i0 + 8 && i < NCP; ++i) copy(c, buf, i);
            }
        };
        issue(0, 0);
        issue(1 < last ? 1 : last, 1);
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        // trip c: chunk c + 2 into the buffer chunk c - 1 used (free since the
        // previous barrier), then wait for chunk c + 1 and meet the computing
        // waves at the barrier of their trip c
        auto ptrip = [&](int c, int dbuf) __attribute__((always_inline)) {
            issue(c + 2 < last ? c + 2 : last, dbuf);
            wait_vmcnt<NCP>();
            __builtin_amdgcn_s_barrier();
        };
        for (int c = 0; c < kchunks; c += 3) {
            ptrip(c, 2);
            if (c + 1 < kchunks) ptrip(c + 1, 0);
            if (c + 2 < kchunks) ptrip(c + 2, 1);
        }
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();  // the epilogue's two barriers
        __builtin_amdgcn_s_barrier();
        return;
    }

    const int h = lane >> 5, c32 = lane & 31;
    floatx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[i][t][j] = 0.f;
    typedef BChunk<2, G, WB> Chunk;
    auto read_b = [&](const uint8_t* sb, Chunk& b) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int colt = wave * 64 + t * 32 + c32;
            const uint8_t* blk = sb + (colt >> 4) * KBLK + (colt & 15) * 16;
#pragma unroll
            for (int qi = 0; qi < 2; ++qi)
#pragma unroll
                for (int p = 0; p < P; ++p)
                    b.raw[t][qi * P + p] = *reinterpret_cast<const uintx4*>(blk + p * 1024 + 16 * 16 * (h + 2 * qi));
#pragma unroll
            for (int g = 0; g < NG; ++g)
                b.sc[t][g] = reinterpret_cast<const uint16_t*>(sb + 16 * KBLK)[g * 256 + colt];
        }
    };
    auto a_frags = [&](const uint16_t* sa, int s, half8 (&a)[4]) {
        const int kg = kgroup_of_step(s, h);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = i * 32 + c32;
            a[i] = *reinterpret_cast<const half8*>(&sa[r * 128 + ((kg ^ (r & 15)) * 8)]);
        }
    };
    auto operands = [&](const uint16_t* sa, const Chunk& b, int s, half8 (&a)[4], half8 (&bf)[2]) {
        a_frags(sa, s, a);
#pragma unroll
        for (int t = 0; t < 2; ++t) bf[t] = b_frag<2, G, WB>(b, t, s);
    };
    auto mfmas = [&](const half8 (&a)[4], const half8 (&bf)[2]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < 2; ++t) acc[i][t] = mfma32(a[i], bf[t], acc[i][t]);
    };
    Chunk b;
    half8 a[4], bf[2];
    auto trip = [&](int buf) __attribute__((always_inline)) {
        const uint16_t* sa = sA + buf * SLAB;
#pragma unroll
        for (int s = 0; s < 7; ++s) {
            half8 an[4], bn[2];
            operands(sa, b, s + 1, an, bn);
            mfmas(a, bf);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                if (q < 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = an[i];
#pragma unroll
            for (int t = 0; t < 2; ++t) bf[t] = bn[t];
        }
        // every wave's reads of chunk c are done; the producer has waited for chunk c + 1
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const int nbuf = buf + 1 < 3 ? buf + 1 : 0;
        read_b(sB + nbuf * BST, b);
        half8 an[4], bn[2];
        a_frags(sA + nbuf * SLAB, 0, an);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            acc[0][t] = mfma32(a[0], bf[t], acc[0][t]);
            acc[1][t] = mfma32(a[1], bf[t], acc[1][t]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            if (q < 2) __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);  // LDS reads
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 2; ++t) bn[t] = b_frag<2, G, WB>(b, t, 0);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            acc[2][t] = mfma32(a[2], bf[t], acc[2][t]);
            acc[3][t] = mfma32(a[3], bf[t], acc[3][t]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = an[i];
#pragma unroll
        for (int t = 0; t < 2; ++t) bf[t] = bn[t];
    };
    __syncthreads();
    read_b(sB, b);
    operands(sA, b, 0, a, bf);
    for (int c = 0; c < kchunks; c += 3) {
        trip(0);
        if (c + 1 < kchunks) trip(1);
        if (c + 2 < kchunks) trip(2);
    }
    __syncthreads();
    constexpr int EPW = 144;
    uint32_t* stile = reinterpret_cast<uint32_t*>(sA);
    const int q = lane & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int r0 = i * 32 + 8 * g + 4 * h;
                const uint32_t v0 = f2h(acc[i][t][4 * g]), v1 = f2h(acc[i][t][4 * g + 1]);
                const uint32_t v2 = f2h(acc[i][t][4 * g + 2]), v3 = f2h(acc[i][t][4 * g + 3]);
                uint32_t e0, e1;
                quad_rows_u16(v0 | (v1 << 16), v2 | (v3 << 16), lane, e0, e1);
                *reinterpret_cast<uintx2*>(&stile[(r0 + q) * EPW + wave * 32 + t * 16 + 2 * (c32 >> 2)]) =
                    uintx2{e0, e1};
            }
    __syncthreads();
    const int tid = threadIdx.x;
#pragma unroll 4
    for (int p = 0; p < 16; ++p) {
        const int idx = tid + 256 * p, row = idx >> 5, piece = idx & 31;
        if (m0 + row < M)
            __builtin_nontemporal_store(*reinterpret_cast<const uintx4*>(&stile[row * EPW + piece * 4]),
                                        reinterpret_cast<uintx4*>(Y + (size_t)(m0 + row) * N + n0 + piece * 8));
    }
}

// ------------------------------------------------------------------ mid M

// measured crossover: at M = 192 and 256 the two row passes re-stream the
// weights and the single-pass prefill kernel is faster (47 us against 52 / 63
// at N = 11008, K = 4096)
constexpr int MID_MAX_M = 128;

// K splits of the mid-M path: as many 128-column x K-range workgroups as fit
// in one round at two per CU (a 513th workgroup would double the time), at
// least one chunk each.
__host__ __device__ inline int mid_splits(int N, int K) {
    const int tiles = N / 128, kchunks = K / 128;
    int s = 512 / tiles;
    if (s > kchunks) s = kchunks;
    if (s > 16) s = 16;
    return s < 1 ? 1 : s;
}

__host__ __device__ inline size_t mid_workspace_bytes(int M, int N, int K) {
    return (size_t)mid_splits(N, K) * M * N * sizeof(float);
}

// Workgroup L: column tile L % tiles (consecutive ids, which the dispatcher
// spreads over the XCDs, take neighbouring tiles), K split L / tiles over
// chunks [ks * kc / S, (ks + 1) * kc / S).  part[ks][m][n] fp32.
template <int WB, int G>
__global__ __launch_bounds__(256, 2) void wq_mid_kernel(const uint16_t* __restrict__ A,
                                                        const uint8_t* __restrict__ wf,
                                                        const uint16_t* __restrict__ S, int ldS,
                                                        float* __restrict__ part, int M, int N, int K,
                                                        int splits) {
    __shared__ __attribute__((aligned(1024))) uint16_t sA[2 * XP_SLAB];
    const int tiles = N / 128, kchunks = K / 128;
    const int ct = blockIdx.x % tiles, ks = blockIdx.x / tiles;
    const int c0 = (int)((long)ks * kchunks / splits), c1 = (int)((long)(ks + 1) * kchunks / splits);
    const uint8_t* wfp[1] = {wf};
    const uint16_t* sp[1] = {S};
    const int ncol0 = ct * 128 + (threadIdx.x >> 6) * 32;
    float* out = part + (size_t)ks * M * N;
    for (int r0 = 0; r0 < M; r0 += 128) {
        const int R = M - r0 < 128 ? M - r0 : 128;
        // element offset of A row r of this pass (M * K < 2^32 is checked at launch)
        auto row_key = [&](int r) -> uint32_t { return (uint32_t)(r0 + r); };
        auto key_off = [&](uint32_t k) -> uint32_t { return k * (uint32_t)K; };
        switch ((R + 31) / 32) {
            case 1: expert_pass<G, 1, 1, 1, WB>(sA, A, row_key, key_off, R, wfp, sp, N, ldS, kchunks, c0, c1, ncol0, r0, out); break;
            case 2: expert_pass<G, 1, 2, 1, WB>(sA, A, row_key, key_off, R, wfp, sp, N, ldS, kchunks, c0, c1, ncol0, r0, out); break;
            case 3: expert_pass<G, 1, 3, 1, WB>(sA, A, row_key, key_off, R, wfp, sp, N, ldS, kchunks, c0, c1, ncol0, r0, out); break;
            default: expert_pass<G, 1, 4, 1, WB>(sA, A, row_key, key_off, R, wfp, sp, N, ldS, kchunks, c0, c1, ncol0, r0, out); break;
        }
        __syncthreads();  // the next pass refills both LDS buffers
    }
}

// Y[i] = fp16(sum over splits s = 0 .. S-1 of part[s][i]), s ascending; eight
// outputs per lane per step, grid-stride.  S is a compile-time constant, so
// every split's loads go out before the first add (a loop over a run-time S
// waited for each split's loads in turn: S memory round trips per output).
template <int S>
__global__ __launch_bounds__(256) void wq_splitk_reduce_kernel(const float* __restrict__ part,
                                                               uint16_t* __restrict__ Y, size_t n8,
                                                               size_t stride_s) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < n8; c += stride) {
        const float* p = part + c * 8;
        floatx4 lo[S], hi[S];
#pragma unroll
        for (int s = 0; s < S; ++s) {
            lo[s] = *reinterpret_cast<const floatx4*>(p + s * stride_s);
            hi[s] = *reinterpret_cast<const floatx4*>(p + s * stride_s + 4);
        }
#pragma unroll
        for (int s = 1; s < S; ++s) {
            lo[0] += lo[s];
            hi[0] += hi[s];
        }
        const uintx4 o = {(uint32_t)f2h(lo[0][0]) | ((uint32_t)f2h(lo[0][1]) << 16),
                          (uint32_t)f2h(lo[0][2]) | ((uint32_t)f2h(lo[0][3]) << 16),
                          (uint32_t)f2h(hi[0][0]) | ((uint32_t)f2h(hi[0][1]) << 16),
                          (uint32_t)f2h(hi[0][2]) | ((uint32_t)f2h(hi[0][3]) << 16)};
        *reinterpret_cast<uintx4*>(Y + c * 8) = o;
    }
}

// Decode launches.  (MT, NSW, KCW): rows of the MFMA tile, 16-column strips
// per wave, 128-k chunks per wave; the workgroup is 32 / KCW waves over NSW
// strips.  Narrow (M <= 2): one strip per workgroup of eight waves, 4 chunks
// per wave.  Balanced (M <= 16): at least one workgroup per CU where there
// are enough strips, each over a contiguous range of at most three strips.
template <int WB, int G>
void launch_wq_decode_narrow(const uint16_t* A, const uint8_t* wf, const uint16_t* S, int ldS, uint16_t* Y,
                             int M, int N, int K, hipStream_t st) {
    const int nwg = decode_grid(N, false);
    if (M == 1)
        hipLaunchKernelGGL((wq_decode_kernel<WB, 1, 1, 4, G, false>), dim3(nwg), dim3(512), 0, st, A, wf,
                           S, ldS, Y, M, N, K);
    else
        hipLaunchKernelGGL((wq_decode_kernel<WB, 2, 1, 4, G, false>), dim3(nwg), dim3(512), 0, st, A, wf,
                           S, ldS, Y, M, N, K);
}

template <int WB, int G>
void launch_wq_decode_balanced(const uint16_t* A, const uint8_t* wf, const uint16_t* S, int ldS, uint16_t* Y,
                               int M, int N, int K, hipStream_t st) {
    const int nwg = decode_grid(N, true);
    if (M <= 4)
        hipLaunchKernelGGL((wq_decode_kernel<WB, 4, 3, 2, G, true>), dim3(nwg), dim3(1024), 0, st, A, wf, S,
                           ldS, Y, M, N, K);
    else if (M <= 8)
        hipLaunchKernelGGL((wq_decode_kernel<WB, 8, 3, 2, G, true>), dim3(nwg), dim3(1024), 0, st, A, wf, S,
                           ldS, Y, M, N, K);
    else
        hipLaunchKernelGGL((wq_decode_kernel<WB, 16, 3, 2, G, true>), dim3(nwg), dim3(1024), 0, st, A, wf, S,
                           ldS, Y, M, N, K);
}

// One launch of the decode kernel for M <= 16 (the shapes measured fastest).
template <int WB, int G>
void launch_wq_decode(const uint16_t* A, const uint8_t* wf, const uint16_t* S, int ldS, uint16_t* Y, int M,
                      int N, int K, hipStream_t st) {
    if (M <= 2)
        launch_wq_decode_narrow<WB, G>(A, wf, S, ldS, Y, M, N, K, st);
    else
        launch_wq_decode_balanced<WB, G>(A, wf, S, ldS, Y, M, N, K, st);
}

template <int WB, int G>
void launch_wq_prefill(const uint16_t* A, const uint8_t* wf, const uint16_t* S, int ldS, uint16_t* Y, int M,
                       int N, int K, hipStream_t st) {
    dim3 grid(((N + PF_BN - 1) / PF_BN) * ((M + PF_BM - 1) / PF_BM));
    hipLaunchKernelGGL((wq_prefill_kernel<WB, G>), grid, dim3(256), 0, st, A, wf, S, ldS, Y, M, N, K);
}

template <int WB, int G>
void launch_wq_mid(const uint16_t* A, const uint8_t* wf, const uint16_t* S, int ldS, uint16_t* Y, int M,
                   int N, int K, float* part, hipStream_t st) {
    const int splits = mid_splits(N, K);
    hipLaunchKernelGGL((wq_mid_kernel<WB, G>), dim3((N / 128) * splits), dim3(256), 0, st, A, wf, S, ldS,
                       part, M, N, K, splits);
    const size_t n8 = (size_t)M * N / 8, want = (n8 + 255) / 256;
    const dim3 grid((int)(want < 4096 ? want : 4096));
    const size_t ss = (size_t)M * N;
    switch (splits) {  // mid_splits keeps 1 <= splits <= 16
#define QG_REDUCE(S_) \
    case S_: hipLaunchKernelGGL(wq_splitk_reduce_kernel<S_>, grid, dim3(256), 0, st, part, Y, n8, ss); break;
        QG_REDUCE(1) QG_REDUCE(2) QG_REDUCE(3) QG_REDUCE(4) QG_REDUCE(5) QG_REDUCE(6) QG_REDUCE(7) QG_REDUCE(8)
        QG_REDUCE(9) QG_REDUCE(10) QG_REDUCE(11) QG_REDUCE(12) QG_REDUCE(13) QG_REDUCE(14) QG_REDUCE(15)
        default: hipLaunchKernelGGL(wq_splitk_reduce_kernel<16>, grid, dim3(256), 0, st, part, Y, n8, ss); break;
#undef QG_REDUCE
    }
}

// Shapes the mid-M path takes (given enough workspace).
inline bool mid_path(int M, int K) {
    return M > 16 && M <= MID_MAX_M && (size_t)M * K < ((size_t)1 << 31);
}

// K or N not a multiple of 128: only the decode and 128x128 prefill kernels
// (register-staged A with a per-piece K test, masked stores) take such
// shapes; the split-K and 128x256 kernels copy A straight to LDS by DMA and
// assume whole 128-k chunks and 128-column tiles.
inline bool ragged(int N, int K) { return N % 128 != 0 || K % 128 != 0; }

}  // namespace
