// B-stationary weight-only pass (int4 or int8 weights, WB bits) shared by
// the MoE grouped GEMMs and the mid-M split-K GEMMs: a workgroup of four
// waves owns 128 columns of NB weight
// matrices (wave w: columns 32w .. 32w + 31) and runs R <= 128 rows of A
// through them over the 128-k chunks c0 .. c1 - 1, so each weight byte of
// its range is read once.  A rows reach LDS by buffer -> LDS DMA, double-
// buffered and XOR-swizzled; B fragments come straight from the fragment
// layout into registers one chunk ahead and are dequantized once per k-step
// for all NRB 32-row MFMA blocks (v_mfma_f32_32x32x16_f16).
#pragma once

#include <type_traits>

#include "wq_tile.hpp"

namespace qg {

constexpr int XP_SLAB = 128 * 128;  // halfs per LDS A buffer: 128 rows of 128 k (32 KB)

// MODE 0 (NB = 2, gate and up): out[slot][n] = fp16(act(g) * u), fp16, act
// the gate activation (moe_act).
// MODE 1: out[slot][n] = the fp32 partial sum over the pass's chunk range
// (the K splits of the MoE down projection and of the mid-M GEMM).
// slot0 + row indexes the output row; key_off(row_key(r)) is the element
// offset of A row r of the pass from abase.  N is the row stride of out, ldS
// that of the scales (0: one scale per column).
// Gate activation of the gated expert FFN (QGEMM_MOE_ACT_*): SiLU, GELU
// (erf form, tanh form) or ReLU, in fp32.
__device__ __forceinline__ float moe_act(float g, int act) {
    switch (act) {
        case QGEMM_MOE_ACT_GELU_ERF: return 0.5f * g * (1.0f + erff(g * 0.70710678f));
        case QGEMM_MOE_ACT_GELU_TANH:
            return 0.5f * g * (1.0f + tanhf(0.79788456f * (g + 0.044715f * g * g * g)));
        case QGEMM_MOE_ACT_RELU: return fmaxf(g, 0.0f);
        default: return g / (1.0f + expf(-g));
    }
}

// row_key(r) names A row r of the pass (it may load: a gathered row's pair
// index), key_off(key) turns that name into the row's element offset from
// abase.
template <int G, int NB, int NRB, int MODE, int WB, typename RowKey, typename KeyOff>
__device__ __forceinline__ void expert_pass(uint16_t* sA, const uint16_t* abase, RowKey row_key,
                                            KeyOff key_off, int R,
                                            const uint8_t* const* wf, const uint16_t* const* S,
                                            int N, int ldS, int kchunks, int c0, int c1, int ncol0,
                                            int slot0, void* out, int act = 0) {
    typedef BChunk<1, G, WB> Chunk;
    // (the wave index from threadIdx.x: its known range lets the compiler
    // tell the copies' LDS targets from the buffer being read)
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int h = lane >> 5, c32 = lane & 31;
    floatx16 acc[NB][NRB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < NRB; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[b][i][j] = 0.f;

    // DMA: the workgroup's 8 NRB wave instructions each fill 1 KB of LDS =
    // rows 4g .. 4g+3 (g = 2 NRB wave + j); lane l fetches piece
    // (l % 16) ^ (row % 16) of row 4g + l / 16.  Rows >= R repeat row R - 1.
    // Every load is a buffer load: a wave-uniform descriptor built per chunk
    // from 64-bit base pointers (A at the chunk's first k, the chunk's
    // fragment tile, its first scale row), a loop-invariant 32-bit byte
    // offset per lane, so a load takes no vector address arithmetic.  The
    // callers keep the A element offsets below 2^31 (byte offsets below
    // 2^32); the descriptors do not bound.
    // The row keys come first (for gathered rows, a load of the pair index
    // each), then the first chunk's B loads go out, and only then are the keys
    // used: loads complete in issue order, so this waits for the keys alone
    // and the weight stream starts one round trip earlier than behind that
    // wait.
    const int rsub = lane >> 4, pos = lane & 15;
    uint32_t src[2 * NRB];  // row keys, then byte offsets from the chunk's first k of abase
#pragma unroll
    for (int j = 0; j < 2 * NRB; ++j) {
        const int r = 4 * (2 * NRB * wave + j) + rsub;
        src[j] = row_key(r < R ? r : R - 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    auto dma_a_one = [&](int c, int buf, int j) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(abase + (size_t)c * 128, 0xffffffffu);
        buffer_load_lds<16>(ra, sA + buf * XP_SLAB + (2 * NRB * wave + j) * 512, src[j], 0);
    };
    auto dma_a = [&](int c, int buf) {
#pragma unroll
        for (int j = 0; j < 2 * NRB; ++j) dma_a_one(c, buf, j);
    };
    constexpr int KBLK = WFormat<WB>::kBlock;
    constexpr int NGC = 128 / G;  // groups per chunk
    // (descriptor bases from the wave-uniform column as a scalar: a base the
    // compiler takes for per-lane would turn every buffer load into a loop)
    const int ncolu = __builtin_amdgcn_readfirstlane(ncol0);
    const size_t wtile = (size_t)(ncolu >> 7) * kchunks * (8 * KBLK);  // the wave's 128-column tile
    const uint32_t boff = b_lane_offset<WB>((ncol0 & 127) + (lane & 31), lane);
    const uint32_t soff = (uint32_t)(lane & 31) * 2u;
    auto load_b = [&](Chunk* bs, int c) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(wf[b] + wtile + (size_t)c * (8 * KBLK), 0xffffffffu);
            const __amdgpu_buffer_rsrc_t rs =
                buffer_rsrc(S[b] + (size_t)c * NGC * ldS + ncolu, 0xffffffffu);
            load_b_chunk_buf<G, WB>(bs[b], rb, rs, boff, soff, ldS);
        }
    };
    // Software-pipelined k-steps: the A operands of step s + 1 are read from
    // LDS at the top of step s, fenced off from the rest of the step, so each
    // read has a whole step of MFMAs to land (left to itself the scheduler
    // reuses the A registers and waits on every read right before its MFMA);
    // the dequant of step s + 1 is interleaved with the MFMAs of step s (one
    // MFMA, then a share of the dequant VALU ops).
    auto read_a = [&](const uint16_t* sa, int s, half8 (&a)[NRB]) {
        const int kg = kgroup_of_step(s, h);
#pragma unroll
        for (int i = 0; i < NRB; ++i) {
            const int r = i * 32 + c32;
            a[i] = *reinterpret_cast<const half8*>(&sa[r * 128 + ((kg ^ (r & 15)) * 8)]);
        }
    };
    auto dequant_b = [&](const Chunk* bs, int s, half8 (&bf)[NB]) {
#pragma unroll
        for (int b = 0; b < NB; ++b) bf[b] = b_frag<1, G, WB>(bs[b], 0, s);
    };
    constexpr int NM = NB * NRB;                 // MFMAs per k-step
    constexpr int VB = WB == 4 ? 13 : 12;        // dequant VALU ops per B fragment
    constexpr int VPER = (VB * NB + NM - 1) / NM;  // dequant VALU ops placed after each MFMA
    // With a next chunk (tag NEXT: std::true_type), its A copies go out under
    // k-steps 0..3 instead of as one burst before the first step (the copies
    // of the workgroup's waves would queue at the address unit while the
    // waves stall at issue).  Each copy comes before the step's operand reads
    // in program order: the compiler keeps copies behind earlier reads of LDS
    // it cannot tell apart.  (The B register loads stay ahead of the steps:
    // placed among them, the compiler waited for them at once.)
    auto compute = [&](const uint16_t* sa, const Chunk* bs, auto next, int cn, int nbuf) {
        constexpr bool NEXT = decltype(next)::value;
        half8 a[NRB], bf[NB];
        read_a(sa, 0, a);
        dequant_b(bs, 0, bf);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            half8 an[NRB], bn[NB];
            __builtin_amdgcn_sched_barrier(0);
            if (s < 7) read_a(sa, s + 1, an);
            __builtin_amdgcn_sched_barrier(0);
            if (NEXT && s < 4) {
#pragma unroll
                for (int j = s * 2 * NRB / 4; j < (s + 1) * 2 * NRB / 4; ++j) dma_a_one(cn, nbuf, j);
            }
            if (s < 7) dequant_b(bs, s + 1, bn);
#pragma unroll
            for (int i = 0; i < NRB; ++i)
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[b][i] = mfma32(a[i], bf[b], acc[b][i]);
            if (s < 7) {
#pragma unroll
                for (int q = 0; q < NM; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    if (NEXT && q < 2 && s < 4) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // one copy
                    __builtin_amdgcn_sched_group_barrier(0x002, VPER, 0);  // VALU
                }
            }
#pragma unroll
            for (int i = 0; i < NRB; ++i) a[i] = an[i];
#pragma unroll
            for (int b = 0; b < NB; ++b) bf[b] = bn[b];
        }
    };

    // Chunk c runs from LDS buffer c % 2 and register set b[c % 2] while A
    // and B of chunk c + 1 are in flight into the other buffer and set.  A
    // trip ends with a full wait: while an LDS-DMA load is outstanding, every
    // wait the compiler itself places on a register load becomes a full
    // wait, so the B registers a trip consumes must be complete before it
    // issues the next DMA.  Two trips per loop pass keep the buffer indices
    // literals; the prefetch past the last chunk reloads the last chunk and
    // an odd chunk count leaves one chunk, already staged, for the tail.
    Chunk b0[NB], b1[NB];
    const int last = c1 - 1;
    load_b(b0, c0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 2 * NRB; ++j) {
        const int r = 4 * (2 * NRB * wave + j) + rsub;
        src[j] = (key_off(src[j]) + (uint32_t)((pos ^ (r & 15)) * 8)) * 2u;
    }
    dma_a(c0, 0);
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    auto trip = [&](int c, int abuf, const Chunk* bc, Chunk* bn) __attribute__((always_inline)) {
        const int cn = c + 1 < c1 ? c + 1 : last;
        load_b(bn, cn);
        __builtin_amdgcn_sched_barrier(0);
        compute(sA + abuf * XP_SLAB, bc, std::true_type{}, cn, abuf ^ 1);
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
    };
    // No branch inside a loop pass: loads used only on one side of a branch
    // are sunk into it by the compiler (the prefetch is lost).
    int c = c0;
    for (; c + 1 < c1; c += 2) {
        trip(c, 0, b0, b1);
        trip(c + 1, 1, b1, b0);
    }
    if (c < c1) compute(sA, b0, std::false_type{}, 0, 1);

    // The epilogue's lane-dependent addresses are formed from a copy of the
    // lane index that the compiler cannot trace back (an empty asm): hoisted
    // above the k loop, those addresses stayed live through it and were
    // spilled to scratch memory (16 registers per lane, 14.7 MB of scratch
    // writes per gate/up launch at the MoE layer's shape).
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    const int we = __builtin_amdgcn_readfirstlane(wave);
    if constexpr (MODE == 0) {
        // h = fp16(act(g) * u) of the pass's R rows x 128 columns goes through
        // an LDS tile (pitch 136 halfs) so that each row is stored as 16 whole
        // 16-byte pieces.  The barrier also drains every copy still in flight
        // into the buffers the tile reuses.
        constexpr int TP = 136;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NRB; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int row = i * 32 + acc_row(j, lane_e);
                const float g = acc[0][i][j], u = acc[NB - 1][i][j];
                if (row < R) sA[row * TP + we * 32 + (lane_e & 31)] = f2h(moe_act(g, act) * u);
            }
        __syncthreads();
        uint16_t* h = static_cast<uint16_t*>(out) + (size_t)slot0 * N + (ncol0 - wave * 32);
        for (int idx = we * 64 + lane_e; idx < R * 16; idx += 256) {
            const int row = idx >> 4, piece = idx & 15;
            __builtin_nontemporal_store(*reinterpret_cast<const uintx4*>(&sA[row * TP + piece * 8]),
                                        reinterpret_cast<uintx4*>(h + (size_t)row * N + piece * 8));
        }
    } else {
        const int col = __builtin_amdgcn_readfirstlane(ncol0 - wave * 32) + we * 32 + (lane_e & 31);
#pragma unroll
        for (int i = 0; i < NRB; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int row = i * 32 + acc_row(j, lane_e);
                if (row < R)
                    __builtin_nontemporal_store(acc[0][i][j], static_cast<float*>(out) + (size_t)(slot0 + row) * N + col);
            }
    }
}

}  // namespace qg
