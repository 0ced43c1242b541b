// W4A16 MFMA tile machinery shared by the prefill GEMM and the MoE grouped
// GEMMs: B operands straight from the fragment layout into registers,
// dequantized there; A operands from an LDS tile.
//
// v_mfma_f32_32x32x16_f16 operand mapping used here (wave64): lane l holds
// row (A) / column (B) l%32 and the 8 k of k-group half h = l/32.  Over one
// 128-k chunk, a lane loads two 16-byte pieces of its column's fragment
// block, lane positions q = h and q = h+2, i.e. the k-groups
// kg = 4*kk + q (kk = 0..3): exactly the 8 k-groups of parity h.  MFMA step
// s (0..7) consumes k-group kg(s, h) = 4*(s%4) + 2*(s/4) + h on both
// operands, so A and B always agree on k.
#pragma once

#include "common.hpp"

namespace qg {

__device__ __forceinline__ int kgroup_of_step(int s, int h) { return 4 * (s & 3) + 2 * (s >> 2) + h; }

// Group index (inside a 128-k chunk) of the k-group used at step s.
template <int G>
__device__ __forceinline__ int group_of_step(int s) {
    if constexpr (G == 128) return 0;
    else if constexpr (G == 64) return (s & 3) >> 1;
    else return s & 3;  // G == 32
}

// Raw B data of WTN 32-column MFMA tiles for one 128-k chunk, plus scales.
// Scales stay scalar until use: nothing consumes a load right after it is
// issued, so the loads of a prefetched chunk are never waited for early.
template <int WTN, int G>
struct BChunk {
    static constexpr int NG = 128 / G;
    uintx4 raw[WTN][2];
    uint32_t sc[WTN][NG];  // fp16 bits, zero-extended (one register each)
};

// Fetch the chunk c of columns ncol0 .. ncol0 + 32*WTN - 1 (ncol0 % 32 == 0).
template <int WTN, int G>
__device__ __forceinline__ void load_b_chunk(BChunk<WTN, G>& b, const uint8_t* __restrict__ wf,
                                             const uint16_t* __restrict__ S, int N, int kchunks,
                                             int c, int ncol0, int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int t = 0; t < WTN; ++t) {
        const int n = ncol0 + 32 * t + (lane & 31);
        const uint8_t* blk = wf + frag_block_offset(n >> 4, c, kchunks);
        const int cl = n & 15;
        b.raw[t][0] = ldg_nt(reinterpret_cast<const uintx4*>(blk + (cl + 16 * h) * 16));
        b.raw[t][1] = ldg_nt(reinterpret_cast<const uintx4*>(blk + (cl + 16 * (h + 2)) * 16));
#pragma unroll
        for (int g = 0; g < BChunk<WTN, G>::NG; ++g) {
            b.sc[t][g] = S[(size_t)(c * BChunk<WTN, G>::NG + g) * N + n];
        }
    }
}

template <int WTN, int G>
__device__ __forceinline__ half8 b_frag(const BChunk<WTN, G>& b, int t, int s) {
    const uintx4 r = b.raw[t][s >> 2];
    const int kk = s & 3;
    const uint32_t d = kk == 0 ? r.x : kk == 1 ? r.y : kk == 2 ? r.z : r.w;
    return dequant8_scaled(d, __builtin_bit_cast(_Float16, (uint16_t)b.sc[t][group_of_step<G>(s)]));
}

__device__ __forceinline__ floatx16 mfma32(half8 a, half8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator held in register j of lane l (column l%32).
__device__ __forceinline__ int acc_row(int j, int lane) {
    return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
}

}  // namespace qg
