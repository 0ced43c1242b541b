// Weight-only (int4 / int8) MFMA tile machinery shared by the prefill GEMMs,
// the mid-M split-K GEMM and the MoE grouped GEMMs: B operands straight from
// a fragment layout into registers, dequantized there; A operands from an
// LDS tile.
//
// Fragment layouts.  Both cut the weights into blocks of 16 columns x 128 k;
// eight blocks (128 columns) form a tile, and the tiles of a 128-column
// strip follow each other in k.  Inside a block, lane position
// p = cl + 16*q (cl = column in the block, q = 0..3) owns the 32 k
// c*128 + kk*32 + q*8 + j (kk = 0..3, j = 0..7):
//   WB = 4 (int4): 1 KB blocks; p owns the 16 bytes at p*16, one 32-bit word
//     per kk (nibble order in raw8 of common.hpp), stored v + 8;
//   WB = 8 (int8): 2 KB blocks; p owns the 16 bytes at h*1024 + p*16 for
//     h = 0, 1, holding kk = 2h and 2h + 1 as 8 bytes each (j ascending),
//     stored v + 128.
// So a wave reads a block with one (int4) or two (int8) fully coalesced
// 16-byte loads per lane, and both formats hand the MFMAs the same k order.
//
// v_mfma_f32_32x32x16_f16 operand mapping used here (wave64): lane l holds
// row (A) / column (B) l%32 and the 8 k of k-group half h = l/32.  Over one
// 128-k chunk, a lane loads the data of lane positions q = h and q = h+2 of
// its column's block, i.e. the k-groups kg = 4*kk + q (kk = 0..3): exactly
// the 8 k-groups of parity h.  MFMA step s (0..7) consumes k-group
// kg(s, h) = 4*(s%4) + 2*(s/4) + h on both operands, so A and B always agree
// on k.
#pragma once

#include "common.hpp"

namespace qg {

template <int WB>
struct WFormat;
// Raw fp16 value - weight of the raw operands (raw8 / raw8_u8): kBias0 for
// elements j % 4 < 2 of a k-step's eight, kBias1 for j % 4 >= 2.
template <>
struct WFormat<4> {
    static constexpr int kBlock = 1024;   // bytes per 16-column x 128-k block
    static constexpr int kPieces = 1;     // 16-byte pieces per lane position
    static constexpr float kBias0 = 1032.f;  // 1024 + offset 8
    static constexpr float kBias1 = 72.f;    // 64 + offset 8
};
template <>
struct WFormat<8> {
    static constexpr int kBlock = 2048;
    static constexpr int kPieces = 2;
    static constexpr float kBias0 = 1152.f;  // 1024 + offset 128
    static constexpr float kBias1 = 1152.f;
};

// Byte offset of block (strip = n / 16, chunk = k / 128).
template <int WB>
__device__ __forceinline__ size_t wblock_offset(int strip, int chunk, int kchunks) {
    constexpr int B = WFormat<WB>::kBlock;
    return ((size_t)(strip >> 3) * kchunks + chunk) * (8u * B) + (size_t)(strip & 7) * B;
}

// fp16 values 1024 + u of eight offset-binary bytes (u0..u3 of w0, then of
// w1): each v_perm_b32 puts two bytes under two 0x64 high bytes, exactly.
__device__ __forceinline__ half8 raw8_u8(uint32_t w0, uint32_t w1) {
    const uint32_t e = 0x64646464u;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 r = {__builtin_amdgcn_perm(w0, e, 0x00050004u), __builtin_amdgcn_perm(w0, e, 0x00070006u),
                     __builtin_amdgcn_perm(w1, e, 0x00050004u), __builtin_amdgcn_perm(w1, e, 0x00070006u)};
    return __builtin_bit_cast(half8, r);
}

// Raw fp16 values (1024 + u, j = 0..7) of k-step kk of one lane position,
// from its kPieces 16-byte pieces.
template <int WB>
__device__ __forceinline__ half8 raw_kstep(const uintx4* p, int kk) {
    if constexpr (WB == 4) {
        const uintx4 r = p[0];
        return raw8(kk == 0 ? r.x : kk == 1 ? r.y : kk == 2 ? r.z : r.w);
    } else {
        const uintx4 r = p[kk >> 1];
        return (kk & 1) ? raw8_u8(r.z, r.w) : raw8_u8(r.x, r.y);
    }
}

// fp16(v * s) of the eight weights: v = raw - bias exactly, then one fp16
// multiply by the column's scale.
template <int WB>
__device__ __forceinline__ half8 dequant_scaled(half8 raw, _Float16 s) {
    const _Float16 c0 = (_Float16)(-WFormat<WB>::kBias0), c1 = (_Float16)(-WFormat<WB>::kBias1);
    const half8 s8 = {s, s, s, s, s, s, s, s};
    return (raw + half8{c0, c0, c1, c1, c0, c0, c1, c1}) * s8;
}

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
template <int WTN, int G, int WB = 4>
struct BChunk {
    static constexpr int NG = 128 / G;
    static constexpr int P = WFormat<WB>::kPieces;
    uintx4 raw[WTN][2 * P];  // [q = h, q = h + 2] x pieces
    uint32_t sc[WTN][NG];    // fp16 bits, zero-extended (one register each)
};

// Fetch chunk c of columns ncol0 .. ncol0 + 32*WTN - 1 (ncol0 % 32 == 0).
// Scale row of group g of chunk c: (c * 128 / G + g) * ldS elements from S
// (ldS = N; ldS = 0 reads row 0 for every group: one scale per column).
// Scale reads past the last group row (gmax) or column (nmax) of a ragged
// shape read those instead: they only meet zero A values or padded columns
// that are never stored, and keep every read inside S.
template <int WTN, int G, int WB = 4>
__device__ __forceinline__ void load_b_chunk(BChunk<WTN, G, WB>& b, const uint8_t* __restrict__ wf,
                                             const uint16_t* __restrict__ S, int ldS, int kchunks,
                                             int c, int ncol0, int lane, int gmax, int nmax) {
    constexpr int P = WFormat<WB>::kPieces;
    const int h = lane >> 5;
#pragma unroll
    for (int t = 0; t < WTN; ++t) {
        const int n = ncol0 + 32 * t + (lane & 31);
        const uint8_t* blk = wf + wblock_offset<WB>(n >> 4, c, kchunks);
        const int cl = n & 15;
#pragma unroll
        for (int qi = 0; qi < 2; ++qi)
#pragma unroll
            for (int p = 0; p < P; ++p)
                b.raw[t][qi * P + p] =
                    ldg_nt(reinterpret_cast<const uintx4*>(blk + p * 1024 + (cl + 16 * (h + 2 * qi)) * 16));
#pragma unroll
        for (int g = 0; g < BChunk<WTN, G, WB>::NG; ++g) {
            const int gr = c * BChunk<WTN, G, WB>::NG + g;
            b.sc[t][g] = S[(size_t)(gr < gmax ? gr : gmax) * ldS + (n < nmax ? n : nmax)];
        }
    }
}

// Byte offset, inside one 128-column fragment tile (column nt = 0..127 of
// the tile), of the first piece this lane loads in a chunk (k-group parity
// h = lane / 32); piece (qi, p) adds 512 qi + 1024 p.
template <int WB>
__device__ __forceinline__ uint32_t b_lane_offset(int nt, int lane) {
    constexpr uint32_t B = WFormat<WB>::kBlock;
    return ((uint32_t)nt >> 4) * B + (((uint32_t)nt & 15u) + 16u * ((uint32_t)lane >> 5)) * 16u;
}

// load_b_chunk for one 32-column tile by buffer loads: rb is a descriptor
// from the chunk's fragment tile (8 blocks), rs one from the chunk's first
// scale row at the tile's first column; boff = b_lane_offset of the lane's
// column, soff = 2 * (its column - the first).  Group g's scale row is
// g * ldS elements further (a scalar offset), so a load takes no vector
// address arithmetic, and no offset exceeds one chunk of one tile.
template <int G, int WB>
__device__ __forceinline__ void load_b_chunk_buf(BChunk<1, G, WB>& b, __amdgpu_buffer_rsrc_t rb,
                                                 __amdgpu_buffer_rsrc_t rs, uint32_t boff, uint32_t soff,
                                                 int ldS) {
    constexpr int P = WFormat<WB>::kPieces;
    constexpr int NG = BChunk<1, G, WB>::NG;
#pragma unroll
    for (int qi = 0; qi < 2; ++qi)
#pragma unroll
        for (int p = 0; p < P; ++p)
            b.raw[0][qi * P + p] = __builtin_amdgcn_raw_buffer_load_b128(rb, boff + 512u * qi + 1024u * p, 0, 2);
#pragma unroll
    for (int g = 0; g < NG; ++g)
        b.sc[0][g] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff, (uint32_t)g * (uint32_t)ldS * 2u, 0);
}

template <int WTN, int G, int WB = 4>
__device__ __forceinline__ half8 b_frag(const BChunk<WTN, G, WB>& b, int t, int s) {
    constexpr int P = WFormat<WB>::kPieces;
    return dequant_scaled<WB>(raw_kstep<WB>(&b.raw[t][(s >> 2) * P], s & 3),
                              __builtin_bit_cast(_Float16, (uint16_t)b.sc[t][group_of_step<G>(s)]));
}

__device__ __forceinline__ floatx16 mfma32(half8 a, half8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator held in register j of lane l (column l%32).
__device__ __forceinline__ int acc_row(int j, int lane) {
    return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
}

}  // namespace qg
