// Shared device helpers for libqgemm (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "libqgemm.h"

namespace qg {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx16 __attribute__((ext_vector_type(16)));
typedef uint32_t uintx4 __attribute__((ext_vector_type(4)));
typedef uint32_t uintx2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- fp16 bits

__device__ __forceinline__ float h2f(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ uint16_t f2h(float f) {  // round to nearest even
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// fp16 of fl32(a * s): the fp32 product, then its fp16 rounding (two
// roundings, as the dequantizers define it).  Without the canonicalize
// between them the compiler fuses the multiply and the conversion into one
// mixed-precision FMA with a +0 addend, which rounds only once and returns +0
// where the product is -0.
__device__ __forceinline__ uint16_t f2h_of_product(float a, float s) {
    return f2h(__builtin_canonicalizef(a * s));
}

// ---------------------------------------------------------------- int4 -> fp16
//
// Fragment-layout word: eight offset-binary nibbles u = v + 8 holding the
// weights v_0..v_7 of eight consecutive k of one column, at nibble positions
// [v0 v2 v4 v6 v1 v3 v5 v7] (bits 0-3 hold v0), so that each fp16 pair of the
// result comes from one nibble of each 16-bit half of a word.  Masking two
// such nibbles and or-ing in a constant exponent gives the pair exactly: a
// nibble in bits 0-3 of a half under exponent 0x6400 (1024, unit spacing) is
// 1024 + u; a nibble in bits 4-7 under 0x5400 (64, spacing 1/16) is 64 + u.
// Elements 0, 1, 4, 5 of the result are therefore 1024 + u and elements
// 2, 3, 6, 7 are 64 + u:
//   (v0, v1) = d & 0x000f000f | 0x64006400,  (v2, v3) = d & 0x00f000f0 | 0x54005400,
//   and the same two with d >> 8 give (v4, v5) and (v6, v7).
// Five VALU ops per eight weights: each mask-and-or is one v_bitop3_b32
// (truth table 0xEA = (a & b) | c; written as & and | the compiler emits two
// ops, since gfx9 three-operand encodings take no literal constants).  All
// visible to the compiler (inline asm is avoided here: LLVM does not track
// MFMA hazards across it).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) {
    return __builtin_amdgcn_bitop3_b32(a, mask, bits, 0xEA);
}
__device__ __forceinline__ half8 raw8(uint32_t d) {
    const uint32_t d8 = d >> 8;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 r = {and_or(d, 0x000f000fu, 0x64006400u), and_or(d, 0x00f000f0u, 0x54005400u),
                     and_or(d8, 0x000f000fu, 0x64006400u), and_or(d8, 0x00f000f0u, 0x54005400u)};
    return __builtin_bit_cast(half8, r);
}

// Workgroups of a 1-D grid are dispatched round-robin over the eight XCDs
// (workgroup b runs on XCD b % 8).  xcd_contiguous(b, n) is a bijection of
// [0, n) that hands each XCD one contiguous run of work items, so items that
// share cache lines (neighbouring column strips reading one row of scales)
// meet in the same L2.
__device__ __forceinline__ int xcd_contiguous(int b, int n) {
    const int x = b & 7, i = b >> 3, q = n >> 3, r = n & 7;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

// Output tile (row tr, column tc) of workgroup b in a grid of mt x nt tiles.
// Each XCD takes a contiguous run of the tile order (xcd_contiguous), and the
// order walks bands of GM tile rows column by column, so the tiles of one XCD
// form a block of about GM rows by (its share / GM) columns: its workgroups
// share A row tiles and weight column tiles in that XCD's L2, and no XCD
// streams the whole weight matrix (at 16 x 16 tiles and GM = 4: a 4 x 8 block
// per XCD instead of 2 rows x all 16 columns).
__device__ __forceinline__ void xcd_tile(int b, int mt, int nt, int GM, int& tr, int& tc) {
    const int o = xcd_contiguous(b, mt * nt);
    const int g = o / (GM * nt), w = o - g * GM * nt;
    const int gs = mt - g * GM < GM ? mt - g * GM : GM;  // rows of this band (the last may be short)
    tr = g * GM + w % gs;
    tc = w / gs;
}

// ---------------------------------------------------------------- loads

// Wait until at most N vector-memory operations of this wave are outstanding
// (s_waitcnt with only the vector-memory counter constrained).  Loads,
// including global or buffer -> LDS DMA, complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until this wave's LDS (and scalar memory) operations are done.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Buffer resource over `bytes` bytes from `base` (raw dword access, no
// stride): a wave-uniform base for buffer loads, so a DMA's address is a
// scalar descriptor plus a per-lane 32-bit offset and a scalar offset, with
// no per-copy vector address arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Buffer -> LDS DMA: lane l's BYTES (4 or 16) from voff + soff go to
// lds + BYTES * l (lds wave-uniform).  Counted by vmcnt like any load.
template <int BYTES>
__device__ __forceinline__ void buffer_load_lds(__amdgpu_buffer_rsrc_t r, const void* lds, uint32_t voff,
                                                uint32_t soff) {
    static_assert(BYTES == 4 || BYTES == 16, "4- or 16-byte copies");
    // (the size must be a literal for the builtin, also in a template)
    auto* l = (__attribute__((address_space(3))) void*)lds;
    if constexpr (BYTES == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voff, soff, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 4, voff, soff, 0, 0);
}

template <typename T>
__device__ __forceinline__ T ldg_nt(const T* p) {
    return __builtin_nontemporal_load(p);
}

// ---- row reductions (int8 and fp8 quantizers)

// max(v, value of another lane of the same 16-lane row), the lane given by a
// DPP control (quad permutation or row mirror)
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
    return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                          CTRL, 0xf, 0xf, false)));
}

// Maximum over each aligned group of LPR lanes (4, 8, 16 or 64), delivered
// to every lane of the group, by register moves only: within a 16-lane row
// lane ^ 1, lane ^ 2 (quad permutations), then the half-row mirror (8 lanes)
// and the row mirror (16); a whole wave then combines its four row maxima
// read from lanes 0, 16, 32 and 48.  The maximum is exact, so the order does
// not matter.
template <int LPR>
__device__ __forceinline__ float group_max(float v) {
    static_assert(LPR == 4 || LPR == 8 || LPR == 16 || LPR == 64, "groups of 4, 8 or 16 lanes or whole waves");
    v = dpp_max<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v = dpp_max<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    if constexpr (LPR >= 8) v = dpp_max<0x141>(v);  // row_half_mirror
    if constexpr (LPR >= 16) v = dpp_max<0x140>(v);  // row_mirror
    if constexpr (LPR == 64) {
        const int b = __builtin_bit_cast(int, v);
        const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
        const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
        const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
        const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
        v = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
    }
    return v;
}

__device__ __forceinline__ float absmax8(uintx4 v) {
    // max |x| of eight fp16 values: sign bits cleared, fp16 maxima of the
    // pairs (exact, and the order of fp16 values is that of their fp32
    // conversions), then the two halves in fp32
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 a0 = __builtin_bit_cast(h2, v.x & 0x7fff7fffu), a1 = __builtin_bit_cast(h2, v.y & 0x7fff7fffu);
    const h2 a2 = __builtin_bit_cast(h2, v.z & 0x7fff7fffu), a3 = __builtin_bit_cast(h2, v.w & 0x7fff7fffu);
    const h2 m = __builtin_elementwise_max(__builtin_elementwise_max(a0, a1), __builtin_elementwise_max(a2, a3));
    return fmaxf(0.0f, fmaxf((float)m[0], (float)m[1]));
}

// ---- accumulator tiles to row-major pieces (GEMM epilogues)
//
// In a 32x32 MFMA accumulator a lane quad (lanes 4k .. 4k+3, lane q holding
// column 4k + q) holds, per group of four registers, four consecutive rows
// r = 0..3.  A 4x4 transpose inside the quad (DPP quad permutations and byte
// permutes) gives lane q row q of the quad's four columns, so a lane can
// store four adjacent outputs of one row at once.

// 8-bit values: d holds row r in byte r; the result holds column c in byte c.
__device__ __forceinline__ uint32_t quad_rows_u8(uint32_t d, int lane) {
    const uint32_t sel1 = (lane & 1) ? 0x03070105u : 0x06020400u;  // with lane ^ 1
    const uint32_t sel2 = (lane & 2) ? 0x03020706u : 0x05040100u;  // with lane ^ 2
    const uint32_t x = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)d, 0xB1, 0xf, 0xf, false);
    const uint32_t d1 = __builtin_amdgcn_perm(x, d, sel1);
    const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)d1, 0x4E, 0xf, 0xf, false);
    return __builtin_amdgcn_perm(y, d1, sel2);
}

// 16-bit values: d0 holds rows 0 (low half) and 1, d1 rows 2 and 3; on
// return e0 holds columns 0 and 1, e1 columns 2 and 3, of row q.
__device__ __forceinline__ void quad_rows_u16(uint32_t d0, uint32_t d1, int lane, uint32_t& e0, uint32_t& e1) {
    const uint32_t sel = (lane & 1) ? 0x03020706u : 0x05040100u;  // with lane ^ 1
    const uint32_t p0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)d0, 0xB1, 0xf, 0xf, false);
    const uint32_t p1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)d1, 0xB1, 0xf, 0xf, false);
    const uint32_t s0 = __builtin_amdgcn_perm(p0, d0, sel);
    const uint32_t s1 = __builtin_amdgcn_perm(p1, d1, sel);
    const uint32_t u0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s0, 0x4E, 0xf, 0xf, false);
    const uint32_t u1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s1, 0x4E, 0xf, 0xf, false);
    e0 = (lane & 2) ? u1 : s0;
    e1 = (lane & 2) ? s1 : u0;
}

}  // namespace qg

// Host-side helpers shared by the entry points.
namespace qgh {

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline int32_t launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? QGEMM_OK : QGEMM_HIP_ERROR;
}

}  // namespace qgh
