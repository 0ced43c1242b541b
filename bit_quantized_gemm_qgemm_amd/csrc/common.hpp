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

// ---------------------------------------------------------------- int4 -> fp16
//
// Fragment-layout word: eight offset-binary nibbles u = v + 8 holding the
// weights v_0..v_7 of eight consecutive k of one column, at nibble positions
// [v0 v2 v4 v6 v1 v3 v5 v7] (bits 0-3 hold v0).  With the fp16 exponent of
// 1024 or'ed in, a nibble in bits 0-3 (16-19) reads as 1024 + u and a nibble
// in bits 4-7 (20-23) as 1024 + 16u, so two and-or ops plus one packed add
// or fma give two exact fp16 integers.
struct HalfPairs {
    half2v w01, w23, w45, w67;
};

__device__ __forceinline__ HalfPairs dequant_pairs(uint32_t d) {
    const uint32_t magic = 0x64006400u;
    const uint32_t d8 = d >> 8;
    const half2v p01 = __builtin_bit_cast(half2v, (d & 0x000f000fu) | magic);
    const half2v p23 = __builtin_bit_cast(half2v, (d & 0x00f000f0u) | magic);
    const half2v p45 = __builtin_bit_cast(half2v, (d8 & 0x000f000fu) | magic);
    const half2v p67 = __builtin_bit_cast(half2v, (d8 & 0x00f000f0u) | magic);
    const half2v off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const half2v sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const half2v off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
    HalfPairs r;
    r.w01 = p01 + off;
    r.w45 = p45 + off;
    r.w23 = __builtin_elementwise_fma(p23, sixteenth, off16);
    r.w67 = __builtin_elementwise_fma(p67, sixteenth, off16);
    return r;
}

// Concatenate four half2 into the 8-element MFMA operand (w0 .. w7).
// (Built with shufflevector: rewriting the elements of a 4 x u32 vector
// through __builtin_bit_cast was miscompiled by this toolchain.)
__device__ __forceinline__ half8 concat8(half2v a, half2v b, half2v c, half2v d) {
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
    const half4 lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    const half4 hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ half8 dequant8(uint32_t d) {
    const HalfPairs p = dequant_pairs(d);
    return concat8(p.w01, p.w23, p.w45, p.w67);
}

// Same, multiplied by a per-column scale (fp16 rounding of q*s).
__device__ __forceinline__ half8 dequant8_scaled(uint32_t d, half2v s2) {
    const HalfPairs p = dequant_pairs(d);
    return concat8(p.w01 * s2, p.w23 * s2, p.w45 * s2, p.w67 * s2);
}

// ---------------------------------------------------------------- fragment layout
//
// Weight block = 16 columns x 128 k = 1024 bytes; tile = 8 blocks (128 columns).
// Block (strip s = n/16, chunk c = k/128) starts at
//   ((s/8) * (K/128) + c) * 8192 + (s%8) * 1024.
// Inside a block, lane position p = cl + 16*q (cl = column in strip, q = 0..3)
// owns 16 bytes at p*16: word kk (0..3) holds k = c*128 + kk*32 + q*8 + j.
__device__ __forceinline__ size_t frag_block_offset(int strip, int chunk, int kchunks) {
    return ((size_t)(strip >> 3) * kchunks + chunk) * 8192u + (size_t)(strip & 7) * 1024u;
}

// ---------------------------------------------------------------- loads

template <typename T>
__device__ __forceinline__ T ldg_nt(const T* p) {
    return __builtin_nontemporal_load(p);
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
