// W8A8 int8 GEMM with a fused requantizing epilogue.
//
// INT8 cross-modal MHA TensorRT plugin interview page: knowledge point 1
// (int8 operands, integer accumulation, then fp32 and requantization to
// int8), knowledge point 2 (per-channel weight / per-token activation scales;
// after the int8 GEMM: rescale + bias + GELU, then requantize), answer step 3
// (a per-tensor output scale and an fp16 bias applied after the GEMM).
//
// A [M][K] and W [N][K] are both K-contiguous.  128x128 output tiles, four
// waves of 64x64, each a 2x2 grid of v_mfma_i32_32x32x32_i8; A and W tiles
// (128 k deep) double-buffered through LDS.  The epilogue runs on the int32
// accumulators in registers and is the bit-exact fp32 sequence of the header
// (no contraction; division correctly rounded).
#include <type_traits>

#include "common.hpp"

namespace {

using namespace qg;

constexpr int BM = 128, BN = 128, BK = 128, LDK = 144;  // LDS row: 128 bytes + 16 pad

__device__ __forceinline__ intx16 mfma_i8(intx4 a, intx4 b, intx16 c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// Abramowitz & Stegun 7.1.28 erf inside GELU, fixed fp32 sequence.
__device__ __forceinline__ float gelu28(float y) {
    const float a1 = 0.0705230784f, a2 = 0.0422820123f, a3 = 0.0092705272f;
    const float a4 = 0.0001520143f, a5 = 0.0002765672f, a6 = 0.0000430638f;
    const float u = y * 0.70710678f;
    const float a = fabsf(u);
    float p = __builtin_fmaf(a, a6, a5);
    p = __builtin_fmaf(a, p, a4);
    p = __builtin_fmaf(a, p, a3);
    p = __builtin_fmaf(a, p, a2);
    p = __builtin_fmaf(a, p, a1);
    p = __builtin_fmaf(a, p, 1.0f);
    p = p * p;
    p = p * p;
    p = p * p;
    p = p * p;
    // 1 - 1/p with the correctly rounded quotient, without a division: for
    // every finite float p >= 1, v_rcp_f32 followed by one fused Newton step
    // gives 1 - r equal to 1 - 1/p bit for bit (checked on gfx950 over all of
    // them; on [1, 2^25] r itself is the correctly rounded 1/p, above it both
    // differences round to 1).  p = +inf (1/p = 0) is clamped to the largest
    // float, which gives the same 1.
    p = fminf(p, 3.40282347e+38f);
    const float r0 = __builtin_amdgcn_rcpf(p);
    const float r = __builtin_fmaf(__builtin_fmaf(-p, r0, 1.0f), r0, r0);
    float e = 1.0f - r;
    e = __builtin_copysignf(e, u);
    return (0.5f * y) * (1.0f + e);
}

// The code in the low byte of the result.  clamp(rne(v), -127, 127) equals
// rne(clamp(v, -127, 127)) (the bounds are integers), and adding 1.5 * 2^23
// to a value of magnitude at most 127 lands in [2^23, 2^24), where the fp32
// spacing is 1: the addition rounds to nearest, ties to even, and leaves
// 0x4B400000 + rne(v) in the bits, whose low byte is the two's-complement code.
__device__ __forceinline__ uint32_t requant_bits(int32_t acc, float sa, float sw, float bias,
                                                 float out_mult, uint32_t flags) {
    float t = (float)acc;
    t = t * sa;
    t = t * sw;
    if (flags & QGEMM_EPI_BIAS) t = t + bias;
    const float g = (flags & QGEMM_EPI_GELU) ? gelu28(t) : t;
    const float v = fminf(fmaxf(g * out_mult, -127.0f), 127.0f);
    return __builtin_bit_cast(uint32_t, v + 12582912.0f);
}

__device__ __forceinline__ int8_t requant(int32_t acc, float sa, float sw, float bias,
                                          float out_mult, uint32_t flags) {
    return (int8_t)(requant_bits(acc, sa, sw, bias, out_mult, flags) & 0xffu);
}

// Runs f with the epilogue flags as a compile-time constant, so the per
// element code has no branches and the compiler can interleave independent
// elements (with run-time flags every element's GELU is a basic block of its
// own, a chain of dependent fp32 operations).
template <typename F>
__device__ __forceinline__ void with_flags(uint32_t flags, F&& f) {
    switch (flags & (QGEMM_EPI_BIAS | QGEMM_EPI_GELU)) {
        case 0: f(std::integral_constant<uint32_t, 0>{}); break;
        case QGEMM_EPI_BIAS: f(std::integral_constant<uint32_t, QGEMM_EPI_BIAS>{}); break;
        case QGEMM_EPI_GELU: f(std::integral_constant<uint32_t, QGEMM_EPI_GELU>{}); break;
        default: f(std::integral_constant<uint32_t, QGEMM_EPI_BIAS | QGEMM_EPI_GELU>{}); break;
    }
}

__global__ __launch_bounds__(256, 2) void w8a8_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ W, const float* __restrict__ sa,
    const float* __restrict__ sw, const uint16_t* __restrict__ bias, float out_mult, uint32_t flags,
    int8_t* __restrict__ Y, int32_t* __restrict__ acc_out, int M, int N, int K) {
    __shared__ __attribute__((aligned(16))) int8_t sA[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) int8_t sW[2][BN * LDK];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int h = lane >> 5, c32 = lane & 31;
    const int kchunks = K / BK;

    intx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[i][t][j] = 0;

    // each tile: 128 rows x 128 bytes = 1024 pieces of 16 bytes, 4 per thread
    uintx4 ra[4], rw[4];
    auto load = [&](int c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i, row = idx >> 3, col = idx & 7;
            const int gm = m0 + row;
            // rows >= M repeat row M-1 (unconditional load; those rows are not stored)
            ra[i] = *reinterpret_cast<const uintx4*>(A + (size_t)(gm < M ? gm : M - 1) * K + c * BK + col * 16);
            rw[i] = *reinterpret_cast<const uintx4*>(W + (size_t)(n0 + row) * K + c * BK + col * 16);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i, row = idx >> 3, col = idx & 7;
            *reinterpret_cast<uintx4*>(&sA[buf][row * LDK + col * 16]) = ra[i];
            *reinterpret_cast<uintx4*>(&sW[buf][row * LDK + col * 16]) = rw[i];
        }
    };

    auto compute = [&](int buf) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            // step s covers k = 32 s .. 32 s + 31; lane half h holds 16 of them
            const int koff = 32 * s + 16 * h;
            intx4 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const intx4*>(&sA[buf][(wm * 64 + i * 32 + c32) * LDK + koff]);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                b[t] = *reinterpret_cast<const intx4*>(&sW[buf][(wn * 64 + t * 32 + c32) * LDK + koff]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int t = 0; t < 2; ++t) acc[i][t] = mfma_i8(a[i], b[t], acc[i][t]);
        }
    };

    // Prefetch of the next chunk into registers, unconditional (the index is
    // clamped) and kept ahead of the compute by scheduling barriers: a load
    // under a branch makes the compiler wait for it at the join, and a load
    // sunk next to its LDS store would not overlap the MFMAs.  The last
    // iteration refills the idle buffer with a chunk nobody reads.
    load(0);
    store(0);
    __syncthreads();
    for (int c = 0; c < kchunks; ++c) {
        const int buf = c & 1;
        load(c + 1 < kchunks ? c + 1 : c);
        __builtin_amdgcn_sched_barrier(0);
        compute(buf);
        __builtin_amdgcn_sched_barrier(0);
        store(buf ^ 1);
        __syncthreads();
    }

    with_flags(flags, [&](auto fl) {
        constexpr uint32_t FL = decltype(fl)::value;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int col = n0 + wn * 64 + t * 32 + c32;
            const float swv = sw[col];
            const float bv = (FL & QGEMM_EPI_BIAS) ? h2f(bias[col]) : 0.0f;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int row = m0 + wm * 64 + i * 32 + 8 * (j >> 2) + 4 * h + (j & 3);
                    if (row < M) {
                        const int32_t a = acc[i][t][j];
                        if (acc_out) acc_out[(size_t)row * N + col] = a;
                        Y[(size_t)row * N + col] = requant(a, sa[row], swv, bv, out_mult, FL);
                    }
                }
            }
        }
    });
}

// Large shapes (M >= 256, N % 256 == 0): 256x256 output tiles, eight waves
// (two per SIMD) of 128x64 (4 x 2 v_mfma_i32_32x32x32_i8 tiles, 128
// accumulators per lane); one workgroup per CU at M = N = 4096.  Per 128-k
// chunk a workgroup stages 32 KB of A and 32 KB of W by buffer -> LDS DMA
// (two buffers each, one array, compile-time offsets), so each operand byte
// fetched feeds 256 output columns or rows (a 128x128 tile fetches twice as
// much per MFMA).  A DMA instruction fills 1 KB = 8 rows of 128 bytes in lane
// order; the lane that fills position pos of row r fetches piece
// pos ^ ((r >> 1) & 7), so the MFMA operand reads (32 rows at one 16-byte
// piece) are free of bank conflicts.  The k-steps are software-pipelined:
// the operand reads of step s + 1 are interleaved with the MFMAs of step s.
constexpr int LB = 256;

__global__ __launch_bounds__(512, 1) void w8a8_large_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ W, const float* __restrict__ sa,
    const float* __restrict__ sw, const uint16_t* __restrict__ bias, float out_mult, uint32_t flags,
    int8_t* __restrict__ Y, int32_t* __restrict__ acc_out, int M, int N, int K) {
    constexpr int SL = LB * 128;  // bytes per operand buffer
    // A0, A1, W0, W1, then the activation scales of the tile's rows
    __shared__ __attribute__((aligned(1024))) int8_t lds[4 * SL + LB * 4];
    float* const s_sa = reinterpret_cast<float*>(lds + 4 * SL);
    // (the wave index from threadIdx.x: its known range lets the compiler
    // tell the copies' LDS targets from the buffer being read)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    // tile of workgroup L: each XCD (workgroups are dealt round-robin by id)
    // owns a block of tiles sharing A rows and W columns in its L2
    const int mtiles = (M + LB - 1) / LB;
    int tr, tc;
    xcd_tile(blockIdx.x, mtiles, N / LB, 4, tr, tc);
    const int m0 = tr * LB, n0 = tc * LB;
    const int kchunks = K / 128, last = kchunks - 1;
    const int h = lane >> 5, c32 = lane & 31;

    intx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[i][t][j] = 0;

    // wave w issues DMA instructions 4w .. 4w + 3 of each operand tile; rows
    // past the last valid one repeat it (their results are never stored).
    // Sources are 32-bit byte offsets from a wave-uniform base (rows * K <
    // 2^32 is checked at launch).
    const int rsub = lane >> 3, pos = lane & 7;
    uint32_t offa[4], offw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 8 * (4 * wave + j) + rsub;
        const uint32_t piece = (uint32_t)((pos ^ ((r >> 1) & 7)) * 16);
        offa[j] = (uint32_t)(m0 + r < M ? m0 + r : M - 1) * (uint32_t)K + piece;
        offw[j] = (uint32_t)(n0 + r) * (uint32_t)K + piece;
    }
    // Buffer -> LDS copies (wave-uniform descriptors over A and W, the chunk's
    // k offset as a scalar offset: no vector address arithmetic per copy).
    // Copy i of a chunk: i < 4 A, else W.
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(A, 0xffffffffu), rw = buffer_rsrc(W, 0xffffffffu);
    auto dma_one = [&](int c, int buf, int i) __attribute__((always_inline)) {
        if (i < 4) buffer_load_lds<16>(ra, lds + buf * SL + (4 * wave + i) * 1024, offa[i], (uint32_t)c * 128u);
        else buffer_load_lds<16>(rw, lds + (2 + buf) * SL + (4 * wave + i - 4) * 1024, offw[i - 4], (uint32_t)c * 128u);
    };
    auto operands = [&](const int8_t* ab, const int8_t* wb, int s, intx4 (&a)[4], intx4 (&b)[2]) {
        const int p = 2 * s + h;  // 16-byte piece of k = 32 s + 16 h .. + 15
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 128 + i * 32 + c32;
            a[i] = *reinterpret_cast<const intx4*>(ab + r * 128 + ((p ^ ((r >> 1) & 7)) * 16));
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int r = wn * 64 + t * 32 + c32;
            b[t] = *reinterpret_cast<const intx4*>(wb + r * 128 + ((p ^ ((r >> 1) & 7)) * 16));
        }
    };
    // The next chunk's eight copies go out three, three and two per k-step
    // under the MFMAs of steps 0..2 (issued as one burst, the copies of the
    // eight waves queue at the address unit and the waves stall at issue).
    auto compute = [&](const int8_t* ab, const int8_t* wb, int cn, int nbuf) {
        intx4 a[4], b[2];
        operands(ab, wb, 0, a, b);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            intx4 an[4], bn[2];
            if (s < 3) {
#pragma unroll
                for (int i = s * 8 / 3; i < (s + 1) * 8 / 3; ++i) dma_one(cn, nbuf, i);
            }
            if (s < 3) operands(ab, wb, s + 1, an, bn);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int t = 0; t < 2; ++t) acc[i][t] = mfma_i8(a[i], b[t], acc[i][t]);
            if (s < 3) {
#pragma unroll
                for (int q = 0; q < 6; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                    if (q < 3) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // one copy
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = an[i];
#pragma unroll
            for (int t = 0; t < 2; ++t) b[t] = bn[t];
        }
    };

    // the tile's 256 activation scales (rows >= M repeat row M - 1) go to LDS
    // with the first chunk, so the epilogue reads each lane's four
    // consecutive rows with one LDS read instead of four clamped gathers
    const int srow = m0 + (int)(threadIdx.x & (LB - 1));
    const float sa_row = sa[srow < M ? srow : M - 1];
#pragma unroll
    for (int i = 0; i < 8; ++i) dma_one(0, 0, i);
    wait_vmcnt<0>();
    if (threadIdx.x < LB) s_sa[threadIdx.x] = sa_row;
    __syncthreads();
    // one trip per chunk: DMA of chunk c + 1 into the idle buffers, MFMAs on
    // chunk c, then wait for this wave's DMA and a bare barrier (buffer
    // indices are literals at every call so that the compiler can tell the
    // DMA targets from the buffers being read)
    auto trip = [&](int c, int buf) __attribute__((always_inline)) {
        const int cn = c + 1 < last ? c + 1 : last;
        compute(lds + buf * SL, lds + (2 + buf) * SL, cn, buf ^ 1);
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
    };
    for (int c = 0; c < kchunks; c += 2) {
        trip(c, 0);
        if (c + 1 < kchunks) trip(c + 1, 1);
    }

    // ---- epilogue.  The codes of the 256x256 tile go through LDS so that Y
    // is written in whole 16-byte row pieces: a lane holds four consecutive
    // rows of one column per register group; a 4x4 byte transpose inside each
    // lane quad (two DPP moves, two byte permutes) gives each lane four
    // consecutive columns of one row, stored as one dword into a row-major
    // LDS tile (pitch 288 bytes: the 32 dwords of a half-wave fall in 32
    // distinct banks).  The operand stages are free: the last trip ended with
    // every wave's DMA drained and a barrier.
    if (acc_out) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int row = m0 + wm * 128 + i * 32 + 8 * (j >> 2) + 4 * h + (j & 3);
                    if (row < M) acc_out[(size_t)row * N + n0 + wn * 64 + t * 32 + c32] = acc[i][t][j];
                }
    }
    constexpr int EPW = 72;  // LDS tile pitch in dwords (256 bytes + 32)
    uint32_t* stile = reinterpret_cast<uint32_t*>(lds);
    const int q = lane & 3;
    with_flags(flags, [&](auto fl) {
        constexpr uint32_t FL = decltype(fl)::value;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int col = n0 + wn * 64 + t * 32 + c32;
            const float swv = sw[col];
            const float bv = (FL & QGEMM_EPI_BIAS) ? h2f(bias[col]) : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int r0 = wm * 128 + i * 32 + 8 * g + 4 * h;  // tile row of register 4g
                    const floatx4 sa4 = *reinterpret_cast<const floatx4*>(&s_sa[r0]);
                    uint32_t fb[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) fb[r] = requant_bits(acc[i][t][4 * g + r], sa4[r], swv, bv, out_mult, FL);
                    // the four codes' low bytes, rows r = 0..3 in bytes 0..3
                    const uint32_t d = __builtin_amdgcn_perm(fb[1], fb[0], 0x0c0c0400u) |
                                       __builtin_amdgcn_perm(fb[3], fb[2], 0x04000c0cu);
                    stile[(r0 + q) * EPW + wn * 16 + t * 8 + (c32 >> 2)] = quad_rows_u8(d, lane);
                }
            }
        }
    });
    __syncthreads();
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int idx = tid + 512 * p, row = idx >> 4, piece = idx & 15;
        if (m0 + row < M)  // non-temporal: Y is not read again here
            __builtin_nontemporal_store(*reinterpret_cast<const uintx4*>(&stile[row * EPW + piece * 4]),
                                        reinterpret_cast<uintx4*>(Y + (size_t)(m0 + row) * N + n0 + piece * 16));
    }
}

}  // namespace

extern "C" int32_t qgemm_w8a8_epilogue(const int8_t* A, const int8_t* W, const float* a_scale,
                                       const float* w_scale, const uint16_t* bias, float out_mult,
                                       uint32_t flags, int8_t* Y, int32_t* acc_out, int32_t M,
                                       int32_t N, int32_t K, void* stream) {
    if (M < 0 || N < 0 || K < 0) return QGEMM_BAD_SHAPE;
    if (M == 0) return QGEMM_OK;
    if (!A || !W || !a_scale || !w_scale || !Y) return QGEMM_NULL_PTR;
    if ((flags & QGEMM_EPI_BIAS) && !bias) return QGEMM_NULL_PTR;
    if (flags & ~(QGEMM_EPI_BIAS | QGEMM_EPI_GELU)) return QGEMM_UNSUPPORTED;
    if (N == 0 || K == 0 || N % BN != 0 || K % BK != 0 || K > 133120) return QGEMM_UNSUPPORTED;
    if (!qgh::aligned(A, 16) || !qgh::aligned(W, 16) || !qgh::aligned(Y, 16) ||
        !qgh::aligned(a_scale, 4) || !qgh::aligned(w_scale, 4) || (bias && !qgh::aligned(bias, 2)) ||
        (acc_out && !qgh::aligned(acc_out, 16)))
        return QGEMM_MISALIGNED;
    if (M >= LB && N % LB == 0 && (size_t)M * K < ((size_t)1 << 32) && (size_t)N * K < ((size_t)1 << 32)) {
        dim3 grid((N / LB) * ((M + LB - 1) / LB));
        hipLaunchKernelGGL(w8a8_large_kernel, grid, dim3(512), 0, (hipStream_t)stream, A, W, a_scale,
                           w_scale, bias, out_mult, flags, Y, acc_out, (int)M, (int)N, (int)K);
    } else {
        dim3 grid(N / BN, (M + BM - 1) / BM);
        hipLaunchKernelGGL(w8a8_kernel, grid, dim3(256), 0, (hipStream_t)stream, A, W, a_scale,
                           w_scale, bias, out_mult, flags, Y, acc_out, (int)M, (int)N, (int)K);
    }
    return qgh::launch_status();
}
