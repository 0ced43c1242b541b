// FP8 (OCP E4M3) path: symmetric quantization, dequantization and an FP8
// GEMM with fp16 output.
//
// FP8-vs-INT8 article for TensorRT-LLM (itzkxy.com): the E4M3 format for the
// GEMMs and the KV cache, per-tensor scaling factors derived from the
// activation A-max, FP8 operands fed straight to the matrix units.
//
// Encoding: v_cvt_pk_fp8_f32 on gfx950 produces OCP E4M3 (E4M3FN: bias 7,
// largest finite 448, S.1111.111 = NaN) and rounds to nearest even; it turns
// magnitudes above 464 into NaN, so every value is clamped to [-448, 448]
// first (the clamp is exact).  The quantizer's arithmetic is the fp32
// sequence of the header: m = 448 / amax, s = amax / 448,
// code = e4m3(clamp(x * m)) -- correctly rounded division, no contraction.
//
// GEMM: v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32 accumulation).  Lane l
// holds row (A) / column (B) l % 32 and 32 consecutive k bytes of a 64-k
// step, the same (lane half, byte) -> k assignment for both operands, so the
// K-contiguous rows of A [M][K] and W [N][K] feed it directly.  The tiling is
// that of the int8 W8A8 kernel: 256x256 output tiles, eight waves (two per
// SIMD) of 128x64, operands by buffer -> LDS DMA (two buffers each, one LDS
// array, compile-time offsets), XOR-swizzled 16-byte pieces, software-
// pipelined steps.
#include "common.hpp"

namespace {

using namespace qg;

typedef int intx8 __attribute__((ext_vector_type(8)));

// four fp16 values (two words) times mult -> four E4M3 codes in one word.
// fl32(x * mult) as fma(x, mult, +0) (v_fma_mix_f32 reads the fp16 operand in
// place): the same single rounding, except that a zero product comes out +0
// where x * mult is -0 for negative x; since mult > 0 the code's sign is that
// of x, so the sign bits of the four inputs are ORed into the codes (one byte
// permute gathers them), which restores -0 as 0x80.  smask (sign_mask) keeps
// them out when mult is 0: a row (or tensor) whose maximum is 0 gets code
// 0x00 for every value, -0 included.  With |x| <= amax and
// mult = fl32(448 / amax) the product is at most 448 (1 + 2^-24) in
// magnitude, which the round-to-nearest-even conversion maps to +-448 (the
// next value up would be 480), so no clamp to [-448, 448] is needed for
// finite input.
__device__ __forceinline__ uint32_t sign_mask(float mult) { return mult > 0.0f ? 0x80808080u : 0u; }

__device__ __forceinline__ uint32_t fp8x4(uint32_t h01, uint32_t h23, float mult, uint32_t smask) {
    float x[4] = {h2f(h01 & 0xffffu), h2f(h01 >> 16), h2f(h23 & 0xffffu), h2f(h23 >> 16)};
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __builtin_fmaf(x[i], mult, 0.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);  // bytes 0, 1
    w = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);       // bytes 2, 3
    // bytes 1 and 3 of each input word hold the fp16 sign bits, in bit 7
    const uint32_t sgn = __builtin_amdgcn_perm(h23, h01, 0x07050301u) & smask;
    return (uint32_t)w | sgn;
}

__device__ __forceinline__ uintx2 fp8x8(uintx4 v, float mult, uint32_t smask) {
    return uintx2{fp8x4(v.x, v.y, mult, smask), fp8x4(v.z, v.w, mult, smask)};
}

// ------------------------------------------------------------------ per-row quant

// Rows held in registers: each of LPR lanes holds CPL chunks of 8 values;
// the row's amax by DPP moves, codes written from the same registers.
// FULL: cols == LPR * CPL * 8, so every chunk is in the row.
template <int LPR, int CPL, bool FULL>
__global__ __launch_bounds__(256) void fp8_quant_rows_kernel(const uint16_t* __restrict__ X,
                                                             uint8_t* __restrict__ Q,
                                                             float* __restrict__ S, int rows,
                                                             int cols) {
    constexpr int RPB = 256 / LPR;  // rows per block
    const int lane = threadIdx.x % LPR;
    const int row = blockIdx.x * RPB + threadIdx.x / LPR;
    const bool live = row < rows;
    const int nchunk = cols / 8;
    const uint16_t* x = X + (size_t)(live ? row : 0) * cols;
    // unconditional loads (a chunk past the row end reads chunk 0 and is zeroed)
    uintx4 v[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + i * LPR;
        v[i] = ldg_nt(reinterpret_cast<const uintx4*>(x) + (FULL || c < nchunk ? c : 0));
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        if (!FULL && lane + i * LPR >= nchunk) v[i] = uintx4{0, 0, 0, 0};
        amax = fmaxf(amax, absmax8(v[i]));
    }
    amax = group_max<LPR>(amax);
    if (!live) return;
    const float mult = amax > 0.0f ? 448.0f / amax : 0.0f;
    const uint32_t smask = sign_mask(mult);
    if (lane == 0) S[row] = amax > 0.0f ? amax / 448.0f : 0.0f;
    uintx2* q = reinterpret_cast<uintx2*>(Q + (size_t)row * cols);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + i * LPR;
        if (FULL || c < nchunk) q[c] = fp8x8(v[i], mult, smask);
    }
}

// ------------------------------------------------------------------ per-tensor quant

// Three stream-ordered launches, no atomics and no memset (the sequence may
// be graph-captured): (1) each of P <= 256 blocks writes the maximum |x| of
// its share of X as an fp32 value into bytes 4b .. 4b + 3 of Q (Q has
// 8 * nchunk >= 4 P bytes); (2) every block takes the maximum of those P
// values (exact, so the order is free) and writes the codes of every chunk
// past the first ceil(P / 2), which hold the partial maxima; (3) one block
// takes the maximum again, writes the codes of those first chunks and the
// scale s = amax / 448.  (Before: a scale slot zeroed by a one-thread
// kernel and raised by one integer atomic max per block, serialized at
// about 10 ns each, then a one-thread kernel turning it into s.)
constexpr int AMAX_BLOCKS = 256;
constexpr int AMAX_LD = 8;

__global__ __launch_bounds__(256) void fp8_amax_kernel(const uint16_t* __restrict__ X, size_t nchunk,
                                                       float* __restrict__ part) {
    __shared__ float red[4];
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const uintx4* x = reinterpret_cast<const uintx4*>(X);
    float amax = 0.0f;
    size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; c + (AMAX_LD - 1) * stride < nchunk; c += AMAX_LD * stride) {
        uintx4 v[AMAX_LD];
#pragma unroll
        for (int i = 0; i < AMAX_LD; ++i) v[i] = ldg_nt(x + c + i * stride);
#pragma unroll
        for (int i = 0; i < AMAX_LD; ++i) amax = fmaxf(amax, absmax8(v[i]));
    }
    for (; c < nchunk; c += stride) amax = fmaxf(amax, absmax8(ldg_nt(x + c)));
    amax = group_max<64>(amax);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// The tensor's amax from the P partial maxima (256 threads).
__device__ __forceinline__ float block_amax(const float* __restrict__ part, int P, float* red) {
    float m = 0.0f;
    for (int i = threadIdx.x; i < P; i += 256) m = fmaxf(m, part[i]);
    m = group_max<64>(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Chunks head .. nchunk - 1, four per thread per step (loads first), over
// at most 512 blocks.  At 4096 x 4096 (one box, the three launches): 19.0 us
// with 512 blocks, 19.2 with 1024, 20.3 with 2048, 21.0 with 8192 (one chunk
// per thread) and with 256; eight loads per step 21.7, two 20.1; 128, 512
// or 1024 amax blocks instead of 256 were slower (more partial maxima for
// every quant block, or fewer loads in flight).
constexpr int QT_BLOCKS = 512;
__global__ __launch_bounds__(256) void fp8_quant_tensor_kernel(const uint16_t* __restrict__ X,
                                                               uint8_t* __restrict__ Q, size_t nchunk, int P) {
    __shared__ float red[4];
    const float amax = block_amax(reinterpret_cast<const float*>(Q), P, red);
    const float mult = amax > 0.0f ? 448.0f / amax : 0.0f;
    const uint32_t smask = sign_mask(mult);
    const uintx4* x = reinterpret_cast<const uintx4*>(X);
    uintx2* q = reinterpret_cast<uintx2*>(Q);
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t c = (size_t)((P + 1) / 2) + (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; c + 3 * stride < nchunk; c += 4 * stride) {
        uintx4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = ldg_nt(x + c + i * stride);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[c + i * stride] = fp8x8(v[i], mult, smask);
    }
    for (; c < nchunk; c += stride) q[c] = fp8x8(ldg_nt(x + c), mult, smask);
}

// One block of 256 threads: the first ceil(P / 2) chunks and the scale.
__global__ __launch_bounds__(256) void fp8_quant_tensor_head_kernel(const uint16_t* __restrict__ X,
                                                                    uint8_t* __restrict__ Q, int P,
                                                                    float* __restrict__ scale) {
    __shared__ float red[4];
    // (every thread's read of the partial maxima is done at the barrier
    // inside, before any code overwrites them)
    const float amax = block_amax(reinterpret_cast<const float*>(Q), P, red);
    const float mult = amax > 0.0f ? 448.0f / amax : 0.0f;
    const uint32_t smask = sign_mask(mult);
    for (int c = threadIdx.x; c < (P + 1) / 2; c += 256)
        reinterpret_cast<uintx2*>(Q)[c] = fp8x8(reinterpret_cast<const uintx4*>(X)[c], mult, smask);
    if (threadIdx.x == 0) *scale = amax > 0.0f ? amax / 448.0f : 0.0f;
}

// ------------------------------------------------------------------ dequant

// A lane turns chunks of 8 codes into 8 fp16 values (cols % 8 == 0, so a
// chunk never straddles rows); grid-stride over chunks, four per lane per
// step with all their loads first, as in the int8 dequantizer (KV cache:
// 6.23 -> 5.52 us against one chunk per lane).
// IDX: the chunk index type (32 bits whenever the indexes fit); row_shift >=
// 0: chunks per row = 1 << row_shift, and the row index is a shift.
constexpr int FDQ_U = 4, FDQ_BLOCKS = 1024;

__device__ __forceinline__ uintx4 fp8_dequant8(uintx2 q, float s) {
    const uint32_t w[2] = {q.x, q.y};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t h0 = f2h_of_product(__builtin_amdgcn_cvt_f32_fp8((int)w[i], 0), s);
        const uint32_t h1 = f2h_of_product(__builtin_amdgcn_cvt_f32_fp8((int)w[i], 1), s);
        const uint32_t h2 = f2h_of_product(__builtin_amdgcn_cvt_f32_fp8((int)w[i], 2), s);
        const uint32_t h3 = f2h_of_product(__builtin_amdgcn_cvt_f32_fp8((int)w[i], 3), s);
        o[2 * i] = h0 | (h1 << 16);
        o[2 * i + 1] = h2 | (h3 << 16);
    }
    return uintx4{o[0], o[1], o[2], o[3]};
}

template <typename IDX>
__global__ __launch_bounds__(256) void fp8_dequant_kernel(const uint8_t* __restrict__ Q,
                                                          const float* __restrict__ S,
                                                          uint16_t* __restrict__ X, IDX nchunk,
                                                          int chunks_per_row, int row_shift, int per_row) {
    const IDX stride = (IDX)gridDim.x * blockDim.x;
    const uintx2* q2 = reinterpret_cast<const uintx2*>(Q);
    uintx4* x4 = reinterpret_cast<uintx4*>(X);
    auto row = [&](IDX c) { return !per_row ? (IDX)0 : row_shift >= 0 ? c >> row_shift : c / (IDX)chunks_per_row; };
    IDX c = (IDX)blockIdx.x * blockDim.x + threadIdx.x;
    for (; c + (FDQ_U - 1) * stride < nchunk; c += FDQ_U * stride) {
        uintx2 q[FDQ_U];
        float s[FDQ_U];
#pragma unroll
        for (int i = 0; i < FDQ_U; ++i) q[i] = ldg_nt(q2 + c + i * stride);
#pragma unroll
        for (int i = 0; i < FDQ_U; ++i) s[i] = S[row(c + i * stride)];
#pragma unroll
        for (int i = 0; i < FDQ_U; ++i) __builtin_nontemporal_store(fp8_dequant8(q[i], s[i]), x4 + c + i * stride);
    }
    for (; c < nchunk; c += stride) __builtin_nontemporal_store(fp8_dequant8(ldg_nt(q2 + c), S[row(c)]), x4 + c);
}

// ------------------------------------------------------------------ GEMM

constexpr int FB = 256;  // output tile edge

__device__ __forceinline__ floatx16 mfma_fp8(intx8 a, intx8 b, floatx16 c) {
    // format 0 for both operands = E4M3; no block scales
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__global__ __launch_bounds__(512, 1) void fp8_gemm_kernel(const uint8_t* __restrict__ A,
                                                          const uint8_t* __restrict__ W,
                                                          const float* __restrict__ sa, int sa_per_row,
                                                          const float* __restrict__ sw, int sw_per_row,
                                                          uint16_t* __restrict__ Y, int M, int N, int K) {
    constexpr int SL = FB * 128;  // bytes per operand buffer (256 rows x 128 k)
    // A0, A1, W0, W1; after the k loop the fp16 output tile (256 rows x 576 bytes)
    __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * SL + 16384];
    // (the wave index from threadIdx.x: its known range lets the compiler
    // tell the copies' LDS targets from the buffer being read)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    // tile of workgroup L: each XCD (workgroups are dealt round-robin by id)
    // owns a block of tiles sharing A rows and W columns in its L2
    const int mtiles = (M + FB - 1) / FB;
    int tr, tc;
    xcd_tile(blockIdx.x, mtiles, (N + FB - 1) / FB, 4, tr, tc);
    const int m0 = tr * FB, n0 = tc * FB;
    const int kchunks = K / 128, last = kchunks - 1;
    const int h = lane >> 5, c32 = lane & 31;

    floatx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[i][t][j] = 0.f;

    // wave w issues DMA instructions 4w .. 4w + 3 of each operand tile (1 KB =
    // 8 rows of 128 bytes each); the lane filling position pos of row r
    // fetches piece pos ^ ((r >> 1) & 7).  Rows past M or N repeat the last
    // row (never stored).  Sources are 32-bit byte offsets from the operand
    // base (rows * K < 2^32 is checked at launch).
    const int rsub = lane >> 3, pos = lane & 7;
    uint32_t offa[4], offw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 8 * (4 * wave + j) + rsub;
        const uint32_t piece = (uint32_t)((pos ^ ((r >> 1) & 7)) * 16);
        offa[j] = (uint32_t)(m0 + r < M ? m0 + r : M - 1) * (uint32_t)K + piece;
        offw[j] = (uint32_t)(n0 + r < N ? n0 + r : N - 1) * (uint32_t)K + piece;
    }
    // Buffer -> LDS copies (wave-uniform descriptors over A and W, the chunk's
    // k offset as a scalar offset: no vector address arithmetic per copy).
    // Copy i of a chunk: i < 4 A, else W.
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(A, 0xffffffffu), rw = buffer_rsrc(W, 0xffffffffu);
    auto dma_one = [&](int c, int buf, int i) __attribute__((always_inline)) {
        if (i < 4) buffer_load_lds<16>(ra, lds + buf * SL + (4 * wave + i) * 1024, offa[i], (uint32_t)c * 128u);
        else buffer_load_lds<16>(rw, lds + (2 + buf) * SL + (4 * wave + i - 4) * 1024, offw[i - 4], (uint32_t)c * 128u);
    };
    // operand of row r for 64-k step s: bytes k = 64 s + 32 h .. + 31 = pieces
    // 4 s + 2 h and 4 s + 2 h + 1 of the row
    auto frag = [&](const uint8_t* buf, int r, int s) {
        const int p = 4 * s + 2 * h, sw = (r >> 1) & 7;
        const intx4 lo = *reinterpret_cast<const intx4*>(buf + r * 128 + ((p ^ sw) * 16));
        const intx4 hi = *reinterpret_cast<const intx4*>(buf + r * 128 + (((p + 1) ^ sw) * 16));
        return intx8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    };
    auto operands = [&](const uint8_t* ab, const uint8_t* wb, int s, intx8 (&a)[4], intx8 (&b)[2]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = frag(ab, wm * 128 + i * 32 + c32, s);
#pragma unroll
        for (int t = 0; t < 2; ++t) b[t] = frag(wb, wn * 64 + t * 32 + c32, s);
    };
    // two 64-k steps per chunk; the operand reads of step 1 and the eight
    // copies of the next chunk are interleaved with the MFMAs of step 0
    // (issued as one burst, the copies of the eight waves queue at the address
    // unit and the waves stall at issue)
    auto compute = [&](const uint8_t* ab, const uint8_t* wb, int cn, int nbuf) {
        intx8 a[4], b[2], an[4], bn[2];
        operands(ab, wb, 0, a, b);
#pragma unroll
        for (int i = 0; i < 8; ++i) dma_one(cn, nbuf, i);
        operands(ab, wb, 1, an, bn);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < 2; ++t) acc[i][t] = mfma_fp8(a[i], b[t], acc[i][t]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
            __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // one copy
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // one copy
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < 2; ++t) acc[i][t] = mfma_fp8(an[i], bn[t], acc[i][t]);
    };

#pragma unroll
    for (int i = 0; i < 8; ++i) dma_one(0, 0, i);
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    // one trip per chunk: DMA of chunk c + 1 into the idle buffers, MFMAs on
    // chunk c, then a wait for this wave's DMA and a bare barrier (buffer
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

    // ---- epilogue: Y = fp16(fl(fl(acc * sa) * sw)) through an LDS tile, so
    // that rows are written in 16-byte pieces: a quad transpose gives each
    // lane four adjacent columns of one row (8 bytes), stored into a
    // row-major tile of pitch 576 bytes.  The operand buffers are free: the
    // last trip ended with every wave's DMA drained and a barrier.
    constexpr int EPW = 144;  // tile pitch in dwords (512 bytes + 64)
    uint32_t* stile = reinterpret_cast<uint32_t*>(lds);
    const int q = lane & 3;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int col = n0 + wn * 64 + t * 32 + c32;
        const float swv = sw[sw_per_row ? (col < N ? col : N - 1) : 0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int r0 = wm * 128 + i * 32 + 8 * g + 4 * h;  // tile row of register 4g
                uint32_t v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = m0 + r0 + r < M ? m0 + r0 + r : M - 1;  // rows >= M are not stored
                    v[r] = f2h_of_product(acc[i][t][4 * g + r] * sa[sa_per_row ? row : 0], swv);
                }
                uint32_t e0, e1;
                quad_rows_u16(v[0] | (v[1] << 16), v[2] | (v[3] << 16), lane, e0, e1);
                *reinterpret_cast<uintx2*>(&stile[(r0 + q) * EPW + wn * 32 + t * 16 + 2 * (c32 >> 2)]) =
                    uintx2{e0, e1};
            }
        }
    }
    __syncthreads();
    // 256 rows x 32 pieces of 8 outputs; a piece past N (or any piece when
    // rows are not 16-byte aligned, N % 8 != 0) is written output by output
    const bool vec = (N & 7) == 0;
    const int tid = threadIdx.x;
#pragma unroll 4
    for (int p = 0; p < 16; ++p) {
        const int idx = tid + 512 * p, row = idx >> 5, piece = idx & 31;
        const int colg = n0 + piece * 8;
        if (m0 + row >= M || colg >= N) continue;
        const uint32_t* src = &stile[row * EPW + piece * 4];
        uint16_t* dst = Y + (size_t)(m0 + row) * N + colg;
        if (vec && colg + 8 <= N) {
            __builtin_nontemporal_store(*reinterpret_cast<const uintx4*>(src), reinterpret_cast<uintx4*>(dst));
        } else {
            for (int e = 0; e < 8 && colg + e < N; ++e) dst[e] = (uint16_t)(src[e >> 1] >> (16 * (e & 1)));
        }
    }
}

int grid_for(size_t nchunk) {
    const size_t want = (nchunk + 255) / 256;
    return (int)(want < 8192 ? (want > 0 ? want : 1) : 8192);
}

}  // namespace

extern "C" int32_t quant_fp8_e4m3(const uint16_t* X, uint8_t* Q, float* scales, int32_t rows,
                                  int32_t cols, int32_t per_row, void* stream) {
    if (rows < 0 || cols < 0) return QGEMM_BAD_SHAPE;
    if (rows == 0) return QGEMM_OK;
    if (!X || !Q || !scales) return QGEMM_NULL_PTR;
    if (cols == 0 || cols % 8 != 0 || (per_row && cols > 4096) || (per_row != 0 && per_row != 1))
        return QGEMM_UNSUPPORTED;
    if (!qgh::aligned(X, 16) || !qgh::aligned(Q, 16) || !qgh::aligned(scales, 4)) return QGEMM_MISALIGNED;
    hipStream_t st = (hipStream_t)stream;
    if (per_row) {
        // 8 lanes of two chunks per row up to 128 values (the KV rows), as
        // for the int8 quantizer; variants without bounds selects for rows
        // that fill the lane group exactly
        auto launch = [&](auto kern, int lpr) {
            const int rpb = 256 / lpr;
            hipLaunchKernelGGL(kern, dim3((rows + rpb - 1) / rpb), dim3(256), 0, st, X, Q, scales, rows, cols);
        };
        if (cols == 128) launch(fp8_quant_rows_kernel<8, 2, true>, 8);
        else if (cols < 128) launch(fp8_quant_rows_kernel<8, 2, false>, 8);
        else if (cols <= 256) launch(fp8_quant_rows_kernel<16, 2, false>, 16);
        else if (cols == 4096) launch(fp8_quant_rows_kernel<64, 8, true>, 64);
        else launch(fp8_quant_rows_kernel<64, 8, false>, 64);
        return qgh::launch_status();
    }
    const size_t nchunk = (size_t)rows * cols / 8;
    // P partial maxima: at most 256 blocks, at most one per 256 chunks, so
    // 4 P <= 8 nchunk bytes of Q hold them
    const int P = grid_for(nchunk) < AMAX_BLOCKS ? grid_for(nchunk) : AMAX_BLOCKS;
    hipLaunchKernelGGL(fp8_amax_kernel, dim3(P), dim3(256), 0, st, X, nchunk, reinterpret_cast<float*>(Q));
    const int qblocks = grid_for(nchunk) < QT_BLOCKS ? grid_for(nchunk) : QT_BLOCKS;
    hipLaunchKernelGGL(fp8_quant_tensor_kernel, dim3(qblocks), dim3(256), 0, st, X, Q, nchunk, P);
    hipLaunchKernelGGL(fp8_quant_tensor_head_kernel, dim3(1), dim3(256), 0, st, X, Q, P, scales);
    return qgh::launch_status();
}

extern "C" int32_t dequant_fp8_e4m3(const uint8_t* Q, const float* scales, uint16_t* X, int32_t rows,
                                    int32_t cols, int32_t per_row, void* stream) {
    if (rows < 0 || cols < 0) return QGEMM_BAD_SHAPE;
    if (rows == 0) return QGEMM_OK;
    if (!Q || !scales || !X) return QGEMM_NULL_PTR;
    if (cols == 0 || cols % 8 != 0 || (per_row != 0 && per_row != 1)) return QGEMM_UNSUPPORTED;
    if (!qgh::aligned(Q, 16) || !qgh::aligned(X, 16) || !qgh::aligned(scales, 4)) return QGEMM_MISALIGNED;
    const size_t nchunk = (size_t)rows * cols / 8;
    const size_t want = (nchunk + 256 * FDQ_U - 1) / (256 * FDQ_U);
    const int blocks = (int)(want < FDQ_BLOCKS ? want : FDQ_BLOCKS), cpr = cols / 8;
    const int shift = (cpr & (cpr - 1)) == 0 ? __builtin_ctz((unsigned)cpr) : -1;
    if (nchunk + (size_t)blocks * 256 * FDQ_U < ((size_t)1 << 32))
        hipLaunchKernelGGL(fp8_dequant_kernel<uint32_t>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, Q,
                           scales, X, (uint32_t)nchunk, cpr, shift, per_row);
    else
        hipLaunchKernelGGL(fp8_dequant_kernel<size_t>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, Q, scales,
                           X, nchunk, cpr, shift, per_row);
    return qgh::launch_status();
}

extern "C" int32_t qgemm_fp8(const uint8_t* A, const uint8_t* W, const float* a_scale, int32_t a_per_row,
                             const float* w_scale, int32_t w_per_row, uint16_t* Y, int32_t M, int32_t N,
                             int32_t K, void* stream) {
    if (M < 0 || N < 0 || K < 0) return QGEMM_BAD_SHAPE;
    if (M == 0 || N == 0) return QGEMM_OK;
    if (!A || !W || !a_scale || !w_scale || !Y) return QGEMM_NULL_PTR;
    if (K == 0 || K % 128 != 0 || (a_per_row != 0 && a_per_row != 1) || (w_per_row != 0 && w_per_row != 1) ||
        (size_t)M * K >= ((size_t)1 << 32) || (size_t)N * K >= ((size_t)1 << 32))
        return QGEMM_UNSUPPORTED;
    if (!qgh::aligned(A, 16) || !qgh::aligned(W, 16) || !qgh::aligned(Y, 16) || !qgh::aligned(a_scale, 4) ||
        !qgh::aligned(w_scale, 4))
        return QGEMM_MISALIGNED;
    const int grid = ((N + FB - 1) / FB) * ((M + FB - 1) / FB);
    hipLaunchKernelGGL(fp8_gemm_kernel, dim3(grid), dim3(512), 0, (hipStream_t)stream, A, W, a_scale, a_per_row,
                       w_scale, w_per_row, Y, M, N, K);
    return qgh::launch_status();
}
