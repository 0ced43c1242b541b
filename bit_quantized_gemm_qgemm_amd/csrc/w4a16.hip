// W4A16 group-wise GEMM: Y[M,N] = A[M,K] (fp16) x (q (int4) * S (fp16, one
// per (K-group, column))), fp32 accumulation, fp16 output.
//
// Int4 Groupwise GEMM Plugin V2 page (class summary: inputs, output and the
// fragment-layout weights; configurePlugin: the token count M steers the
// kernel choice; getValidTactics / setTactic: listed kernel variants).
// Four kernels: the decode (M <= 16), mid-M split-K (16 < M <= 128, with
// workspace) and 128x128 prefill kernels shared with the int8 path
// (wq_gemm.hpp), and the large prefill kernel below (chosen by default when
// it has enough tiles to fill the chip): 256x128 tiles, four waves of 128x64;
// A tiles go global -> LDS by direct DMA with an XOR swizzle, B fragment
// blocks and scale rows likewise.  Each launch shape is also a tactic a
// caller can list, select or autotune.
#include "common.hpp"
#include "wq_gemm.hpp"

namespace {

using namespace qg;

// ------------------------------------------------------------------ large prefill

// Large-M prefill: 128x256 output tiles, four waves side by side, each
// 128 rows x 64 columns (4 x 2 v_mfma_f32_32x32x16_f16 tiles, accumulators in
// the unified VGPR/AGPR file); one workgroup per CU at M = 2048.  A tile that
// is wide in N suits W4A16: per 128-k chunk a workgroup streams 32 KB of fp16
// A and 16 KB of int4 B (a 256 x 128 tile would need 64 KB + 8 KB for the
// same MFMA work), and each wave owns its columns, so every B element is
// dequantized once per workgroup.
//
// Every load in the main loop is a global -> LDS DMA (no VGPR destinations,
// no VALU): A (two buffers) and B (fragment blocks plus scale rows, three
// stages, so B is fetched two chunks ahead).  A wave's A-DMA instruction
// fills 1 KB of LDS in lane order (four 256-byte rows); the lane that fills
// position pos of row r fetches piece pos ^ (r & 15) of that row, so the MFMA
// fragment reads, 16 rows at one k-group, hit 16 distinct 16-byte bank
// groups.  The loop waits for the DMA it needs with an explicit counter wait
// and a bare barrier: __syncthreads() would also wait for the B prefetch
// still in flight.
constexpr int PL_BM = 128, PL_BN = 256;

template <int G>
__global__ __launch_bounds__(256, 1) void w4a16_prefill_large_kernel(const uint16_t* __restrict__ A,
                                                                      const uint8_t* __restrict__ wf,
                                                                      const uint16_t* __restrict__ S,
                                                                      uint16_t* __restrict__ Y, int M,
                                                                      int N, int K) {
    constexpr int NG = 128 / G;
    constexpr int SLAB = PL_BM * 128;        // halfs per A buffer (32 KB)
    constexpr int BST = 16384 + 512 * NG;    // bytes per B stage: two fragment blocks + NG scale rows
    constexpr int BDMA = 4 + 2 * NG;         // DMA instructions per wave for one B stage
    // One LDS array for A and B: the compiler tells DMA targets from the
    // buffers being read by their offsets within one array, but not across
    // two arrays (it would then wait for every DMA before each LDS read).
    // (Sized for the largest stage, G = 32: an array whose size depends on
    // the template parameter, passed to the DMA builtin, made the host
    // compiler drop the kernel's launch stub without a diagnostic.)
    __shared__ __attribute__((aligned(1024))) uint16_t sA[2 * PL_BM * 128 + 3 * (16384 + 512 * 4) / 2];
    uint8_t* const sB = reinterpret_cast<uint8_t*>(sA + 2 * SLAB);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // Workgroups are dealt to the 8 XCDs round-robin by id.  Tile (x, y) of
    // id L has y = L % (row tiles), so the workgroups on one XCD share their
    // A row tiles in that XCD's L2 and stream distinct B tiles.
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
    const int rsub = lane >> 4, pos = lane & 15;
    auto dma_a = [&](int c, int buf) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 4 * (8 * wave + j) + rsub;
            const int gm = m0 + r < M ? m0 + r : M - 1;
            const uint16_t* src = A + (size_t)gm * K + c * 128 + ((pos ^ (r & 15)) * 8);
            __builtin_amdgcn_global_load_lds(src, sA + buf * SLAB + (8 * wave + j) * 512, 16, 0, 0);
        }
    };
    // B: the tile's 256 columns are strips n0/16 .. n0/16 + 15, two 8 KB
    // fragment blocks per chunk (stored one after the other in a stage);
    // wave w copies strips 4w .. 4w + 3.  Each wave also copies every scale
    // row of the chunk (512 bytes each; the four copies write identical
    // bytes), which keeps the per-wave DMA count equal.
    const uint8_t* wtile = wf + (size_t)(n0 >> 7) * kchunks * 8192;
    const size_t sb_stride = (size_t)kchunks * 8192;  // between the two fragment blocks
    auto dma_b = [&](int c, int stage) {
        uint8_t* dst = sB + stage * BST;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int strip = 4 * wave + j;
            __builtin_amdgcn_global_load_lds(wtile + (strip >> 3) * sb_stride + (size_t)c * 8192 +
                                                 (strip & 7) * 1024 + lane * 16,
                                             dst + strip * 1024, 16, 0, 0);
        }
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                __builtin_amdgcn_global_load_lds(S + (size_t)(c * NG + g) * N + n0 + 128 * hh + 2 * lane,
                                                 dst + 16384 + g * 512 + hh * 256, 4, 0, 0);
    };
    // this lane's B fragment pieces inside a stage: tile t, k-group parity h,
    // pieces q = h and q = h + 2 of the strip holding column 64 wave + 32 t + c32
    auto read_b = [&](const uint8_t* sb, BChunk<2, G>& b) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int colt = wave * 64 + t * 32 + c32;  // column inside the tile
            const uint8_t* blk = sb + (colt >> 4) * 1024 + (colt & 15) * 16;
            b.raw[t][0] = *reinterpret_cast<const uintx4*>(blk + 16 * 16 * h);
            b.raw[t][1] = *reinterpret_cast<const uintx4*>(blk + 16 * 16 * (h + 2));
#pragma unroll
            for (int g = 0; g < NG; ++g)
                b.sc[t][g] = reinterpret_cast<const uint16_t*>(sb + 16384)[g * 256 + colt];
        }
    };
    // Software-pipelined k-steps: the LDS reads and the dequant of step s + 1
    // are interleaved with the eight MFMAs of step s (one MFMA, then at most
    // one LDS read and four VALU ops), so the in-order wave keeps the MFMA
    // unit busy while it prepares the next operands.
    auto operands = [&](const uint16_t* sa, const BChunk<2, G>& b, int s, half8 (&a)[4], half8 (&bf)[2]) {
        const int kg = kgroup_of_step(s, h);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = i * 32 + c32;
            a[i] = *reinterpret_cast<const half8*>(&sa[r * 128 + ((kg ^ (r & 15)) * 8)]);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) bf[t] = b_frag<2, G>(b, t, s);
    };
    // issue(): this trip's DMAs, placed after the LDS reads of step 0 so that
    // their issue overlaps the read latency
    auto compute = [&](const uint16_t* sa, const BChunk<2, G>& b, auto issue) {
        half8 a[4], bf[2];
        operands(sa, b, 0, a, bf);
        __builtin_amdgcn_sched_barrier(0);
        issue();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            half8 an[4], bn[2];
            if (s < 7) operands(sa, b, s + 1, an, bn);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int t = 0; t < 2; ++t) acc[i][t] = mfma32(a[i], bf[t], acc[i][t]);
            if (s < 7) {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    if (q < 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = an[i];
#pragma unroll
            for (int t = 0; t < 2; ++t) bf[t] = bn[t];
        }
    };

    dma_a(0, 0);
    dma_b(0, 0);
    dma_b(last < 1 ? last : 1, 1);
    wait_vmcnt<0>();
    __syncthreads();
    // One trip = one chunk.  Every LDS offset a DMA writes is a compile-time
    // constant in each trip (A buffer c % 2, B stage c % 3, so six trips per
    // loop pass): with a run-time buffer or stage index the compiler cannot
    // tell the DMA target from the buffer being read and waits for the DMA
    // before every LDS read.
    // (buf and stage are literals at every call; after inlining they fold)
    auto trip = [&](int c, int buf, int stage) __attribute__((always_inline)) {
        const int s2 = (stage + 2) % 3;  // stage of chunk c + 2
        // B of chunk c goes to registers before this trip's DMAs are issued
        // (LDS reads of a B stage after them would wait for those DMAs)
        BChunk<2, G> b;
        read_b(sB + stage * BST, b);
        compute(sA + buf * SLAB, b, [&]() {
            dma_a(c + 1 < last ? c + 1 : last, buf ^ 1);
            dma_b(c + 2 < last ? c + 2 : last, s2);
        });
        // chunk c + 1's A (and, issued before it, its B) has landed; chunk
        // c + 2's B may still be in flight
        wait_vmcnt<BDMA>();
        wait_lgkmcnt0();  // this wave's LDS reads of the buffers refilled next are done
        __builtin_amdgcn_s_barrier();
    };
    for (int c = 0; c < kchunks; c += 6) {
        trip(c, 0, 0);
        if (c + 1 < kchunks) trip(c + 1, 1, 1);
        if (c + 2 < kchunks) trip(c + 2, 0, 2);
        if (c + 3 < kchunks) trip(c + 3, 1, 0);
        if (c + 4 < kchunks) trip(c + 4, 0, 1);
        if (c + 5 < kchunks) trip(c + 5, 1, 2);
    }
    // ---- epilogue: Y through an LDS tile in 16-byte row pieces.  A quad
    // transpose gives each lane four adjacent columns of one row (8 bytes of
    // fp16), stored into a row-major tile of pitch 576 bytes; then every
    // thread writes whole 16-byte pieces.  Each wave first drains its last
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
            *reinterpret_cast<uintx4*>(Y + (size_t)(m0 + row) * N + n0 + piece * 8) =
                *reinterpret_cast<const uintx4*>(&stile[row * EPW + piece * 4]);
    }
}

// Tactics (ids in the header): the kernels and launch shapes above, one id
// each.  validity follows from what each kernel assumes of the shape.
bool tactic_valid(int tactic, int M, int N, int K) {
    switch (tactic) {
        case QGEMM_W4A16_TACTIC_DECODE_NARROW: return M <= 2;
        case QGEMM_W4A16_TACTIC_DECODE_BALANCED: return M <= 16;
        case QGEMM_W4A16_TACTIC_SPLITK: return M <= 512 && (size_t)M * K < ((size_t)1 << 32);
        case QGEMM_W4A16_TACTIC_PREFILL: return true;
        case QGEMM_W4A16_TACTIC_PREFILL_LARGE: return N % PL_BN == 0;
        default: return false;
    }
}

// The tactic the default call takes (workspace: enough for the split-K path).
// Above the split-K range the 128x256 kernel (one workgroup per CU) wins once
// it has at least 160 tiles to spread over the 256 CUs; with fewer, the
// 128x128 kernel's twice as many workgroups keep more CUs busy (measured at
// K = 4096: N = 11008, M = 512, 172 tiles: 54 us against 74; N = 4096,
// M = 1024, 128 tiles: 52 us against 47).
int default_tactic(int M, int N, int K, bool workspace) {
    if (M <= 2) return QGEMM_W4A16_TACTIC_DECODE_NARROW;
    if (M <= 16) return QGEMM_W4A16_TACTIC_DECODE_BALANCED;
    if (workspace && mid_path(M, K)) return QGEMM_W4A16_TACTIC_SPLITK;
    const long large_tiles = (long)(N / PL_BN) * ((M + PL_BM - 1) / PL_BM);
    if (N % PL_BN != 0 || large_tiles < 160) return QGEMM_W4A16_TACTIC_PREFILL;
    return QGEMM_W4A16_TACTIC_PREFILL_LARGE;
}

template <int G>
void launch_w4a16(int tactic, const uint16_t* A, const uint8_t* wf, const uint16_t* S, uint16_t* Y, int M, int N,
                  int K, float* part, hipStream_t st) {
    switch (tactic) {
        case QGEMM_W4A16_TACTIC_DECODE_NARROW: launch_wq_decode_narrow<4, G>(A, wf, S, N, Y, M, N, K, st); break;
        case QGEMM_W4A16_TACTIC_DECODE_BALANCED:
            launch_wq_decode_balanced<4, G>(A, wf, S, N, Y, M, N, K, st);
            break;
        case QGEMM_W4A16_TACTIC_SPLITK: launch_wq_mid<4, G>(A, wf, S, N, Y, M, N, K, part, st); break;
        case QGEMM_W4A16_TACTIC_PREFILL: launch_wq_prefill<4, G>(A, wf, S, N, Y, M, N, K, st); break;
        default: {
            dim3 grid((N / PL_BN) * ((M + PL_BM - 1) / PL_BM));
            hipLaunchKernelGGL(w4a16_prefill_large_kernel<G>, grid, dim3(256), 0, st, A, wf, S, Y, M, N, K);
        }
    }
}

int32_t launch_w4a16_g(int tactic, const uint16_t* A, const uint8_t* wf, const uint16_t* S, uint16_t* Y, int M,
                       int N, int K, int G, float* part, hipStream_t st) {
    switch (G) {
        case 32: launch_w4a16<32>(tactic, A, wf, S, Y, M, N, K, part, st); break;
        case 64: launch_w4a16<64>(tactic, A, wf, S, Y, M, N, K, part, st); break;
        default: launch_w4a16<128>(tactic, A, wf, S, Y, M, N, K, part, st);
    }
    return qgh::launch_status();
}

// Shape and group support of every W4A16 call (M > 0).
bool w4a16_shape_ok(int M, int N, int K, int G) {
    return M > 0 && N > 0 && K > 0 && N % 128 == 0 && K % 128 == 0 && (G == 32 || G == 64 || G == 128);
}

// Validation shared by the launching entry points; QGEMM_OK means "launch".
int32_t w4a16_check(const uint16_t* A, const uint8_t* w_frag, const uint16_t* scales, uint16_t* Y, int M, int N,
                    int K, int G) {
    if (M < 0 || N < 0 || K < 0 || G <= 0) return QGEMM_BAD_SHAPE;
    if (K % G != 0) return QGEMM_BAD_SHAPE;
    if (!A || !w_frag || !scales || !Y) return QGEMM_NULL_PTR;
    if (N == 0 || K == 0 || N % 128 != 0 || K % 128 != 0) return QGEMM_UNSUPPORTED;
    if (G != 32 && G != 64 && G != 128) return QGEMM_UNSUPPORTED;
    if (!qgh::aligned(A, 16) || !qgh::aligned(w_frag, 16) || !qgh::aligned(scales, 4) ||
        !qgh::aligned(Y, 16))
        return QGEMM_MISALIGNED;
    return QGEMM_OK;
}

}  // namespace

// the mid-M path's fp32 split partials; 0 for every other shape
extern "C" size_t qgemm_w4a16_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t G) {
    if (M <= 0 || N <= 0 || K <= 0 || G <= 0 || N % 128 != 0 || K % 128 != 0 || K % G != 0) return 0;
    return mid_path(M, K) ? mid_workspace_bytes(M, N, K) : 0;
}

extern "C" int32_t qgemm_w4a16(const uint16_t* A, const uint8_t* w_frag, const uint16_t* scales,
                               uint16_t* Y, int32_t M, int32_t N, int32_t K, int32_t G,
                               void* workspace, size_t workspace_bytes, void* stream) {
    if (M == 0 && N >= 0 && K >= 0 && G > 0 && K % G == 0) return QGEMM_OK;
    const int32_t st = w4a16_check(A, w_frag, scales, Y, M, N, K, G);
    if (st != QGEMM_OK) return st;
    float* part = nullptr;
    if (mid_path(M, K) && workspace && qgh::aligned(workspace, 16) &&
        workspace_bytes >= mid_workspace_bytes(M, N, K))
        part = static_cast<float*>(workspace);
    return launch_w4a16_g(default_tactic(M, N, K, part != nullptr), A, w_frag, scales, Y, M, N, K, G, part,
                          (hipStream_t)stream);
}

extern "C" int32_t qgemm_w4a16_tactics(int32_t M, int32_t N, int32_t K, int32_t G, int32_t* tactics,
                                       int32_t capacity) {
    if (!w4a16_shape_ok(M, N, K, G)) return 0;
    int32_t n = 0;
    for (int t = 1; t <= QGEMM_W4A16_TACTIC_PREFILL_LARGE; ++t)
        if (tactic_valid(t, M, N, K)) {
            if (tactics && n < capacity) tactics[n] = t;
            ++n;
        }
    return n;
}

extern "C" size_t qgemm_w4a16_tactic_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t G, int32_t tactic) {
    if (!w4a16_shape_ok(M, N, K, G)) return 0;
    if (tactic == QGEMM_TACTIC_DEFAULT) return qgemm_w4a16_workspace_bytes(M, N, K, G);
    if (tactic == QGEMM_W4A16_TACTIC_SPLITK && tactic_valid(tactic, M, N, K)) return mid_workspace_bytes(M, N, K);
    return 0;
}

extern "C" int32_t qgemm_w4a16_tactic(const uint16_t* A, const uint8_t* w_frag, const uint16_t* scales, uint16_t* Y,
                                      int32_t M, int32_t N, int32_t K, int32_t G, int32_t tactic, void* workspace,
                                      size_t workspace_bytes, void* stream) {
    if (tactic == QGEMM_TACTIC_DEFAULT)
        return qgemm_w4a16(A, w_frag, scales, Y, M, N, K, G, workspace, workspace_bytes, stream);
    if (M == 0 && N >= 0 && K >= 0 && G > 0 && K % G == 0) return QGEMM_OK;
    const int32_t st = w4a16_check(A, w_frag, scales, Y, M, N, K, G);
    if (st != QGEMM_OK) return st;
    if (!tactic_valid(tactic, M, N, K)) return QGEMM_UNSUPPORTED;
    float* part = nullptr;
    if (tactic == QGEMM_W4A16_TACTIC_SPLITK) {
        if (!workspace || workspace_bytes < mid_workspace_bytes(M, N, K)) return QGEMM_WORKSPACE_TOO_SMALL;
        if (!qgh::aligned(workspace, 16)) return QGEMM_MISALIGNED;
        part = static_cast<float*>(workspace);
    }
    return launch_w4a16_g(tactic, A, w_frag, scales, Y, M, N, K, G, part, (hipStream_t)stream);
}

extern "C" int32_t qgemm_w4a16_autotune(const uint16_t* A, const uint8_t* w_frag, const uint16_t* scales,
                                        uint16_t* Y, int32_t M, int32_t N, int32_t K, int32_t G, void* workspace,
                                        size_t workspace_bytes, int32_t reps, int32_t* best_tactic,
                                        float* best_us, void* stream) {
    if (!best_tactic) return QGEMM_NULL_PTR;
    if (reps <= 0) return QGEMM_BAD_SHAPE;
    if (M == 0) return QGEMM_BAD_SHAPE;  // nothing to time
    const int32_t st0 = w4a16_check(A, w_frag, scales, Y, M, N, K, G);
    if (st0 != QGEMM_OK) return st0;
    hipStream_t st = (hipStream_t)stream;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return QGEMM_HIP_ERROR;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return QGEMM_HIP_ERROR;
    }
    int32_t best = 0, status = QGEMM_OK;
    float best_ms = 0.f;
    for (int t = 1; t <= QGEMM_W4A16_TACTIC_PREFILL_LARGE && status == QGEMM_OK; ++t) {
        if (!tactic_valid(t, M, N, K)) continue;
        if (t == QGEMM_W4A16_TACTIC_SPLITK &&
            (!workspace || !qgh::aligned(workspace, 16) || workspace_bytes < mid_workspace_bytes(M, N, K)))
            continue;
        for (int i = 0; i < 2 && status == QGEMM_OK; ++i)  // warm-up
            status = qgemm_w4a16_tactic(A, w_frag, scales, Y, M, N, K, G, t, workspace, workspace_bytes, stream);
        if (status != QGEMM_OK || hipEventRecord(e0, st) != hipSuccess) break;
        for (int i = 0; i < reps && status == QGEMM_OK; ++i)
            status = qgemm_w4a16_tactic(A, w_frag, scales, Y, M, N, K, G, t, workspace, workspace_bytes, stream);
        float ms = 0.f;
        if (status != QGEMM_OK || hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
            hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
            if (status == QGEMM_OK) status = QGEMM_HIP_ERROR;
            break;
        }
        if (best == 0 || ms < best_ms) {
            best = t;
            best_ms = ms;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (status != QGEMM_OK) return status;
    *best_tactic = best;
    if (best_us) *best_us = best_ms * 1000.f / (float)reps;
    return QGEMM_OK;
}
