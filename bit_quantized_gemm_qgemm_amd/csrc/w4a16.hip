// W4A16 group-wise GEMM: Y[M,N] = A[M,K] (fp16) x (q (int4) * S (fp16, one
// per (K-group, column))), fp32 accumulation, fp16 output.
//
// Int4 Groupwise GEMM Plugin V2 page (class summary: inputs, output and the
// fragment-layout weights; configurePlugin: the token count M steers the
// kernel choice; getValidTactics / setTactic: listed kernel variants).
// Four kernels, all shared with the int8 path (wq_gemm.hpp): decode
// (M <= 16), mid-M split-K (16 < M <= 128, with workspace), 128x128 prefill,
// and 128x256 prefill (chosen by default when it has enough tiles to fill
// the chip; A tiles and B fragment blocks reach LDS by direct DMA).  Each
// launch shape is also a tactic a caller can list, select or autotune.
// K or N that are not multiples of 128 (the page's ceil(K/G) scale rows and
// padded fragment tiles) run the decode or the 128x128 prefill kernel.
#include "common.hpp"
#include "wq_gemm.hpp"

namespace {

using namespace qg;

// ------------------------------------------------------------------ large prefill


// Tactics (ids in the header): the kernels and launch shapes above, one id
// each.  validity follows from what each kernel assumes of the shape.
bool tactic_valid(int tactic, int M, int N, int K) {
    switch (tactic) {
        case QGEMM_W4A16_TACTIC_DECODE_NARROW: return M <= 2;
        case QGEMM_W4A16_TACTIC_DECODE_BALANCED: return M <= 16;
        case QGEMM_W4A16_TACTIC_SPLITK: return !ragged(N, K) && M <= 512 && (size_t)M * K < ((size_t)1 << 31);
        case QGEMM_W4A16_TACTIC_PREFILL: return true;
        case QGEMM_W4A16_TACTIC_PREFILL_LARGE: return !ragged(N, K) && N % PL_BN == 0;
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
    if (ragged(N, K)) return QGEMM_W4A16_TACTIC_PREFILL;
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
            hipLaunchKernelGGL((wq_prefill_large_pc_kernel<G>), grid, dim3(320), 0, st, A, wf, S, N, Y, M, N, K);
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

// Shape and group support of every W4A16 call (M > 0): K and N multiples of
// 8 (16-byte rows of A and Y), not necessarily of 128 or of G.
bool w4a16_shape_ok(int M, int N, int K, int G) {
    return M > 0 && N > 0 && K > 0 && N % 8 == 0 && K % 8 == 0 && (G == 32 || G == 64 || G == 128);
}

// Validation shared by the launching entry points; QGEMM_OK means "launch".
int32_t w4a16_check(const uint16_t* A, const uint8_t* w_frag, const uint16_t* scales, uint16_t* Y, int M, int N,
                    int K, int G) {
    if (M < 0 || N < 0 || K < 0 || G <= 0) return QGEMM_BAD_SHAPE;
    if (!A || !w_frag || !scales || !Y) return QGEMM_NULL_PTR;
    if (N == 0 || K == 0 || N % 8 != 0 || K % 8 != 0) return QGEMM_UNSUPPORTED;
    if (G != 32 && G != 64 && G != 128) return QGEMM_UNSUPPORTED;
    if (!qgh::aligned(A, 16) || !qgh::aligned(w_frag, 16) || !qgh::aligned(scales, 4) ||
        !qgh::aligned(Y, 16))
        return QGEMM_MISALIGNED;
    return QGEMM_OK;
}

}  // namespace

// the mid-M path's fp32 split partials; 0 for every other shape
extern "C" size_t qgemm_w4a16_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t G) {
    if (!w4a16_shape_ok(M, N, K, G) || ragged(N, K)) return 0;
    return mid_path(M, K) ? mid_workspace_bytes(M, N, K) : 0;
}

extern "C" int32_t qgemm_w4a16(const uint16_t* A, const uint8_t* w_frag, const uint16_t* scales,
                               uint16_t* Y, int32_t M, int32_t N, int32_t K, int32_t G,
                               void* workspace, size_t workspace_bytes, void* stream) {
    if (M == 0 && N >= 0 && K >= 0 && G > 0) return QGEMM_OK;
    const int32_t st = w4a16_check(A, w_frag, scales, Y, M, N, K, G);
    if (st != QGEMM_OK) return st;
    float* part = nullptr;
    if (!ragged(N, K) && mid_path(M, K) && workspace && qgh::aligned(workspace, 16) &&
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
    if (M == 0 && N >= 0 && K >= 0 && G > 0) return QGEMM_OK;
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
