// INT8 multi-head attention chain: O = requant(P V), P = int8 softmax of the
// int32 logits Q K^T.
//
// Interview Q&A "INT8 cross-modal multi-head-attention TensorRT plugin"
// (cms365.cn), answer step 3 (enqueue core): an int8 QK^T GEMM to int32
// logits, an online softmax from fp32 to int8 probabilities with the factor
// scale_q * scale_k, an int8 P.V GEMM, then requantization with the output
// scale and an fp16 bias; answer step 2: output [batch, seq, heads,
// head_dim].  The page runs three library calls with the logits and the
// probabilities in a workspace; here one kernel keeps both on chip.
//
// A workgroup of NW waves owns QB = 32 NW queries of one (batch, head); wave
// w owns 32 of them and holds their Q fragments in registers.  K and V go
// through LDS in blocks of 32 keys (two buffers, one barrier per block).
// Pass 1 runs S^T = K Q^T for every key block with v_mfma_i32_32x32x32_i8
// (keys as rows, so a lane holds 16 keys of one query) and keeps the online
// row maximum (of the integer logits) and exp-sum; pass 2 recomputes each
// block's S^T, turns it into int8 codes P = rne(exp(x - m) * fl(127 / l)) in
// the same registers (v_cvt_pk_u8_f32 rounds and packs), and feeds them as
// the B operand of
// O^T = V^T P^T: the k order of that
// MFMA is the accumulator's row order (keys 8 (j / 4) + 4 (lane / 32) + j % 4
// for register j), so V is written to LDS transposed in that key order.
#include <type_traits>

#include "common.hpp"

namespace {

using namespace qg;

constexpr int KB = 32;       // keys per block
constexpr int NW = 4;        // waves per workgroup
constexpr int QB = 32 * NW;  // queries per workgroup
constexpr float LOG2E = 1.44269504088896340736f;

__device__ __forceinline__ intx16 mfma_i8(intx4 a, intx4 b, intx16 c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// Key (inside a 32-key block) of accumulator register j in lane l.
__device__ __forceinline__ int key_of(int j, int lane) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }

constexpr int NBUF = 2;      // LDS stages: a block is fetched one block ahead

template <int D>
struct MhaLds {
    int8_t k[NBUF][KB][D + 16];        // K block, row-major (16-byte pad per row)
    uint32_t vt[NBUF][D][KB / 4 + 4];  // V block transposed: row d, dword g = keys of position 4g .. 4g + 3
};

// Transpose a 4 x 4 byte block: in[r] holds bytes (r, c = 0..3); out[c]
// holds bytes (r = 0..3, c).
__device__ __forceinline__ void transpose4(const uint32_t (&in)[4], uint32_t (&out)[4]) {
    const uint32_t a_lo = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);
    const uint32_t a_hi = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);
    const uint32_t b_lo = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
    const uint32_t b_hi = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
    out[0] = __builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u);
    out[1] = __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u);
    out[2] = __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u);
}

// One block's staging data in registers (a thread's K piece and V sub-block).
struct Stage {
    uintx4 k;
    uint32_t v[4];
};

// DBG: also write the logits (s_out) and the probability codes (p_out), each
// only if its pointer is not NULL (tests only).
// Four workgroups per CU: the compiler keeps the kernel to 128 registers, so
// four waves share a SIMD instead of three (it had taken 132 for D = 128):
// 75.4 -> 58.8 us at B = 8, L = 512, H = 32, D = 128, the VALU-bound softmax
// having more waves to interleave.  The test-only variant keeps two, which
// it needs to stay out of scratch memory.
template <int D, bool DBG>
__global__ __launch_bounds__(64 * NW, DBG ? 2 : 4) void mha_int8_kernel(
    const int8_t* __restrict__ Q, const int8_t* __restrict__ K, const int8_t* __restrict__ V,
    const uint16_t* __restrict__ bias, int8_t* __restrict__ O, int32_t* __restrict__ s_out,
    int8_t* __restrict__ p_out, int H, int Lq, int Lk, float alpha, float pv_scale, float out_mult,
    uint32_t flags) {
    constexpr int DS = D / 32;  // 32-wide k steps of S, 32-row d tiles of O
    __shared__ __attribute__((aligned(16))) MhaLds<D> L;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int hh = lane >> 5, c32 = lane & 31;
    // Workgroups are dealt to the eight XCDs round-robin by linear id.  When
    // the (batch, head) pairs come in multiples of eight, id L runs query tile
    // (L / 8) % tiles of pair 8 ((L / 8) / tiles) + L % 8, so all tiles of one
    // head share an XCD and read its K and V through one L2.
    const int ntile = gridDim.x, nbh = gridDim.y * gridDim.z;
    int tile = blockIdx.x, b = blockIdx.z, h = blockIdx.y;
    if (nbh % 8 == 0) {
        const int L = blockIdx.x + ntile * (blockIdx.y + gridDim.y * blockIdx.z);
        const int slot = L >> 3, bh = (slot / ntile) * 8 + (L & 7);
        tile = slot % ntile;
        b = bh / H;
        h = bh % H;
    }
    const int q = tile * QB + wave * 32 + c32;  // this lane's query
    const int qc = q < Lq ? q : Lq - 1;
    // element offsets fit 32 bits (B * max(Lq, Lk) * H * D < 2^31 is checked at launch)
    const uint32_t rs = (uint32_t)H * D;  // bytes between consecutive tokens
    const uint32_t kvbase = (uint32_t)b * Lk * rs + (uint32_t)h * D;
    const int nkb = (Lk + KB - 1) / KB;
    const int nfull = Lk / KB;              // blocks with no key past Lk
    // exponents in base 2: e = exp2(fl(S) * a2 - m2) with a2 = fl(alpha * log2(e)) and
    // m2 = fl(fl(max S) * a2), one fused multiply-add per element (alpha > 0, so the
    // maximum of the scaled logits is the scaled maximum)
    const float a2 = alpha * LOG2E;

    intx4 qf[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s)
        qf[s] = *reinterpret_cast<const intx4*>(Q + (((uint32_t)b * Lq + qc) * rs + (uint32_t)h * D + 32 * s + 16 * hh));

    // Staging: thread t < 2D copies K piece t (row t / (D/16), 16 bytes) and
    // transposes V sub-block t (keys 4 (t / (D/4)) + 0..3, channels
    // 4 (t % (D/4)) + 0..3).  Key rows past Lk repeat row Lk - 1: their
    // logits are masked and their probabilities are 0.  A block's loads are
    // issued before the previous block's compute and written to the other
    // LDS buffer after it.
    const bool stager = tid < 2 * D;
    const int kr = tid / (D / 16), kp = tid % (D / 16);
    const int vg = tid / (D / 4), vd = tid % (D / 4);
    const int vdw = 4 * (vg & 1) + (vg >> 1);  // dword of key group vg in the permuted order
    auto key_off = [&](int kb, int r) {
        const int k = kb * KB + r;
        return kvbase + (uint32_t)(k < Lk ? k : Lk - 1) * rs;
    };
    auto load = [&](Stage& st, int kb, bool with_v) {
        if (stager) {
            st.k = *reinterpret_cast<const uintx4*>(K + (key_off(kb, kr) + 16 * kp));
            if (with_v) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    st.v[r] = *reinterpret_cast<const uint32_t*>(V + (key_off(kb, 4 * vg + r) + 4 * vd));
            }
        }
    };
    auto store = [&](const Stage& st, int buf, bool with_v) {
        if (stager) {
            *reinterpret_cast<uintx4*>(&L.k[buf][kr][16 * kp]) = st.k;
            if (with_v) {
                uint32_t t[4];
                transpose4(st.v, t);
#pragma unroll
                for (int c = 0; c < 4; ++c) L.vt[buf][4 * vd + c][vdw] = t[c];
            }
        }
    };
    auto barrier = [&]() {
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
    };
    // S^T of the block staged in buf for this wave's 32 queries
    auto scores = [&](int buf) {
        intx16 acc;
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = 0;
#pragma unroll
        for (int s = 0; s < DS; ++s) {
            const intx4 a = *reinterpret_cast<const intx4*>(&L.k[buf][c32][32 * s + 16 * hh]);
            acc = mfma_i8(a, qf[s], acc);
        }
        return acc;
    };
    // Runs full(kb, buf) over the blocks below nfull and masked(kb, buf) over
    // the rest, with the staging pipeline around them.  Two loops rather than
    // one with a branch per block: the accumulators then stay in place (with
    // a join in the loop body the compiler copied all of them every block).
    auto sweep = [&](bool with_v, auto full, auto masked) {
        Stage st;
        load(st, 0, with_v);
        store(st, 0, with_v);
        barrier();
        int kb = 0;
        for (; kb < nfull; ++kb) {
            load(st, kb + 1 < nkb ? kb + 1 : kb, with_v);
            full(kb, kb & 1);
            store(st, (kb + 1) & 1, with_v);
            barrier();
        }
        for (; kb < nkb; ++kb) {
            load(st, kb + 1 < nkb ? kb + 1 : kb, with_v);
            masked(kb, kb & 1);
            store(st, (kb + 1) & 1, with_v);
            barrier();
        }
    };

    // A block from nfull on (the last one, when Lk is not a multiple of 32)
    // tests each key against Lk: the block bodies are instantiated with and
    // without the test.
    typedef std::integral_constant<bool, true> Masked;
    typedef std::integral_constant<bool, false> Full;
    auto valid = [&](auto masked, int kb, int j) {
        if constexpr (decltype(masked)::value) return kb * KB + key_of(j, lane) < Lk;
        else return true;
    };

    // ---- pass 1: running maximum of S and sum l of exp2(S a2 - m2), online over the blocks
    int ms = INT32_MIN;
    float m2 = -INFINITY, lsum = 0.f;
    auto pass1 = [&](auto masked, int kb, int buf) {
        const intx16 acc = scores(buf);
        int bm = INT32_MIN;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            bm = max(bm, valid(masked, kb, j) ? acc[j] : INT32_MIN);
            if constexpr (DBG) {
                const int key = kb * KB + key_of(j, lane);
                if (s_out && q < Lq && key < Lk) s_out[(((size_t)b * H + h) * Lq + q) * Lk + key] = acc[j];
            }
        }
        bm = max(bm, __shfl_xor(bm, 32));
        if (bm > ms) {  // the maximum grew: rescale the sum
            const float mn = (float)bm * a2;
            lsum = lsum * __builtin_amdgcn_exp2f(m2 - mn);
            m2 = mn;
            ms = bm;
        }
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf((float)acc[j], a2, -m2));
            part += valid(masked, kb, j) ? e : 0.f;
        }
        lsum += part;
    };
    sweep(false, [&](int kb, int buf) { pass1(Full(), kb, buf); }, [&](int kb, int buf) { pass1(Masked(), kb, buf); });
    const float l = lsum + __shfl_xor(lsum, 32);
    const float cq = 127.0f / l;  // code = rne(e * fl(127 / l))

    // ---- pass 2: int8 probabilities and O^T = V^T P^T
    intx16 oacc[DS];
#pragma unroll
    for (int t = 0; t < DS; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[t][j] = 0;
    auto pass2 = [&](auto masked, int kb, int buf) {
        const intx16 acc = scores(buf);
        uint32_t pk[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf((float)acc[j], a2, -m2));
            // e <= 1 and cq <= 127, so e * cq lies in [0, 127]; the byte conversion rounds
            // it to nearest, ties to even (checked on gfx950 for every float in [0, 128])
            const float c = valid(masked, kb, j) ? e * cq : 0.f;
            pk[j >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(c, j & 3, pk[j >> 2]);
            if constexpr (DBG) {
                const int key = kb * KB + key_of(j, lane);
                if (p_out && q < Lq && key < Lk)
                    p_out[(((size_t)b * H + h) * Lq + q) * Lk + key] = (int8_t)((pk[j >> 2] >> (8 * (j & 3))) & 0xffu);
            }
        }
        const intx4 pb = {(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
#pragma unroll
        for (int t = 0; t < DS; ++t) {
            const intx4 a = *reinterpret_cast<const intx4*>(&L.vt[buf][32 * t + c32][4 * hh]);
            oacc[t] = mfma_i8(a, pb, oacc[t]);
        }
    };
    sweep(true, [&](int kb, int buf) { pass2(Full(), kb, buf); }, [&](int kb, int buf) { pass2(Masked(), kb, buf); });

    // ---- epilogue: t = fl(acc) * pv_scale (+ bias), code = clamp(rne(t * out_mult), +-127);
    // registers 4g .. 4g + 3 of d tile t are channels 32 t + 8 g + 4 (lane / 32) + 0..3
    if (q >= Lq) return;
    int8_t* orow = O + (((uint32_t)b * Lq + q) * rs + (uint32_t)h * D);
#pragma unroll
    for (int t = 0; t < DS; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = 32 * t + 8 * g + 4 * hh;
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = (float)oacc[t][4 * g + i];
                v = v * pv_scale;
                if (flags & QGEMM_EPI_BIAS) v = v + h2f(bias[h * D + d0 + i]);
                v = __builtin_rintf(v * out_mult);
                v = fminf(fmaxf(v, -127.0f), 127.0f);
                word |= ((uint32_t)(int)v & 0xffu) << (8 * i);
            }
            *reinterpret_cast<uint32_t*>(orow + d0) = word;
        }
}

template <int D>
void launch_mha(dim3 grid, hipStream_t st, const int8_t* Q, const int8_t* K, const int8_t* V, const uint16_t* bias,
                int8_t* O, int32_t* s_out, int8_t* p_out, int H, int Lq, int Lk, float alpha, float pv_scale,
                float out_mult, uint32_t flags) {
    if (s_out || p_out)
        hipLaunchKernelGGL((mha_int8_kernel<D, true>), grid, dim3(64 * NW), 0, st, Q, K, V, bias, O, s_out, p_out,
                           H, Lq, Lk, alpha, pv_scale, out_mult, flags);
    else
        hipLaunchKernelGGL((mha_int8_kernel<D, false>), grid, dim3(64 * NW), 0, st, Q, K, V, bias, O, s_out,
                           p_out, H, Lq, Lk, alpha, pv_scale, out_mult, flags);
}

}  // namespace

extern "C" int32_t mha_int8(const int8_t* Q, const int8_t* K, const int8_t* V, const uint16_t* bias,
                            int8_t* O, int32_t* s_out, int8_t* p_out, int32_t B, int32_t H, int32_t Lq,
                            int32_t Lk, int32_t D, float alpha, float pv_scale, float out_mult,
                            uint32_t flags, void* stream) {
    if (B < 0 || H < 0 || Lq < 0 || Lk < 0 || D < 0) return QGEMM_BAD_SHAPE;
    if (B == 0 || H == 0 || Lq == 0) return QGEMM_OK;
    if (!Q || !K || !V || !O) return QGEMM_NULL_PTR;
    if ((flags & QGEMM_EPI_BIAS) && !bias) return QGEMM_NULL_PTR;
    if (Lk == 0) return QGEMM_BAD_SHAPE;  // softmax over no keys
    if (!(alpha > 0.f) || !(alpha < INFINITY)) return QGEMM_BAD_SHAPE;  // a positive, finite logit factor
    if (D != 64 && D != 128) return QGEMM_UNSUPPORTED;
    if (flags & ~(uint32_t)QGEMM_EPI_BIAS) return QGEMM_UNSUPPORTED;
    if (Lk > 133143) return QGEMM_UNSUPPORTED;  // sum_j P V must fit int32: Lk * 127 * 127 < 2^31
    if (B > 65535 || H > 65535) return QGEMM_UNSUPPORTED;
    // 32-bit element offsets inside the kernel
    if ((int64_t)B * (Lq > Lk ? Lq : Lk) * H * D >= ((int64_t)1 << 31)) return QGEMM_UNSUPPORTED;
    if (!qgh::aligned(Q, 16) || !qgh::aligned(K, 16) || !qgh::aligned(V, 16) || !qgh::aligned(O, 16) ||
        (bias && !qgh::aligned(bias, 4)) || (s_out && !qgh::aligned(s_out, 4)))
        return QGEMM_MISALIGNED;
    dim3 grid((Lq + QB - 1) / QB, H, B);
    if (D == 64)
        launch_mha<64>(grid, (hipStream_t)stream, Q, K, V, bias, O, s_out, p_out, H, Lq, Lk, alpha, pv_scale,
                       out_mult, flags);
    else
        launch_mha<128>(grid, (hipStream_t)stream, Q, K, V, bias, O, s_out, p_out, H, Lq, Lk, alpha, pv_scale,
                        out_mult, flags);
    return qgh::launch_status();
}
