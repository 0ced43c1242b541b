// Measurement aid: a plain streaming read of a device buffer with 16-byte
// non-temporal loads per lane, the achievable-HBM-read reference against which
// the memory-bound kernels (decode GEMV, quant / dequant) are read.  It does
// nothing the quantized-GEMM method needs.
#include "common.hpp"

namespace {

using namespace qg;

// 16-byte loads per lane (all issued before the first wait) and threads per
// workgroup: the fastest of a sweep at a 23 MB working set (16 rotated
// buffers, plain launches): 2 x 128 4.72-4.78 us, 1 x 256 4.77-4.85,
// 2 x 256 4.82, 2 x 512 4.85, 3 x 256 4.89, 8 x 256 4.92-4.94,
// 16 x 256 5.27 -- many short workgroups stream best
constexpr int kLoads = 2, kThreads = 128;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uintx4* __restrict__ p, size_t n16,
                                                               uint32_t* __restrict__ sink) {
    const size_t base = (size_t)blockIdx.x * kLoads * kThreads + threadIdx.x;
    uintx4 v[kLoads];
    if (base + (size_t)(kLoads - 1) * kThreads < n16) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) v[i] = ldg_nt(p + base + (size_t)i * kThreads);
    } else {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const size_t j = base + (size_t)i * kThreads;
            v[i] = j < n16 ? ldg_nt(p + j) : uintx4{0u, 0u, 0u, 0u};
        }
    }
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    // a store that depends on every loaded byte keeps the loads; it almost never happens
    if (x == 0x9e3779b9u) sink[0] = x;
}

// Read-and-write references with the traffic shapes of the quantizers: each
// lane reads L pieces of RB bytes and writes L pieces of WB bytes derived
// from them, all loads before the first store, both non-temporal (the
// non-temporal stores ran both shapes faster: 5.76 -> 5.56 and 6.18 ->
// 6.03 us at the KV-cache size).  RB = 16, WB = 8
// is the int8 quantizer's shape (16.8 MB of fp16 in, 8.4 MB of codes out at
// the KV-cache size), RB = 8, WB = 16 the dequantizer's.  Four pieces per
// lane in workgroups of 256 threads, each lane's pieces 256 apart: 4.97 to
// 5.01 us (dequant shape) and 5.48 to 5.57 us (quant shape), against 5.86 and
// 5.63 with one or two pieces per lane in 128-thread workgroups and 4.99 and
// 5.84 with the pieces spread over the whole buffer (one box).
template <int RB, int WB, int L>
__global__ __launch_bounds__(256) void stream_copy_kernel(const uint8_t* __restrict__ src,
                                                          uint8_t* __restrict__ dst, size_t n) {
    typedef uint32_t r_t __attribute__((ext_vector_type(RB / 4)));
    typedef uint32_t w_t __attribute__((ext_vector_type(WB / 4)));
    const r_t* in = reinterpret_cast<const r_t*>(src);
    w_t* out = reinterpret_cast<w_t*>(dst);
    const size_t base = (size_t)blockIdx.x * L * 256 + threadIdx.x;
    r_t v[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const size_t j = base + (size_t)i * 256;
        v[i] = j < n ? __builtin_nontemporal_load(in + j) : r_t{};
    }
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const size_t j = base + (size_t)i * 256;
        w_t o;
        if constexpr (RB > WB) {
#pragma unroll
            for (int e = 0; e < WB / 4; ++e) o[e] = v[i][2 * e] ^ v[i][2 * e + 1];
        } else {
#pragma unroll
            for (int e = 0; e < WB / 4; ++e) o[e] = v[i][e % (RB / 4)] + (uint32_t)(e / (RB / 4));
        }
        if (j < n) __builtin_nontemporal_store(o, out + j);
    }
}

}  // namespace

extern "C" int32_t qgemm_stream_copy(const void* src, size_t src_bytes, void* dst, size_t dst_bytes,
                                     void* stream) {
    if (src_bytes == 0 && dst_bytes == 0) return QGEMM_OK;
    if (!src || !dst) return QGEMM_NULL_PTR;
    const bool shrink = dst_bytes * 2 == src_bytes, grow = src_bytes * 2 == dst_bytes;
    if (!(shrink || grow) || src_bytes % 16 != 0 || dst_bytes % 16 != 0) return QGEMM_BAD_SHAPE;
    if (!qgh::aligned(src, 16) || !qgh::aligned(dst, 16)) return QGEMM_MISALIGNED;
    const size_t n = shrink ? src_bytes / 16 : src_bytes / 8;  // lane-steps
    constexpr int L = 4;
    const size_t blocks = (n + (size_t)L * 256 - 1) / ((size_t)L * 256);
    if (blocks > 0x7fffffff) return QGEMM_UNSUPPORTED;
    const auto* s8 = static_cast<const uint8_t*>(src);
    auto* d8 = static_cast<uint8_t*>(dst);
    if (shrink)
        hipLaunchKernelGGL((stream_copy_kernel<16, 8, L>), dim3((unsigned)blocks), dim3(256), 0,
                           (hipStream_t)stream, s8, d8, n);
    else
        hipLaunchKernelGGL((stream_copy_kernel<8, 16, L>), dim3((unsigned)blocks), dim3(256), 0,
                           (hipStream_t)stream, s8, d8, n);
    return qgh::launch_status();
}

extern "C" int32_t qgemm_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (bytes == 0) return QGEMM_OK;
    if (!buf || !sink) return QGEMM_NULL_PTR;
    if (bytes % 16 != 0) return QGEMM_BAD_SHAPE;
    if (!qgh::aligned(buf, 16) || !qgh::aligned(sink, 4)) return QGEMM_MISALIGNED;
    const size_t n16 = bytes / 16;
    const size_t blocks = (n16 + kLoads * kThreads - 1) / (kLoads * kThreads);
    if (blocks > 0x7fffffff) return QGEMM_UNSUPPORTED;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const uintx4*>(buf), n16, sink);
    return qgh::launch_status();
}
