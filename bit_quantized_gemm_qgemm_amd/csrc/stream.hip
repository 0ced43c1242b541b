// Measurement aid: a plain streaming read of a device buffer with 16-byte
// non-temporal loads per lane, the achievable-HBM-read reference against which
// the memory-bound kernels (decode GEMV, quant / dequant) are read.  It does
// nothing the quantized-GEMM method needs.
#include "common.hpp"

namespace {

using namespace qg;

constexpr int kLoads = 8;  // 16-byte loads per lane, all issued before the first wait

__global__ __launch_bounds__(256) void stream_read_kernel(const uintx4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
    const size_t base = (size_t)blockIdx.x * kLoads * 256 + threadIdx.x;
    uintx4 v[kLoads];
    if (base + (size_t)(kLoads - 1) * 256 < n16) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) v[i] = ldg_nt(p + base + (size_t)i * 256);
    } else {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const size_t j = base + (size_t)i * 256;
            v[i] = j < n16 ? ldg_nt(p + j) : uintx4{0u, 0u, 0u, 0u};
        }
    }
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    // a store that depends on every loaded byte keeps the loads; it almost never happens
    if (x == 0x9e3779b9u) sink[0] = x;
}

}  // namespace

extern "C" int32_t qgemm_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (bytes == 0) return QGEMM_OK;
    if (!buf || !sink) return QGEMM_NULL_PTR;
    if (bytes % 16 != 0) return QGEMM_BAD_SHAPE;
    if (!qgh::aligned(buf, 16) || !qgh::aligned(sink, 4)) return QGEMM_MISALIGNED;
    const size_t n16 = bytes / 16;
    const size_t blocks = (n16 + kLoads * 256 - 1) / (kLoads * 256);
    if (blocks > 0x7fffffff) return QGEMM_UNSUPPORTED;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const uintx4*>(buf), n16, sink);
    return qgh::launch_status();
}
