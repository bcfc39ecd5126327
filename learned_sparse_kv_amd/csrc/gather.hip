// Device-to-device page gather (gfx950): copies whole chunk pages from the
// cold tier into HBM slots when the cold tier is itself in device memory.
// Selected chunks move from the cold pool into GPU memory (cjcn.com.cn
// explainer, section 二).  One block per page, 16-byte coalesced copies.
#include "lsa_internal.h"

namespace {

__global__ __launch_bounds__(256) void k_gather(const int32_t* __restrict__ pairs,
                                                const uint8_t* __restrict__ src,
                                                uint8_t* __restrict__ dst, int64_t page_bytes) {
    const int32_t sp = pairs[2 * blockIdx.x], dp = pairs[2 * blockIdx.x + 1];
    const uint4* s = (const uint4*)(src + (int64_t)sp * page_bytes);
    uint4* d = (uint4*)(dst + (int64_t)dp * page_bytes);
    const int64_t n = page_bytes / 16;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) d[i] = s[i];
}

}  // namespace

hipError_t launch_gather(const int32_t* pairs, int n_pairs, const void* src, void* dst,
                         int64_t page_bytes, hipStream_t s) {
    if (n_pairs <= 0) return hipSuccess;
    timing_begin("k_gather", s);
    hipLaunchKernelGGL(k_gather, dim3(n_pairs), dim3(256), 0, s, pairs, (const uint8_t*)src,
                       (uint8_t*)dst, page_bytes);
    timing_end("k_gather", s);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Diagnostic: a plain streaming read of a device buffer (8 x 16-byte loads
// in flight per lane, grid-stride), the achievable-read-bandwidth line the
// kernels' HBM figures are compared with.  The loaded words are folded
// into one value so that the loads stay.
// ----------------------------------------------------------------------------
namespace {

constexpr int kReadU = 8;

__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ src, int64_t n16,
                                                     uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * 256 * kReadU;
    for (int64_t base = (int64_t)blockIdx.x * 256 * kReadU + threadIdx.x; base < n16; base += stride) {
        uint4 v[kReadU];
#pragma unroll
        for (int u = 0; u < kReadU; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            v[u] = i < n16 ? src[i] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kReadU; ++u) acc ^= v[u].x + v[u].y + v[u].z + v[u].w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;  // practically never; keeps the loads
}

}  // namespace

extern "C" lsa_status lsa_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (!src || !sink || ((uintptr_t)src & 15u) || bytes % 16) return LSA_ERR_INVALID_ARG;
    if (bytes == 0) return LSA_OK;
    hipStream_t s = (hipStream_t)stream;
    timing_begin("k_stream_read", s);
    hipLaunchKernelGGL(k_stream_read, dim3(2048), dim3(256), 0, s, (const uint4*)src,
                       (int64_t)(bytes / 16), sink);
    timing_end("k_stream_read", s);
    return hipGetLastError() == hipSuccess ? LSA_OK : LSA_ERR_HIP;
}
