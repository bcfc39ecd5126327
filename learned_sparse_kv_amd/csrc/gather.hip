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
