// Growing context (gfx950).  The pages' indexer fires every 64 decode steps
// to predict the history the next 64 steps need (cjcn.com.cn explainer,
// section 二); between two triggers every step adds one token to the recent
// region, and at a trigger the recent region's oldest full chunk joins the
// history.  Both moves are plain copies in 16-byte units; the layouts give
// every request fixed capacities (rec_off[r] = r * recent_cap, chunk_off[r]
// = r * chunk_cap), so no other request's rows move.
#include "lsa_internal.h"

namespace {

// Block r writes request r's newest row: recent row rec_off[r] + R_r - 1.
__global__ void k_append_kv(GeomDev g, const uint8_t* __restrict__ rows, int64_t row_bytes,
                            uint8_t* __restrict__ recent) {
    const int r = blockIdx.x;
    const uint4* src = (const uint4*)(rows + (int64_t)r * row_bytes);
    uint4* dst = (uint4*)(recent + (g.rec_off[r] + g.nrec[r] - 1) * row_bytes);
    for (int i = threadIdx.x; i < row_bytes / 16; i += blockDim.x) dst[i] = src[i];
}

// Grid (X, B).  Request r commits when its recent region holds a full chunk
// beyond the window (R_r >= W + 64): recent rows [64, R_r) go to rows
// [0, R_r - 64) of dst, rows [0, 64) to the KV part of cold page
// chunk_off[r] + N_r, the chunk's index keys to that page at ikey_off, its
// KIComp row to kic.  Otherwise rows [0, R_r) go to dst unchanged.
__global__ void k_commit_chunk(GeomDev g, int64_t row_bytes, int64_t page_bytes, int64_t ikey_off,
                               const uint8_t* __restrict__ rsrc, uint8_t* __restrict__ rdst,
                               uint8_t* __restrict__ cold, int64_t key_row_bytes,
                               const uint8_t* __restrict__ new_ikeys, const float* __restrict__ new_iks,
                               float* __restrict__ ikey_scale, const uint8_t* __restrict__ new_kic,
                               const float* __restrict__ new_kcs, uint8_t* __restrict__ kic,
                               float* __restrict__ kic_scale, int fp8) {
    const int r = blockIdx.y;
    const bool commit = g.nrec[r] >= g.W + 64;
    const int shift = commit ? 64 : 0;
    const int64_t n16 = row_bytes / 16;
    const uint4* src = (const uint4*)(rsrc + g.rec_off[r] * row_bytes);
    uint4* dst = (uint4*)(rdst + g.rec_off[r] * row_bytes);
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t units = (int64_t)(g.nrec[r] - shift) * n16;
    for (int64_t u = tid; u < units; u += stride) dst[u] = src[u + shift * n16];
    if (!commit) return;
    const int64_t c = g.chunk_off[r] + g.nhist[r];
    uint4* pg = (uint4*)(cold + c * page_bytes);
    for (int64_t u = tid; u < 64 * n16; u += stride) pg[u] = src[u];
    const int64_t k16 = key_row_bytes / 16;
    uint4* pk = (uint4*)(cold + c * page_bytes + ikey_off);
    const uint4* sk = (const uint4*)(new_ikeys + (int64_t)r * 64 * key_row_bytes);
    for (int64_t u = tid; u < 64 * k16; u += stride) pk[u] = sk[u];
    const uint4* sr = (const uint4*)(new_kic + (int64_t)r * key_row_bytes);
    uint4* dr = (uint4*)(kic + c * key_row_bytes);
    for (int64_t u = tid; u < k16; u += stride) dr[u] = sr[u];
    if (fp8 && tid == 0) {
        ikey_scale[c] = new_iks[r];
        kic_scale[c] = new_kcs[r];
    }
}

// Grid (X, B).  The window pipeline's commit (growing context): request r
// with f.on[r] moves chunk nhist[r] into its history ahead of the window's
// end, so that the next trigger can score it: recent rows [0, 64) (rows
// rec_off[r] ..) to the KV part of cold page chunk_off[r] + nhist[r], the
// chunk's index keys (ikeys[r]) to that page at ikey_off, its scale to
// ikey_scale.  The recent rows stay where they are until the window ends.
__global__ void k_commit_page(GeomDev g, CommitSet f, int64_t row_bytes, int64_t page_bytes,
                              int64_t ikey_off, const uint8_t* __restrict__ recent,
                              uint8_t* __restrict__ cold, int64_t key_row_bytes,
                              const uint8_t* __restrict__ ikeys, const float* __restrict__ iks,
                              float* __restrict__ ikey_scale) {
    const int r = blockIdx.y;
    if (!f.on[r]) return;
    const int64_t c = g.chunk_off[r] + g.nhist[r];
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const uint4* src = (const uint4*)(recent + g.rec_off[r] * row_bytes);
    uint4* pg = (uint4*)(cold + c * page_bytes);
    for (int64_t u = tid; u < 64 * row_bytes / 16; u += stride) pg[u] = src[u];
    const uint4* sk = (const uint4*)(ikeys + (int64_t)r * 64 * key_row_bytes);
    uint4* pk = (uint4*)(cold + c * page_bytes + ikey_off);
    for (int64_t u = tid; u < 64 * key_row_bytes / 16; u += stride) pk[u] = sk[u];
    if (iks && tid == 0) ikey_scale[c] = iks[r];
}

// Grid (X, B).  Request r with m.n[r] > 0 moves its recent rows
// [src[r], src[r] + n[r]) to [dst[r], ..); the ranges do not overlap.
__global__ void k_compact_recent(RecentMoves m, int64_t row_bytes, uint8_t* __restrict__ recent) {
    const int r = blockIdx.y;
    if (m.n[r] <= 0) return;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const uint4* src = (const uint4*)(recent + m.src[r] * row_bytes);
    uint4* dst = (uint4*)(recent + m.dst[r] * row_bytes);
    for (int64_t u = tid; u < (int64_t)m.n[r] * row_bytes / 16; u += stride) dst[u] = src[u];
}

}  // namespace

hipError_t launch_commit_page(const GeomDev& g, const CommitSet& f, int64_t row_bytes,
                              int64_t page_bytes, int64_t ikey_off, const void* recent, void* cold,
                              int64_t key_row_bytes, const void* ikeys, const float* iks,
                              float* ikey_scale, hipStream_t s) {
    timing_begin("k_commit_page", s);
    hipLaunchKernelGGL(k_commit_page, dim3(16, g.B), dim3(256), 0, s, g, f, row_bytes, page_bytes,
                       ikey_off, (const uint8_t*)recent, (uint8_t*)cold, key_row_bytes,
                       (const uint8_t*)ikeys, iks, ikey_scale);
    timing_end("k_commit_page", s);
    return hipGetLastError();
}

hipError_t launch_compact_recent(int B, const RecentMoves& m, int64_t row_bytes, void* recent,
                                 hipStream_t s) {
    timing_begin("k_compact_recent", s);
    hipLaunchKernelGGL(k_compact_recent, dim3(64, B), dim3(256), 0, s, m, row_bytes, (uint8_t*)recent);
    timing_end("k_compact_recent", s);
    return hipGetLastError();
}

hipError_t launch_append_kv(const GeomDev& g, const void* rows, int64_t row_bytes, void* recent,
                            hipStream_t s) {
    timing_begin("k_append_kv", s);
    hipLaunchKernelGGL(k_append_kv, dim3(g.B), dim3(256), 0, s, g, (const uint8_t*)rows, row_bytes,
                       (uint8_t*)recent);
    timing_end("k_append_kv", s);
    return hipGetLastError();
}

hipError_t launch_commit_chunk(const GeomDev& g, int64_t row_bytes, int64_t page_bytes, int64_t ikey_off,
                               const void* rsrc, void* rdst, void* cold, int64_t key_row_bytes,
                               const void* new_ikeys, const float* new_iks, float* ikey_scale,
                               const void* new_kic, const float* new_kcs, void* kic, float* kic_scale,
                               bool fp8, hipStream_t s) {
    // about 64 blocks per request: each copies ~R_r * row_bytes / 64 bytes
    timing_begin("k_commit_chunk", s);
    hipLaunchKernelGGL(k_commit_chunk, dim3(64, g.B), dim3(256), 0, s, g, row_bytes, page_bytes, ikey_off,
                       (const uint8_t*)rsrc, (uint8_t*)rdst, (uint8_t*)cold, key_row_bytes,
                       (const uint8_t*)new_ikeys, new_iks, ikey_scale, (const uint8_t*)new_kic, new_kcs,
                       (uint8_t*)kic, kic_scale, fp8 ? 1 : 0);
    timing_end("k_commit_chunk", s);
    return hipGetLastError();
}
