// Chunk scoring and threshold selection (gfx950).
//
// The memory indexer's lookahead score between the current query state and
// each history chunk's compressed index key is a head-fused matching score
// through a sigmoid (gist.science summary, section 2.1); every chunk whose
// score exceeds 0.5 is fetched (cjcn.com.cn explainer, section 二).  The
// score's logit is a dot product of one KIComp row with the head-fused query
//     qbar = sum_h w_h q_h,   z_c = fma(s_c, qbar . k_c, b),
// and sigmoid(z) > 0.5 exactly when z > 0.
//
// Arithmetic order (shared by definition with the CPU oracle, not by code):
// fp32, IEEE fma chains from +0 over h (fusion) and over i (dot product), no
// denormal flush, no other contraction.  One lane owns one chunk so each
// dot product is a plain sequential chain.
//
// The union over several indexer layers (OR mode: a chunk is fetched when
// any layer's score exceeds 0.5; cjcn.com.cn explainer, section 四;
// gist.science summary, section 2.4) scores the layers one after another
// into the same z, each later layer keeping the per-chunk maximum, so that
// z > theta exactly when some layer's logit is.
//
// k_score streams KIComp from HBM: each wave takes about two tiles of 64
// chunks of one request; rows come in with coalesced 16-byte loads (the next
// tile in flight while the current one is scored), go through a wave-private
// LDS tile, and are read back one row per lane.  1 (bf16) to 2 (fp8) flop
// per byte: HBM-bound.  The window pipeline has it record, per tile of 64
// chunks, the mask of chunks with z > theta and its count, from which
// k_select_tiles writes the ordered selection with one wave per tile.
#include "lsa_internal.h"

namespace {

__device__ __forceinline__ float bf16f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

template <int QDT>
__global__ void k_fuse_query(GeomDev g, const void* __restrict__ q, const float* __restrict__ w,
                             int H, int d, float* __restrict__ qbar) {
    const int r = blockIdx.x;
    const int i = threadIdx.x;
    if (i >= d) return;
    float acc = 0.0f;
#pragma unroll 16
    for (int h = 0; h < H; ++h) {
        const size_t e = ((size_t)r * H + h) * d + i;
        float qv;
        if constexpr (QDT == LSA_F32)
            qv = ((const float*)q)[e];
        else
            qv = bf16f(((const uint16_t*)q)[e]);
        acc = __builtin_fmaf(w[(size_t)r * H + h], qv, acc);
    }
    qbar[(size_t)r * d + i] = acc;
}

// Dot product of a row held as 16-byte pieces (ROWB bytes) with qbar (in
// LDS, read as float4 broadcasts), as a sequential fma chain in element order.
template <int KDT, int D>
__device__ __forceinline__ float row_dot(const uint4* __restrict__ row,
                                         const float4* __restrict__ qb) {
    float acc = 0.0f;
    if constexpr (KDT == LSA_F32) {
#pragma unroll 4
        for (int j = 0; j < D / 4; ++j) {
            const uint4 v = row[j];
            const float4 q = qb[j];
            acc = __builtin_fmaf(q.x, __uint_as_float(v.x), acc);
            acc = __builtin_fmaf(q.y, __uint_as_float(v.y), acc);
            acc = __builtin_fmaf(q.z, __uint_as_float(v.z), acc);
            acc = __builtin_fmaf(q.w, __uint_as_float(v.w), acc);
        }
    } else if constexpr (KDT == LSA_BF16) {
#pragma unroll 2
        for (int j = 0; j < D / 8; ++j) {
            const uint4 v = row[j];
            const float4 qa = qb[2 * j], qc = qb[2 * j + 1];
            acc = __builtin_fmaf(qa.x, __uint_as_float(v.x << 16), acc);
            acc = __builtin_fmaf(qa.y, __uint_as_float(v.x & 0xffff0000u), acc);
            acc = __builtin_fmaf(qa.z, __uint_as_float(v.y << 16), acc);
            acc = __builtin_fmaf(qa.w, __uint_as_float(v.y & 0xffff0000u), acc);
            acc = __builtin_fmaf(qc.x, __uint_as_float(v.z << 16), acc);
            acc = __builtin_fmaf(qc.y, __uint_as_float(v.z & 0xffff0000u), acc);
            acc = __builtin_fmaf(qc.z, __uint_as_float(v.w << 16), acc);
            acc = __builtin_fmaf(qc.w, __uint_as_float(v.w & 0xffff0000u), acc);
        }
    } else {  // fp8 e4m3fn (OCP), converted exactly to fp32 by the hardware
#pragma unroll 2
        for (int j = 0; j < D / 16; ++j) {
            const uint4 v = row[j];
            const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float4 q = qb[4 * j + e];
                const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wds[e], false);
                const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wds[e], true);
                acc = __builtin_fmaf(q.x, lo[0], acc);
                acc = __builtin_fmaf(q.y, lo[1], acc);
                acc = __builtin_fmaf(q.z, hi[0], acc);
                acc = __builtin_fmaf(q.w, hi[1], acc);
            }
        }
    }
    return acc;
}

// Waves per block so that the block's LDS tiles stay near 36 KB.
template <int KDT, int D>
constexpr int score_waves() {
    constexpr int rowb = D * (KDT == LSA_F32 ? 4 : (KDT == LSA_BF16 ? 2 : 1));
    return rowb <= 128 ? 4 : (rowb <= 256 ? 2 : 1);
}

// Grid (X, B): the waves of block column x of request r take the request's
// tiles x*nw + wave, stepping by X*nw, and load the next tile into registers
// while the current one is scored from LDS.  The launcher gives every wave
// one tile of the longest request (all loads of the pass in flight at once:
// faster than two tiles a wave, which kept the second one's loads behind the
// first).
template <int KDT, int D>
__global__ __launch_bounds__((64 * score_waves<KDT, D>())) void k_score(
    GeomDev g, const uint8_t* __restrict__ kic, const float* __restrict__ kscale,
    const float* __restrict__ qbar, const float* __restrict__ bias, float* __restrict__ z,
    int combine, float theta, uint64_t* __restrict__ tmask, int32_t* __restrict__ tcount) {
    constexpr int kScoreWaves = score_waves<KDT, D>();
    constexpr int EB = KDT == LSA_F32 ? 4 : (KDT == LSA_BF16 ? 2 : 1);
    constexpr int ROWB = D * EB;          // bytes per KIComp row
    constexpr int PIECES = ROWB / 16;     // 16-byte pieces per row = per lane per tile
    constexpr int STRIDE = ROWB + 16;     // padded LDS row (conflict-free reads)
    __shared__ __attribute__((aligned(16))) uint8_t tile[kScoreWaves][64 * STRIDE];
    __shared__ __attribute__((aligned(16))) float qs[D];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int r = blockIdx.y;
    const int nh = g.nhist[r];
    const int ntile = (nh + 63) >> 6;
    const int step = gridDim.x * kScoreWaves;
    if ((int)blockIdx.x * kScoreWaves >= ntile) return;  // uniform across the block
    for (int i = threadIdx.x; i < D; i += blockDim.x) qs[i] = qbar[(size_t)r * D + i];
    __syncthreads();
    int t = blockIdx.x * kScoreWaves + wv;
    if (t >= ntile) return;  // whole wave leaves together
    const int64_t off = g.chunk_off[r];
    const float br = bias[r];
    uint8_t* lt = tile[wv];
    uint4 raw[PIECES];
    float sc = 1.0f;
    // tile tt: rows off + 64tt .. (nvalid of them), contiguous; lane takes the
    // 16-byte pieces j*64 + lane, and the scale of row 64tt + lane
    auto fetch = [&](int tt) {
        const int nvalid = min(64, nh - tt * 64);
        const uint4* src = (const uint4*)(kic + (off + (int64_t)tt * 64) * ROWB);
#pragma unroll
        for (int j = 0; j < PIECES; ++j) {
            const int piece = j * 64 + lane;
            raw[j] = (piece / PIECES < nvalid) ? src[piece] : make_uint4(0, 0, 0, 0);
        }
        if constexpr (KDT == LSA_FP8_E4M3FN)
            sc = lane < nvalid ? kscale[off + (int64_t)tt * 64 + lane] : 1.0f;
    };
    fetch(t);
    for (; t < ntile; t += step) {
#pragma unroll
        for (int j = 0; j < PIECES; ++j) {
            const int piece = j * 64 + lane;
            *(uint4*)(lt + (piece / PIECES) * STRIDE + (piece % PIECES) * 16) = raw[j];
        }
        const float s = sc;
        if (t + step < ntile) fetch(t + step);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int c = t * 64 + lane;
        const float acc = row_dot<KDT, D>((const uint4*)(lt + lane * STRIDE), (const float4*)qs);
        float zf = -INFINITY;
        if (c < nh) {
            const float zl = __builtin_fmaf(s, acc, br);
            // union over indexer layers: keep the earlier logit unless this one
            // is strictly larger (the per-chunk max, first of equals)
            if (combine) {
                const float zo = z[off + c];
                zf = zl > zo ? zl : zo;
            } else {
                zf = zl;
            }
            z[off + c] = zf;
        }
        if (tmask) {  // uniform
            const uint64_t m = __ballot(c < nh && zf > theta);
            if (lane == 0) {
                tmask[g.tile_off[r] + t] = m;
                tcount[g.tile_off[r] + t] = __popcll(m);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();  // the LDS tile is rewritten next round
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// Ordered stream compaction of {c : z_c > theta} per request: wave ballot,
// in-wave rank by popcount, wave totals through LDS.  One block per request;
// the first kSelPre rounds of logits are loaded before any is compacted.
constexpr int kSelPre = 16;

__global__ __launch_bounds__(1024) void k_select(GeomDev g, const float* __restrict__ z,
                                                 float theta, int32_t* __restrict__ sel,
                                                 int32_t* __restrict__ cnt) {
    __shared__ int wsum[16];
    const int r = blockIdx.x;
    const int n = g.nhist[r];
    const int64_t off = g.chunk_off[r];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int base = 0;
    for (int c00 = 0; c00 < n; c00 += 1024 * kSelPre) {
        bool fl[kSelPre];
#pragma unroll
        for (int u = 0; u < kSelPre; ++u) {
            const int c = c00 + u * 1024 + (int)threadIdx.x;
            fl[u] = (c < n) && (z[off + c] > theta);
        }
#pragma unroll
        for (int u = 0; u < kSelPre; ++u) {
            const int c0 = c00 + u * 1024;
            if (c0 < n) {  // uniform
                const int c = c0 + (int)threadIdx.x;
                const bool f = fl[u];
                const uint64_t m = __ballot(f);
                const int pre = __popcll(m & ((1ull << lane) - 1ull));
                if (lane == 0) wsum[wv] = __popcll(m);
                __syncthreads();
                int wpre = 0, tot = 0;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int v = wsum[i];
                    wpre += (i < wv) ? v : 0;
                    tot += v;
                }
                if (f) sel[off + base + wpre + pre] = c;
                base += tot;
                __syncthreads();
            }
        }
    }
    if (threadIdx.x == 0) cnt[r] = base;
}

// Ordered compaction from the tile masks: one wave per tile of 64 chunks.
// The wave adds the counts of its request's earlier tiles (a fixed-order
// lane tree), then writes the chunk ids of its mask at their ranks; the wave
// of a request's last tile writes the request's count.  Requests without
// history chunks get their zero count from block 0.
__global__ __launch_bounds__(256) void k_select_tiles(GeomDev g, const uint64_t* __restrict__ tmask,
                                                     const int32_t* __restrict__ tcount,
                                                     int32_t* __restrict__ sel,
                                                     int32_t* __restrict__ cnt) {
    const int lane = threadIdx.x & 63;
    const int gt = blockIdx.x * 4 + (threadIdx.x >> 6);  // tile over all requests
    if (blockIdx.x == 0 && threadIdx.x < g.B && g.nhist[threadIdx.x] == 0) cnt[threadIdx.x] = 0;
    if (gt >= g.tile_off[g.B]) return;  // whole wave
    int r = 0;
    while (g.tile_off[r + 1] <= gt) ++r;  // uniform
    const int t0 = g.tile_off[r], t = gt - t0;
    const uint64_t m = tmask[gt];
    int pre = 0;
    for (int i = lane; i < t; i += 64) pre += tcount[t0 + i];
    for (int o = 32; o > 0; o >>= 1) pre += __shfl_xor(pre, o);
    const int64_t off = g.chunk_off[r];
    if ((m >> lane) & 1ull) sel[off + pre + __popcll(m & ((1ull << lane) - 1ull))] = t * 64 + lane;
    if (t == g.tile_off[r + 1] - t0 - 1 && lane == 0) cnt[r] = pre + __popcll(m);
}

}  // namespace

hipError_t launch_fuse_query(const GeomDev& g, const void* q, lsa_dtype q_dt, const float* w,
                             int H, int d, float* qbar, hipStream_t s) {
    timing_begin("k_fuse_query", s);
    if (q_dt == LSA_F32)
        hipLaunchKernelGGL(k_fuse_query<LSA_F32>, dim3(g.B), dim3(128), 0, s, g, q, w, H, d, qbar);
    else
        hipLaunchKernelGGL(k_fuse_query<LSA_BF16>, dim3(g.B), dim3(128), 0, s, g, q, w, H, d, qbar);
    timing_end("k_fuse_query", s);
    return hipGetLastError();
}

hipError_t launch_score(const GeomDev& g, const void* kic, lsa_dtype kdt, const float* kscale,
                        const float* qbar, const float* bias, int d, float* z, hipStream_t s,
                        bool combine, float theta, uint64_t* tmask, int32_t* tcount) {
    const int tiles = g.tile_off[g.B];
    if (tiles == 0) return hipSuccess;
    int mt = 0;  // tiles of the longest request
    for (int r = 0; r < g.B; ++r) mt = g.tile_off[r + 1] - g.tile_off[r] > mt ? g.tile_off[r + 1] - g.tile_off[r] : mt;
    const uint8_t* k = (const uint8_t*)kic;
#define LSA_SCORE_CASE(KDT, D)                                                                  \
    if (kdt == KDT && d == D) {                                                                 \
        constexpr int nw = score_waves<KDT, D>();                                               \
        timing_begin("k_score", s);                                                             \
        hipLaunchKernelGGL((k_score<KDT, D>), dim3((mt + nw - 1) / nw, g.B),                     \
                           dim3(64 * nw), 0, s,                                                 \
                           g, k, kscale, qbar, bias, z, combine ? 1 : 0, theta, tmask, tcount); \
        timing_end("k_score", s);                                                               \
        return hipGetLastError();                                                               \
    }
    LSA_SCORE_CASE(LSA_F32, 64)
    LSA_SCORE_CASE(LSA_F32, 128)
    LSA_SCORE_CASE(LSA_BF16, 64)
    LSA_SCORE_CASE(LSA_BF16, 128)
    LSA_SCORE_CASE(LSA_FP8_E4M3FN, 64)
    LSA_SCORE_CASE(LSA_FP8_E4M3FN, 128)
#undef LSA_SCORE_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_select(const GeomDev& g, const float* z, float theta, int32_t* sel,
                         int32_t* cnt, hipStream_t s) {
    timing_begin("k_select", s);
    hipLaunchKernelGGL(k_select, dim3(g.B), dim3(1024), 0, s, g, z, theta, sel, cnt);
    timing_end("k_select", s);
    return hipGetLastError();
}

hipError_t launch_select_tiles(const GeomDev& g, const uint64_t* tmask, const int32_t* tcount,
                               int32_t* sel, int32_t* cnt, hipStream_t s) {
    const int tiles = g.tile_off[g.B];
    timing_begin("k_select_tiles", s);
    hipLaunchKernelGGL(k_select_tiles, dim3(tiles > 0 ? (tiles + 3) / 4 : 1), dim3(256), 0, s, g,
                       tmask, tcount, sel, cnt);
    timing_end("k_select_tiles", s);
    return hipGetLastError();
}
