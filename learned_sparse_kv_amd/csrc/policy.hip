// Comparison policies of the pages' experiments (gfx950).
//
// The pages compare LSA with a recency-only scheme (the recent 8K tokens
// only), a scheme that keeps a random 10 % of the history chunks, and an
// oracle that keeps the top 50 / 25 / 10 % of the history chunks by the
// attention weight the full decode gives them (cjcn.com.cn explainer,
// sections 五 and 六).  Recency-only is the threshold selection with nothing
// above it.  The other two need:
//
// k_select_ranked  the m best chunks of each request by a per-chunk key (the
//    smallest uint32 keys, or the largest fp32 values), ties to the lower
//    chunk, listed ascending.  One block per request: an exact radix select
//    (four passes of 8 bits over an LDS histogram) finds the m-th best key T
//    and its rank among the keys equal to it; an ordered compaction keeps
//    the keys better than T and that many of the keys equal to T, in chunk
//    order.
//
// k_chunk_ml, k_mass_lse, k_mass_sum  the attention mass of each history
//    chunk under the full softmax of given decode steps' queries over EVERY
//    token of the context:
//        mass_c = sum_j sum_h sum_{s in chunk c} softmax_s(sm q_{j,h} . K_s).
//    The context is cut into pseudo-chunks of 64 tokens: the history chunks,
//    then the recent window.  k_chunk_ml makes one pass over the KV rows per
//    step and writes, per (step, head, pseudo-chunk), the max m and the sum
//    l of exp2 of the scores (log2 units); S^T = K Q^T runs on the matrix
//    cores with the chunk's rows staged in LDS and the step's queries held
//    in registers.  k_mass_lse takes the log-sum-exp per (step, head) over
//    the pseudo-chunks, k_mass_sum the sum over steps and heads of
//    exp2(m - lse) l per pseudo-chunk, in a fixed order; the recent window's
//    pseudo-chunks give the recent mass.  HBM-bound: each step reads every
//    KV row's 1,152 key bytes once.
#include "lsa_internal.h"
#include "mfma_util.h"

#include <algorithm>

namespace {

using namespace lsa_dev;

// ---------------------------------------------------------------------------
constexpr int kRankThreads = 1024;
constexpr int kRankWaves = kRankThreads / 64;

// Rank key: smaller is better.  Largest-value keys map fp32 to an
// order-preserving uint32 (-0 as +0) and complement it.
__device__ __forceinline__ uint32_t rank_key(const void* keys, int kind, int64_t i) {
    if (kind == LSA_RANK_SMALLEST_U32) return ((const uint32_t*)keys)[i];
    const float f = ((const float*)keys)[i];
    uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ~u;
}

// Exclusive block prefix of a per-thread flag; total in *tot.
__device__ __forceinline__ int block_prefix(bool f, int* wsum, int* tot) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint64_t m = __ballot(f);
    const int pre = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wv] = __popcll(m);
    __syncthreads();
    int wp = 0, t = 0;
#pragma unroll
    for (int i = 0; i < kRankWaves; ++i) {
        const int v = wsum[i];
        wp += i < wv ? v : 0;
        t += v;
    }
    __syncthreads();
    *tot = t;
    return wp + pre;
}

__global__ __launch_bounds__(kRankThreads) void k_select_ranked(GeomDev g, const void* __restrict__ keys,
                                                               int kind, RankCounts mc,
                                                               int32_t* __restrict__ sel,
                                                               int32_t* __restrict__ cnt) {
    __shared__ uint32_t hist[256];
    __shared__ int wsum[kRankWaves];
    __shared__ uint32_t s_prefix;
    __shared__ int s_rem;
    const int r = blockIdx.x, tid = threadIdx.x;
    const int n = g.nhist[r];
    const int64_t off = g.chunk_off[r];
    const int m = min(mc.m[r], n);
    if (m <= 0) {
        if (tid == 0) cnt[r] = 0;
        return;
    }
    const bool keep_all = m == n;
    uint32_t T = 0;
    int take_eq = 0;
    if (!keep_all) {
        // the m-th smallest key, 8 bits at a time from the top; rem is its
        // rank among the keys that share the prefix found so far
        uint32_t prefix = 0;
        int rem = m;
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            const uint32_t hmask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
            for (int i = tid; i < 256; i += kRankThreads) hist[i] = 0;
            __syncthreads();
            for (int i = tid; i < n; i += kRankThreads) {
                const uint32_t k = rank_key(keys, kind, off + i);
                if ((k & hmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid == 0) {
                int acc = 0, b = 0;
                for (; b < 255; ++b) {
                    const int c = (int)hist[b];
                    if (acc + c >= rem) break;
                    acc += c;
                }
                s_prefix = prefix | ((uint32_t)b << shift);
                s_rem = rem - acc;
            }
            __syncthreads();
            prefix = s_prefix;
            rem = s_rem;
        }
        T = prefix;
        take_eq = rem;
    }
    // ordered compaction: keys below T, and the first take_eq keys equal to T
    int base = 0, eqbase = 0;
    for (int c0 = 0; c0 < n; c0 += kRankThreads) {
        const int c = c0 + tid;
        const bool in = c < n;
        const uint32_t k = in ? rank_key(keys, kind, off + c) : 0u;
        int etot;
        const int erank = block_prefix(in && !keep_all && k == T, wsum, &etot);
        const bool f = in && (keep_all || k < T || (k == T && eqbase + erank < take_eq));
        int tot;
        const int pos = block_prefix(f, wsum, &tot);
        if (f) sel[off + base + pos] = c;
        base += tot;
        eqbase += etot;
    }
    if (tid == 0) cnt[r] = base;
}

// ---------------------------------------------------------------------------
constexpr int kMlWaves = 4;                   // 16 heads per wave, 64 per block
constexpr int kLatB = 1152;                   // key bytes of a latent row (576 bf16)
constexpr int kKS = kLatB / 64;               // MFMA k-steps (32 dims each)
constexpr int kRowStride = kLatB + 16;        // LDS row stride (spreads banks)
constexpr int kPieces = kLatB / 16;           // 16-byte pieces per row
constexpr int kPerThread = 64 * kPieces / (64 * kMlWaves);  // pieces staged per thread
static_assert(64 * kPieces % (64 * kMlWaves) == 0, "whole pieces per thread");

// Grid (X, n_steps * Hq/64, B).  Block x of request r takes pseudo-chunks
// [x*cpb, (x+1)*cpb) for step j and head group hg; each wave holds its 16
// heads' queries (the B operands) in registers, the block stages one
// pseudo-chunk's 64 key rows in LDS while the next one's are loaded.
__global__ __launch_bounds__(64 * kMlWaves, 1) void k_chunk_ml(
    GeomDev g, MassGeom mg, const uint16_t* __restrict__ q, int Hq, const uint8_t* __restrict__ pages,
    int64_t page_bytes, const int32_t* __restrict__ page_table, const uint8_t* __restrict__ recent,
    int64_t row_bytes, float sl2, int cpb, float2* __restrict__ ml) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[64 * kRowStride];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, lq = lane >> 4;
    const int r = blockIdx.z;
    const int ngrp = Hq >> 6;
    const int j = blockIdx.y / ngrp, hg = blockIdx.y % ngrp;
    const int N = g.nhist[r], NC = mg.nc[r];
    const int c0 = blockIdx.x * cpb;
    if (c0 >= NC) return;  // uniform across the block
    const int c1 = min(NC, c0 + cpb);
    const int head = hg * 64 + wv * 16 + l16;
    const uint16_t* qh = q + (((int64_t)j * g.B + r) * Hq + head) * (kLatB / 2);
    uint4 qb[kKS];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qb[ks] = *(const uint4*)(qh + ks * 32 + lq * 8);

    // the 64 rows of pseudo-chunk c, 16 bytes per piece; rows past the end
    // of the recent window are not loaded (their scores are masked)
    uint4 stg[kPerThread];
    auto rows_of = [&](int c) -> int { return c < N ? 64 : min(64, g.nrec[r] - (c - N) * 64); };
    auto load = [&](int c) __attribute__((always_inline)) {
        const int nt = rows_of(c);
        const uint8_t* base;
        if (c < N) {
            const int64_t pg = page_table ? (int64_t)page_table[g.chunk_off[r] + c] : g.chunk_off[r] + c;
            base = pages + pg * page_bytes;
        } else {
            base = recent + (g.rec_off[r] + (int64_t)(c - N) * 64) * row_bytes;
        }
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int p = i * 64 * kMlWaves + tid;
            const int row = p / kPieces, col = p % kPieces;
            stg[i] = row < nt ? *(const uint4*)(base + row * row_bytes + col * 16) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int p = i * 64 * kMlWaves + tid;
            *(uint4*)(tile + (p / kPieces) * kRowStride + (p % kPieces) * 16) = stg[i];
        }
    };
    load(c0);
    store();
    __syncthreads();
    const int64_t mlb = mg.ml_off[r] + ((int64_t)j * Hq + head) * NC;
    for (int c = c0; c < c1; ++c) {
        if (c + 1 < c1) load(c + 1);
        // S^T for 64 tokens x 16 heads: acc[tb][e] = score of token
        // tb*16 + 4lq + e with head l16
        f32x4_t acc[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const uint4 a = *(const uint4*)(tile + (tb * 16 + l16) * kRowStride + ks * 64 + lq * 16);
                acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                                  __builtin_bit_cast(bf16x8_t, qb[ks]),
                                                                  acc[tb], 0, 0, 0);
            }
        const int nt = rows_of(c);
        float mx = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = (tb * 16 + 4 * lq + e < nt) ? acc[tb][e] * sl2 : -INFINITY;
                acc[tb][e] = x;
                mx = fmaxf(mx, x);
            }
        mx = max_xor32(max_xor16(mx));
        float l = 0.0f;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int e = 0; e < 4; ++e) l += __builtin_amdgcn_exp2f(acc[tb][e] - mx);
        l = add_xor32(add_xor16(l));
        if (lq == 0) ml[mlb + c] = make_float2(mx, l);
        __syncthreads();  // every wave is done with the tile
        if (c + 1 < c1) {
            store();
            __syncthreads();
        }
    }
}

// Grid (Hq/4, n_steps, B), 4 waves: one wave per (step, head) folds the
// request's pseudo-chunk pairs (m, l) into lse2 = M + log2(sum l 2^(m - M)).
__global__ __launch_bounds__(256) void k_mass_lse(GeomDev g, MassGeom mg, int Hq, int n_steps,
                                                  const float2* __restrict__ ml, float* __restrict__ lse2) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int r = blockIdx.z, j = blockIdx.y, h = blockIdx.x * 4 + wv;
    if (h >= Hq) return;
    const int NC = mg.nc[r];
    const float2* p = ml + mg.ml_off[r] + ((int64_t)j * Hq + h) * NC;
    float M = -INFINITY, S = 0.0f;
    for (int c = lane; c < NC; c += 64) {
        const float2 v = p[c];
        const float nm = fmaxf(M, v.x);
        S = S * __builtin_amdgcn_exp2f(M - nm) + v.y * __builtin_amdgcn_exp2f(v.x - nm);
        M = nm;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float om = __shfl_xor(M, o), os = __shfl_xor(S, o);
        const float nm = fmaxf(M, om);
        S = (M == -INFINITY ? 0.0f : S * __builtin_amdgcn_exp2f(M - nm)) +
            (om == -INFINITY ? 0.0f : os * __builtin_amdgcn_exp2f(om - nm));
        M = nm;
    }
    if (lane == 0) lse2[((int64_t)r * n_steps + j) * Hq + h] = M + __log2f(S);
}

// Grid (ceil(max NC / 256), B): one thread per pseudo-chunk sums
// exp2(m - lse2) l over steps and heads in order.  History chunks go to
// mass, the recent window's pseudo-chunks to recbuf.
__global__ __launch_bounds__(256) void k_mass_sum(GeomDev g, MassGeom mg, int Hq, int n_steps,
                                                  const float2* __restrict__ ml,
                                                  const float* __restrict__ lse2, float* __restrict__ mass,
                                                  float* __restrict__ recbuf) {
    extern __shared__ float sl[];  // the request's lse2, n_steps * Hq
    const int r = blockIdx.y;
    const int NC = mg.nc[r], N = g.nhist[r];
    for (int i = threadIdx.x; i < n_steps * Hq; i += blockDim.x) sl[i] = lse2[(int64_t)r * n_steps * Hq + i];
    __syncthreads();
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= NC) return;
    const float2* p = ml + mg.ml_off[r] + c;
    float acc = 0.0f;
    for (int u = 0; u < n_steps * Hq; ++u) {
        const float2 v = p[(int64_t)u * NC];
        acc = __builtin_fmaf(__builtin_amdgcn_exp2f(v.x - sl[u]), v.y, acc);
    }
    if (c < N) mass[g.chunk_off[r] + c] = acc;
    else recbuf[mg.rc_off[r] + (c - N)] = acc;
}

__global__ void k_rec_mass(GeomDev g, MassGeom mg, const float* __restrict__ recbuf,
                           float* __restrict__ rec) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= g.B) return;
    float acc = 0.0f;
    for (int i = 0; i < mg.nc[r] - g.nhist[r]; ++i) acc += recbuf[mg.rc_off[r] + i];
    rec[r] = acc;
}

}  // namespace

void mass_geom(const GeomDev& g, int Hq, int n_steps, MassGeom* mg) {
    int64_t mo = 0, ro = 0;
    for (int r = 0; r < g.B; ++r) {
        const int nr = (g.nrec[r] + 63) / 64;
        mg->nc[r] = g.nhist[r] + nr;
        mg->ml_off[r] = mo;
        mg->rc_off[r] = (int32_t)ro;
        mo += (int64_t)n_steps * Hq * mg->nc[r];
        ro += nr;
    }
    mg->ml_total = mo;
    mg->rc_total = ro;
}

hipError_t launch_select_ranked(const GeomDev& g, const void* keys, int kind, const RankCounts& m,
                                int32_t* sel, int32_t* cnt, hipStream_t s) {
    timing_begin("k_select_ranked", s);
    hipLaunchKernelGGL(k_select_ranked, dim3(g.B), dim3(kRankThreads), 0, s, g, keys, kind, m, sel, cnt);
    timing_end("k_select_ranked", s);
    return hipGetLastError();
}

hipError_t launch_chunk_mass(const GeomDev& g, const MassGeom& mg, const void* q, int Hq, int n_steps,
                             const void* pages, int64_t page_bytes, const int32_t* page_table,
                             const void* recent, int64_t row_bytes, float sm_scale, float* mass,
                             float* rec, float2* ml, float* lse2, float* recbuf, hipStream_t s) {
    int ncmax = 0;
    for (int r = 0; r < g.B; ++r) ncmax = std::max(ncmax, mg.nc[r]);
    if (ncmax == 0) return hipSuccess;
    // about 8 pseudo-chunks per block keeps the query set-up small beside
    // the rows it serves
    const int cpb = 8;
    const float sl2 = sm_scale * 1.4426950408889634f;
    timing_begin("k_chunk_ml", s);
    hipLaunchKernelGGL(k_chunk_ml, dim3((ncmax + cpb - 1) / cpb, n_steps * (Hq / 64), g.B),
                       dim3(64 * kMlWaves), 0, s, g, mg, (const uint16_t*)q, Hq,
                       (const uint8_t*)pages, page_bytes, page_table, (const uint8_t*)recent, row_bytes,
                       sl2, cpb, ml);
    timing_end("k_chunk_ml", s);
    hipLaunchKernelGGL(k_mass_lse, dim3((Hq + 3) / 4, n_steps, g.B), dim3(256), 0, s, g, mg, Hq, n_steps,
                       (const float2*)ml, lse2);
    hipLaunchKernelGGL(k_mass_sum, dim3((ncmax + 255) / 256, g.B), dim3(256),
                       (size_t)n_steps * Hq * sizeof(float), s, g, mg, Hq, n_steps, (const float2*)ml,
                       (const float*)lse2, mass, recbuf);
    hipLaunchKernelGGL(k_rec_mass, dim3(1), dim3(64), 0, s, g, mg, (const float*)recbuf, rec);
    return hipGetLastError();
}
