// Lightning refine score and top-k over the candidate tokens (gfx950).
//
// Inside the candidate set fetched by the memory indexer, the model's own
// lightning indexer takes a fine-grained top-k for the final core attention
// (gist.science summary, section 2.1 "Gestufte Selektion"; cjcn.com.cn
// explainer, section 二, whose ReLU the memory indexer replaces by a sigmoid).
// Per step j and candidate token s (chunk c):
//     a_h = q_h . key_s,  I_s = sum_h w_h * ReLU(a_h)  (* chunk scale for fp8)
// then the min(k, |T|) largest I_s, ties to the lower token, ascending.
//
// Arithmetic order (the CPU oracle computes the same values by definition):
// fp32 fma chain over i for each a_h from +0, ReLU giving +0, fma chain over
// h for I from +0, one multiply by the scale.  One lane owns one token, so
// both chains are plain sequential chains; four heads' chains are
// interleaved only for instruction-level parallelism.
//
// k_refine: one wave per selected chunk (64 tokens = 64 lanes), four waves
// per block on chunks of one request, the step's queries converted to fp32
// in LDS and read as wave-uniform broadcasts.  8K fma per token at H=64,
// d=128: VALU-bound.
//
// k_topk: one block per request.  Radix select over the order-preserving
// uint32 keys (digits of 12, 12 and 8 bits, 4096-bin LDS histograms with
// integer atomics) finds the k-th largest key; an ordered emit pass keeps
// keys above it plus the lowest-index ties.
#include "lsa_internal.h"

namespace {

__device__ __forceinline__ float bf16f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

constexpr int kRefineWaves = 4;

// Decode one key row (D elements held in 16-byte pieces) to fp32.
template <int KDT, int D>
__device__ __forceinline__ void load_key(const uint8_t* __restrict__ p, float (&kf)[D]) {
    constexpr int EB = KDT == LSA_F32 ? 4 : (KDT == LSA_BF16 ? 2 : 1);
    constexpr int PIECES = D * EB / 16;
    const uint4* src = (const uint4*)p;
#pragma unroll
    for (int j = 0; j < PIECES; ++j) {
        const uint4 v = src[j];
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (KDT == LSA_F32) {
                kf[4 * j + e] = __uint_as_float(w4[e]);
            } else if constexpr (KDT == LSA_BF16) {
                kf[8 * j + 2 * e] = __uint_as_float(w4[e] << 16);
                kf[8 * j + 2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
            } else {
                const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w4[e], false);
                const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w4[e], true);
                kf[16 * j + 4 * e + 0] = lo[0];
                kf[16 * j + 4 * e + 1] = lo[1];
                kf[16 * j + 4 * e + 2] = hi[0];
                kf[16 * j + 4 * e + 3] = hi[1];
            }
        }
    }
}

__device__ __forceinline__ float relu0(float a) { return a > 0.0f ? a : 0.0f; }

template <int KDT, int D>
__global__ __launch_bounds__(64 * kRefineWaves) void k_refine(
    GeomDev g, const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt,
    const uint8_t* __restrict__ pages, int64_t page_bytes, int64_t ikey_off,
    const int32_t* __restrict__ page_table, const float* __restrict__ ikey_scale,
    const void* __restrict__ q, int q_is_f32, const float* __restrict__ w, int H,
    float* __restrict__ scores) {
    constexpr int EB = KDT == LSA_F32 ? 4 : (KDT == LSA_BF16 ? 2 : 1);
    constexpr int ROWB = D * EB;
    extern __shared__ __attribute__((aligned(16))) float smem[];  // [H*D] q, then [H] w
    __shared__ int goff[LSA_MAX_BATCH + 1];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    float* qf = smem;
    float* wf = smem + H * D;

    if (threadIdx.x == 0) {
        int acc = 0;
        for (int r = 0; r < g.B; ++r) {
            goff[r] = acc;
            acc += (cnt[r] + kRefineWaves - 1) / kRefineWaves;
        }
        goff[g.B] = acc;
    }
    __syncthreads();
    const int total = goff[g.B];
    int cur_r = -1;
    for (int gi = blockIdx.x; gi < total; gi += gridDim.x) {
        int r = 0;
        while (gi >= goff[r + 1]) ++r;
        if (r != cur_r) {  // uniform across the block
            __syncthreads();
            const size_t qb = (size_t)r * H * D;
            for (int e = threadIdx.x; e < H * D; e += blockDim.x)
                qf[e] = q_is_f32 ? ((const float*)q)[qb + e] : bf16f(((const uint16_t*)q)[qb + e]);
            for (int e = threadIdx.x; e < H; e += blockDim.x) wf[e] = w[(size_t)r * H + e];
            __syncthreads();
            cur_r = r;
        }
        const int i = (gi - goff[r]) * kRefineWaves + wv;
        if (i >= cnt[r]) continue;
        const int64_t off = g.chunk_off[r];
        const int c = sel[off + i];
        const int64_t pg = page_table ? (int64_t)page_table[off + c] : off + c;
        float kf[D];
        load_key<KDT, D>(pages + pg * page_bytes + ikey_off + (int64_t)lane * ROWB, kf);

        float I = 0.0f;
        int h = 0;
        for (; h + 4 <= H; h += 4) {
            const float* q0 = qf + h * D;
            float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
            for (int e = 0; e < D; e += 4) {
                const float4 x0 = *(const float4*)(q0 + e);
                const float4 x1 = *(const float4*)(q0 + D + e);
                const float4 x2 = *(const float4*)(q0 + 2 * D + e);
                const float4 x3 = *(const float4*)(q0 + 3 * D + e);
                a0 = __builtin_fmaf(x0.x, kf[e], a0);
                a1 = __builtin_fmaf(x1.x, kf[e], a1);
                a2 = __builtin_fmaf(x2.x, kf[e], a2);
                a3 = __builtin_fmaf(x3.x, kf[e], a3);
                a0 = __builtin_fmaf(x0.y, kf[e + 1], a0);
                a1 = __builtin_fmaf(x1.y, kf[e + 1], a1);
                a2 = __builtin_fmaf(x2.y, kf[e + 1], a2);
                a3 = __builtin_fmaf(x3.y, kf[e + 1], a3);
                a0 = __builtin_fmaf(x0.z, kf[e + 2], a0);
                a1 = __builtin_fmaf(x1.z, kf[e + 2], a1);
                a2 = __builtin_fmaf(x2.z, kf[e + 2], a2);
                a3 = __builtin_fmaf(x3.z, kf[e + 2], a3);
                a0 = __builtin_fmaf(x0.w, kf[e + 3], a0);
                a1 = __builtin_fmaf(x1.w, kf[e + 3], a1);
                a2 = __builtin_fmaf(x2.w, kf[e + 3], a2);
                a3 = __builtin_fmaf(x3.w, kf[e + 3], a3);
            }
            I = __builtin_fmaf(wf[h], relu0(a0), I);
            I = __builtin_fmaf(wf[h + 1], relu0(a1), I);
            I = __builtin_fmaf(wf[h + 2], relu0(a2), I);
            I = __builtin_fmaf(wf[h + 3], relu0(a3), I);
        }
        for (; h < H; ++h) {
            const float* q0 = qf + h * D;
            float a0 = 0.0f;
#pragma unroll
            for (int e = 0; e < D; ++e) a0 = __builtin_fmaf(q0[e], kf[e], a0);
            I = __builtin_fmaf(wf[h], relu0(a0), I);
        }
        if constexpr (KDT == LSA_FP8_E4M3FN) I = I * ikey_scale[off + c];
        scores[off * 64 + (int64_t)i * 64 + lane] = I;
    }
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key);
// -0 is first made +0 so the two compare equal.
__device__ __forceinline__ uint32_t fkey(float f) {
    const uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide exclusive prefix of a per-thread count over NW waves, and the
// block total.
template <int NW = 16>
__device__ __forceinline__ int block_scan(int v, int* wsum, int& total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int wpre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int x = wsum[i];
        wpre += (i < wv) ? x : 0;
        tot += x;
    }
    __syncthreads();
    total = tot;
    return wpre + incl - v;
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBatch = 8;  // independent loads in flight per thread

// Radix select over the order-preserving uint32 keys with digits of 12, 12
// and 8 bits (4096-bin LDS histograms, integer atomics).  Each pass streams
// the request's scores (L2-resident) with kBatch loads in flight per thread;
// only keys matching the digits chosen so far are counted.
__device__ __forceinline__ void topk_select(const float* __restrict__ sc, int n, int k,
                                            uint32_t* hist, int* wsum, uint32_t* s_prefix,
                                            int* s_remaining, int* s_eq, uint32_t& K, int& need,
                                            int& eq_total) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, mask = 0;
    int remaining = k;
    const int shifts[3] = {20, 8, 0};
    const int widths[3] = {12, 12, 8};
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = shifts[pass];
        const int nb = 1 << widths[pass];
        for (int i = tid; i < nb; i += kTopkThreads) hist[i] = 0;
        __syncthreads();
        for (int p0 = 0; p0 < n; p0 += kBatch * kTopkThreads) {
            float v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int p = p0 + j * kTopkThreads + tid;
                v[j] = p < n ? sc[p] : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int p = p0 + j * kTopkThreads + tid;
                const uint32_t key = fkey(v[j]);
                if (p < n && (key & mask) == prefix)
                    atomicAdd(&hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
            }
        }
        __syncthreads();
        // suffix scan from the top digit: thread t owns 4 digits
        int c4[4], s4 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = nb - 1 - (4 * tid + j);
            c4[j] = b >= 0 ? (int)hist[b] : 0;
            s4 += c4[j];
        }
        int tot;
        const int excl = block_scan<kTopkWaves>(s4, wsum, tot);
        if (excl < remaining && excl + s4 >= remaining) {
            int acc = excl, j = 0;
            for (; j < 3; ++j) {
                if (acc + c4[j] >= remaining) break;
                acc += c4[j];
            }
            *s_prefix = prefix | ((uint32_t)(nb - 1 - (4 * tid + j)) << shift);
            *s_remaining = remaining - acc;
            *s_eq = c4[j];
        }
        __syncthreads();
        prefix = *s_prefix;
        remaining = *s_remaining;
        mask |= (uint32_t)(nb - 1) << shift;
    }
    K = prefix;
    need = remaining;
    eq_total = *s_eq;  // keys equal to K (the final digit's count)
}

// One block per request: select the k-th largest key K, then emit in
// ascending candidate order every key above K and the `need` lowest-index
// keys equal to K.  When every key equal to K is taken (the usual case)
// the emit needs one block scan per batch; otherwise a second scan ranks
// the ties.
__global__ __launch_bounds__(kTopkThreads) void k_topk(GeomDev g, const int32_t* __restrict__ sel,
                                                      const int32_t* __restrict__ cnt,
                                                      const float* __restrict__ scores, int k,
                                                      int32_t* __restrict__ topk,
                                                      int32_t* __restrict__ tcnt) {
    __shared__ uint32_t hist[4096];
    __shared__ int wsum[kTopkWaves];
    __shared__ uint32_t s_prefix;
    __shared__ int s_remaining, s_eq;
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t off = g.chunk_off[r];
    const int n = cnt[r] * 64;
    const float* sc = scores + off * 64;
    const int32_t* sl = sel + off;
    int32_t* out = topk + (int64_t)r * k;

    if (n <= k) {  // every candidate is kept; candidates are already ascending
        for (int p = tid; p < n; p += kTopkThreads) out[p] = sl[p >> 6] * 64 + (p & 63);
        if (tid == 0) tcnt[r] = n;
        return;
    }
    uint32_t K;
    int need, eq_total;
    topk_select(sc, n, k, hist, wsum, &s_prefix, &s_remaining, &s_eq, K, need, eq_total);
    const bool all_ties = (eq_total == need);
    // ordered emit: thread t owns 4 consecutive candidates of each 4096-block
    int base = 0, eqbase = 0;
    float4 nxt = make_float4(0.f, 0.f, 0.f, 0.f);
    if (4 * tid < n) nxt = *(const float4*)(sc + 4 * tid);
    for (int p0 = 0; p0 < n; p0 += 4 * kTopkThreads) {
        const int pb = p0 + 4 * tid;
        const float4 cur = nxt;
        if (pb + 4 * kTopkThreads < n) nxt = *(const float4*)(sc + pb + 4 * kTopkThreads);
        const uint32_t key[4] = {fkey(cur.x), fkey(cur.y), fkey(cur.z), fkey(cur.w)};
        bool take[4];
        int tc = 0, tot;
        if (all_ties) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                take[j] = pb + j < n && key[j] >= K;
                tc += take[j];
            }
        } else {
            int eqc = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) eqc += (pb + j < n && key[j] == K);
            int eqr = eqbase + block_scan<kTopkWaves>(eqc, wsum, tot);
            eqbase += tot;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool valid = pb + j < n;
                const bool eq = valid && key[j] == K;
                take[j] = valid && (key[j] > K || (eq && eqr < need));
                eqr += eq;
                tc += take[j];
            }
        }
        int pos = base + block_scan<kTopkWaves>(tc, wsum, tot);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (take[j]) {
                const int p = pb + j;
                out[pos++] = sl[p >> 6] * 64 + (p & 63);
            }
        base += tot;
    }
    if (tid == 0) tcnt[r] = base;
}

}  // namespace

hipError_t launch_refine(const GeomDev& g, const int32_t* sel, const int32_t* cnt,
                         const void* pages, int64_t page_bytes, int64_t ikey_off,
                         const int32_t* page_table, lsa_dtype idx_dt, const float* ikey_scale,
                         const void* q, lsa_dtype q_dt, const float* w, int H, int d,
                         float* scores, int grid_hint, hipStream_t s) {
    int grid = grid_hint;
    if (grid <= 0) {  // upper bound: every history chunk selected
        const int64_t nmax = g.chunk_off[g.B] / kRefineWaves + g.B;
        grid = (int)(nmax < 2048 ? nmax : 2048);
    }
    if (grid <= 0) return hipSuccess;
    const size_t shm = ((size_t)H * d + H) * sizeof(float);
    const uint8_t* pg = (const uint8_t*)pages;
    const int qf32 = q_dt == LSA_F32;
#define LSA_REFINE_CASE(KDT, D)                                                                 \
    if (idx_dt == KDT && d == D) {                                                              \
        timing_begin("k_refine", s);                                                            \
        hipLaunchKernelGGL((k_refine<KDT, D>), dim3(grid), dim3(64 * kRefineWaves), shm, s, g,   \
                           sel, cnt, pg, page_bytes, ikey_off, page_table, ikey_scale, q, qf32, \
                           w, H, scores);                                                       \
        timing_end("k_refine", s);                                                              \
        return hipGetLastError();                                                               \
    }
    LSA_REFINE_CASE(LSA_F32, 64)
    LSA_REFINE_CASE(LSA_F32, 128)
    LSA_REFINE_CASE(LSA_BF16, 64)
    LSA_REFINE_CASE(LSA_BF16, 128)
    LSA_REFINE_CASE(LSA_FP8_E4M3FN, 64)
    LSA_REFINE_CASE(LSA_FP8_E4M3FN, 128)
#undef LSA_REFINE_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_topk(const GeomDev& g, const int32_t* sel, const int32_t* cnt,
                       const float* scores, int k, int32_t* topk, int32_t* tcnt, hipStream_t s) {
    timing_begin("k_topk", s);
    hipLaunchKernelGGL(k_topk, dim3(g.B), dim3(kTopkThreads), 0, s, g, sel, cnt, scores, k, topk,
                       tcnt);
    timing_end("k_topk", s);
    return hipGetLastError();
}
