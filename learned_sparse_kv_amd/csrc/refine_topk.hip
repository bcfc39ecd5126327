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
// k_topk: one block per request.  Radix select (4 passes of 8 bits, LDS
// histograms with integer atomics) finds the k-th largest order-preserving
// key; an ordered emit pass keeps keys above it plus the lowest-index ties.
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

// Exclusive rank of flag f among the block's threads in thread order, and
// the block total.  1024 threads = 16 waves.
__device__ __forceinline__ int block_rank(bool f, int* wsum, int& total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
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
    __syncthreads();
    total = tot;
    return wpre + pre;
}

__global__ __launch_bounds__(1024) void k_topk(GeomDev g, const int32_t* __restrict__ sel,
                                               const int32_t* __restrict__ cnt,
                                               const float* __restrict__ scores, int k,
                                               int32_t* __restrict__ topk,
                                               int32_t* __restrict__ tcnt) {
    __shared__ uint32_t hist[256];
    __shared__ int wsum[16];
    __shared__ uint32_t s_prefix;
    __shared__ int s_remaining;
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t off = g.chunk_off[r];
    const int n = cnt[r] * 64;
    const float* sc = scores + off * 64;
    const int32_t* sl = sel + off;
    int32_t* out = topk + (int64_t)r * k;

    if (n <= k) {  // every candidate is kept; candidates are already ascending
        for (int p = tid; p < n; p += blockDim.x) out[p] = sl[p >> 6] * 64 + (p & 63);
        if (tid == 0) tcnt[r] = n;
        return;
    }
    uint32_t prefix = 0, mask = 0;
    int remaining = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int p = tid; p < n; p += blockDim.x) {
            const uint32_t key = fkey(sc[p]);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 64) {  // wave 0: find the digit holding the remaining-th largest
            const int lane = tid;
            int c4[4], s = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c4[j] = (int)hist[255 - 4 * lane - j];
                s += c4[j];
            }
            int incl = s;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(incl, o);
                if (lane >= o) incl += t;
            }
            const int excl = incl - s;
            if (excl < remaining && incl >= remaining) {
                int acc = excl, j = 0;
                for (; j < 3; ++j) {
                    if (acc + c4[j] >= remaining) break;
                    acc += c4[j];
                }
                s_prefix = prefix | ((uint32_t)(255 - 4 * lane - j) << shift);
                s_remaining = remaining - acc;
            }
        }
        __syncthreads();
        prefix = s_prefix;
        remaining = s_remaining;
        mask |= 255u << shift;
    }
    // prefix is the k-th largest key; take every key above it and the
    // `remaining` lowest-index keys equal to it, in ascending order.
    int base = 0, eqbase = 0;
    for (int p0 = 0; p0 < n; p0 += blockDim.x) {
        const int p = p0 + tid;
        const uint32_t key = p < n ? fkey(sc[p]) : 0u;
        const bool gt = p < n && key > prefix;
        const bool eq = p < n && key == prefix;
        int eqtot, taketot;
        const int eqrank = eqbase + block_rank(eq, wsum, eqtot);
        const bool take = gt || (eq && eqrank < remaining);
        const int pos = base + block_rank(take, wsum, taketot);
        if (take) out[pos] = sl[p >> 6] * 64 + (p & 63);
        base += taketot;
        eqbase += eqtot;
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
    hipLaunchKernelGGL(k_topk, dim3(g.B), dim3(1024), 0, s, g, sel, cnt, scores, k, topk, tcnt);
    timing_end("k_topk", s);
    return hipGetLastError();
}
