// Lightning refine + top-k on matrix cores, with an exact re-score band (gfx950).
//
// The selection must equal the one made on the canonical fp32 scores
//     a_h = fma chain over i of q_h[i] * key[i],  I = fma chain over h of
//     w_h * ReLU(a_h),  times the chunk scale (fp8 keys)
// bit for bit, but those chains cost 8K dependent-order fma per token.  So:
//
//  K1 k_refine_mfma  every candidate token: a'_h = q_h . key on MFMA (bf16
//     inputs, exact products, fp32 accumulation), I' = sum_h w_h ReLU(a'_h),
//     and a rigorous bound E with |I' - I| <= E.  Writes L = I' - E and
//     U = I' + E, and each block's range of L.
//  K2 k_band         per request: a histogram of L over its range finds a
//     key tau no larger than the k-th largest L; every candidate with
//     U >= tau (the band: never fewer than k) is listed, ascending.
//  K3 k_rescore      the listed candidates get the canonical score.
//  K4 k_topk_list    exact top-k among them, ties to the lower token.
// A candidate left out has I <= U < tau <= the k-th largest L <= the k-th
// largest I among the listed ones, so it is strictly below k others and
// cannot be in the top-k: the result is the canonical one.
//
// The bound.  Both the canonical chain and the MFMA sum differ from the exact
// dot product by at most gamma(n) * sum_i |q_i k_i| (any summation order,
// one rounding per operation, Higham's bound), taken here with two ulps per
// operation (u = 2^-22) to cover truncating accumulation;
// sum_i |q_i k_i| <= |q_h| |key| (Cauchy-Schwarz).  ReLU is 1-Lipschitz and
// the head sums add gamma(H) * sum_h |w_h| (ReLU(a'_h) + eps_h).
#include "lsa_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ uint32_t fkey(float f) {
    const uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr float kU2 = 2.384185791015625e-07f;  // 2^-22: two ulps of fp32 per operation
__host__ __device__ constexpr float gam(int n) { return n * kU2 / (1.0f - n * kU2); }

constexpr int kBandWaves = 4;
constexpr int kBandBins = 4096;   // histogram bins over a request's range of L
constexpr int kSlice = 4096;      // candidates per slice in the band kernels
constexpr int kRedStride = 33;    // per-token row of 16 + 16 partial sums (+1 pad)

// 8 fp8 e4m3fn bytes -> 8 bf16 (exact: every e4m3 value is a bf16 value)
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint2 v) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, true);
    uint4 r;
    r.x = (__float_as_uint(a[0]) >> 16) | (__float_as_uint(a[1]) & 0xffff0000u);
    r.y = (__float_as_uint(b[0]) >> 16) | (__float_as_uint(b[1]) & 0xffff0000u);
    r.z = (__float_as_uint(c[0]) >> 16) | (__float_as_uint(c[1]) & 0xffff0000u);
    r.w = (__float_as_uint(d[0]) >> 16) | (__float_as_uint(d[1]) & 0xffff0000u);
    return r;
}

__device__ __forceinline__ float sumsq_bf16x8(uint4 v) {
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(w4[e] << 16), hi = __uint_as_float(w4[e] & 0xffff0000u);
        s = __builtin_fmaf(lo, lo, s);
        s = __builtin_fmaf(hi, hi, s);
    }
    return s;
}

// Work items: groups of kBandWaves selected chunks of one request.  The
// counts are loaded by B threads at once, then prefix-summed by thread 0.
// Must be called by every thread of the block.
__device__ __forceinline__ void group_offsets(const GeomDev& g, const int32_t* cnt, int* goff) {
    if ((int)threadIdx.x < g.B) goff[threadIdx.x + 1] = (cnt[threadIdx.x] + kBandWaves - 1) / kBandWaves;
    __syncthreads();
    if (threadIdx.x == 0) {
        goff[0] = 0;
        for (int r = 0; r < g.B; ++r) goff[r + 1] += goff[r];
    }
    __syncthreads();
}

template <int KDT, int D, int H>
__global__ __launch_bounds__(64 * kBandWaves) void k_refine_mfma(
    GeomDev g, const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt,
    const uint8_t* __restrict__ pages, int64_t page_bytes, int64_t ikey_off,
    const int32_t* __restrict__ page_table, const float* __restrict__ ikey_scale,
    const uint16_t* __restrict__ q, const float* __restrict__ w, float2* __restrict__ lu,
    uint2* __restrict__ stats, uint32_t* __restrict__ band_hist) {
    constexpr int EB = KDT == LSA_BF16 ? 2 : 1;
    constexpr int ROWB = D * EB;
    constexpr int KS = D / 32;   // MFMA k-steps
    constexpr int HB = H / 16;   // head blocks
    __shared__ int goff[LSA_MAX_BATCH + 1];
    __shared__ uint32_t s_mn[kBandWaves], s_mx[kBandWaves];
    __shared__ float red[kBandWaves][64 * kRedStride];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, lq = lane >> 4;
    for (int e = blockIdx.x * blockDim.x + tid; e < g.B * kBandBins; e += gridDim.x * blockDim.x)
        band_hist[e] = 0;  // histogram of the next kernel
    group_offsets(g, cnt, goff);
    const int total = goff[g.B];
    int cur_r = -1;
    uint4 qb[HB][KS];
    float wl[HB], wa[HB];
    float wq = 0.0f;
    for (int gi = blockIdx.x; gi < total; gi += gridDim.x) {
        int r = 0;
        while (gi >= goff[r + 1]) ++r;
        if (r != cur_r) {  // uniform across the block
            const uint16_t* qr = q + (int64_t)r * H * D;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    qb[hb][ks] = *(const uint4*)(qr + (hb * 16 + l16) * D + ks * 32 + lq * 8);
                wl[hb] = w[(int64_t)r * H + hb * 16 + l16];
                wa[hb] = fabsf(wl[hb]);
            }
            // Wq = sum_h |w_h| * |q_h|_2 (rounded up), from the operands held:
            // lane (l16, lq) has dims lq*8.. of every k-step of head hb*16 + l16
            float part = 0.0f;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                float ss = 0.0f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) ss += sumsq_bf16x8(qb[hb][ks]);
                ss += __shfl_xor(ss, 16);
                ss += __shfl_xor(ss, 32);
                part += wa[hb] * sqrtf(ss * (1.0f + gam(D + 8))) * (1.0f + 4 * kU2);
            }
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) part += __shfl_xor(part, o);
            wq = part * (1.0f + gam(H + 8));
            cur_r = r;
        }
        const int i = (gi - goff[r]) * kBandWaves + wv;
        uint32_t kmin = 0xffffffffu, kmax = 0u;
        if (i < cnt[r]) {
            const int64_t off = g.chunk_off[r];
            const int c = sel[off + i];
            const int64_t pg = page_table ? (int64_t)page_table[off + c] : off + c;
            const uint8_t* base = pages + pg * page_bytes + ikey_off;
            const float scale = (KDT == LSA_FP8_E4M3FN) ? ikey_scale[off + c] : 1.0f;
            // A operands: key rows of tokens tb*16 + l16, dims ks*32 + lq*8 .. +8
            uint4 ka[4][KS];
            float kss[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const uint8_t* row = base + (int64_t)(tb * 16 + l16) * ROWB;
                float ss = 0.0f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if constexpr (KDT == LSA_BF16)
                        ka[tb][ks] = *(const uint4*)(row + (ks * 32 + lq * 8) * 2);
                    else
                        ka[tb][ks] = fp8x8_to_bf16x8(*(const uint2*)(row + ks * 32 + lq * 8));
                    ss += sumsq_bf16x8(ka[tb][ks]);
                }
                ss += __shfl_xor(ss, 16);
                ss += __shfl_xor(ss, 32);
                kss[tb] = ss;  // |key|^2 of token tb*16 + l16 (every lq)
            }
            // partial head sums per lane (heads hb*16 + l16), then through LDS
            // to one lane per token: red[token][l16], fixed summation order
            float* pr = red[wv];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                f32x4_t acc[HB];
#pragma unroll
                for (int hb = 0; hb < HB; ++hb) {
                    f32x4_t c4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, ka[tb][ks]),
                            __builtin_bit_cast(bf16x8_t, qb[hb][ks]), c4, 0, 0, 0);
                    acc[hb] = c4;  // a'[token tb*16 + 4*lq + e][head hb*16 + l16]
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float sI = 0.0f, sW = 0.0f;
#pragma unroll
                    for (int hb = 0; hb < HB; ++hb) {
                        const float rr = fmaxf(acc[hb][e], 0.0f);
                        sI = __builtin_fmaf(wl[hb], rr, sI);
                        sW = __builtin_fmaf(wa[hb], rr, sW);
                    }
                    const int t = tb * 16 + 4 * lq + e;
                    pr[t * kRedStride + l16] = sI;
                    pr[t * kRedStride + 16 + l16] = sW;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // lane = token of the chunk
            float sI = 0.0f, sW = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                sI += pr[lane * kRedStride + j];
                sW += pr[lane * kRedStride + 16 + j];
            }
            const float kn2 = lq == 0 ? kss[0] : (lq == 1 ? kss[1] : (lq == 2 ? kss[2] : kss[3]));
            const float kn = sqrtf(kn2 * (1.0f + gam(D + 8))) * (1.0f + 4 * kU2);
            const float ek = gam(D) * 2.0f * kn * wq;  // sum_h |w_h| eps_h
            float E = ek + 2.0f * gam(H + 24) * (sW + ek);
            const float Is = sI * scale;
            E = (E * scale + 4 * kU2 * (fabsf(Is) + E * scale)) * (1.0f + 16 * kU2) + 1e-30f;
            const float L = Is - E, U = Is + E;
            lu[(off * 64) + (int64_t)i * 64 + lane] = make_float2(L, U);
            kmin = fkey(L);
            kmax = kmin;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
            kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
        }
        if (lane == 0) {
            s_mn[wv] = kmin;
            s_mx[wv] = kmax;
        }
        __syncthreads();
        if (tid == 0) {
            uint32_t a = s_mn[0], b = s_mx[0];
            for (int j = 1; j < kBandWaves; ++j) {
                a = min(a, s_mn[j]);
                b = max(b, s_mx[j]);
            }
            stats[gi] = make_uint2(a, b);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
constexpr int kT = 1024, kTW = kT / 64;

template <int NW>
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

// Range [lo, hi] of the L keys of request r, from K1's per-block ranges.
__device__ __forceinline__ void band_range(const GeomDev& g, const int32_t* cnt,
                                           const uint2* stats, int r, int* goff, uint32_t* red,
                                           uint32_t& lo, uint32_t& hi) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;
    group_offsets(g, cnt, goff);
    uint32_t mn = 0xffffffffu, mx = 0u;
    for (int j = goff[r] + tid; j < goff[r + 1]; j += blockDim.x) {
        const uint2 st = stats[j];
        mn = min(mn, st.x);
        mx = max(mx, st.y);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    }
    if (lane == 0) {
        red[wv] = mn;
        red[16 + wv] = mx;
    }
    __syncthreads();
    lo = red[0];
    hi = red[16];
    for (int i = 1; i < nw; ++i) {
        lo = min(lo, red[i]);
        hi = max(hi, red[16 + i]);
    }
    __syncthreads();
}

__device__ __forceinline__ int band_shift(uint32_t lo, uint32_t hi) {
    const uint64_t width = (uint64_t)hi - lo + 1;
    int shift = 0;
    while ((width + (1ull << shift) - 1) >> shift > (uint64_t)kBandBins) ++shift;
    return shift;
}

// K2a: histogram of L over [lo, hi] (kBandBins bins), one block per slice of
// kSlice candidates; block counts are added to the request's histogram.
__global__ __launch_bounds__(256) void k_band_hist(GeomDev g, const int32_t* __restrict__ cnt,
                                                   const float2* __restrict__ lu,
                                                   const uint2* __restrict__ stats, int k,
                                                   uint32_t* __restrict__ band_hist) {
    __shared__ uint32_t hist[kBandBins];
    __shared__ int goff[LSA_MAX_BATCH + 1];
    __shared__ uint32_t red[32];
    const int r = blockIdx.y, tid = threadIdx.x;
    const int n = cnt[r] * 64;
    const int p0 = blockIdx.x * kSlice;
    if (n <= k || p0 >= n) return;
    uint32_t lo, hi;
    band_range(g, cnt, stats, r, goff, red, lo, hi);
    const int shift = band_shift(lo, hi);
    for (int i = tid; i < kBandBins; i += 256) hist[i] = 0;
    __syncthreads();
    const float2* v = lu + g.chunk_off[r] * 64;
    const int p1 = min(n, p0 + kSlice);
#pragma unroll 4
    for (int p = p0 + tid; p < p1; p += 256) atomicAdd(&hist[(fkey(v[p].x) - lo) >> shift], 1u);
    __syncthreads();
    uint32_t* gh = band_hist + (int64_t)r * kBandBins;
    for (int i = tid; i < kBandBins; i += 256)
        if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

// K2b: the request's threshold tau (lowest key of the histogram bin holding
// the k-th largest L), then each block lists, in order, the candidates of its
// slice with U >= tau.  Requests with no more than k candidates keep them all.
__global__ __launch_bounds__(256) void k_band_list(GeomDev g, const int32_t* __restrict__ sel,
                                                   const int32_t* __restrict__ cnt,
                                                   const float2* __restrict__ lu,
                                                   const uint2* __restrict__ stats, int k,
                                                   const uint32_t* __restrict__ band_hist,
                                                   int32_t* __restrict__ ulist,
                                                   int32_t* __restrict__ scnt,
                                                   int32_t* __restrict__ topk,
                                                   int32_t* __restrict__ tcnt, int nslices) {
    __shared__ int wsum[4];
    __shared__ int goff[LSA_MAX_BATCH + 1];
    __shared__ uint32_t red[32];
    __shared__ uint32_t s_tau;
    const int r = blockIdx.y, tid = threadIdx.x;
    const int n = cnt[r] * 64;
    const int p0 = blockIdx.x * kSlice;
    const int64_t off = g.chunk_off[r];
    int32_t* sc_out = scnt + (int64_t)r * nslices;
    if (p0 >= n) {
        if (blockIdx.x < nslices) sc_out[blockIdx.x] = 0;
        return;
    }
    const int p1 = min(n, p0 + kSlice);
    if (n <= k) {  // every candidate is kept, already ascending
        for (int p = p0 + tid; p < p1; p += 256)
            topk[(int64_t)r * k + p] = sel[off + (p >> 6)] * 64 + (p & 63);
        if (blockIdx.x == 0 && tid == 0) tcnt[r] = n;
        if (tid == 0) sc_out[blockIdx.x] = 0;
        return;
    }
    uint32_t lo, hi;
    band_range(g, cnt, stats, r, goff, red, lo, hi);
    const int shift = band_shift(lo, hi);
    const int nb = (int)((((uint64_t)hi - lo + 1) + (1ull << shift) - 1) >> shift);
    const uint32_t* gh = band_hist + (int64_t)r * kBandBins;
    // suffix scan from the top bin: thread t owns 16 bins
    int c16[16], s16 = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int bn = nb - 1 - (16 * tid + j);
        c16[j] = bn >= 0 ? (int)gh[bn] : 0;
        s16 += c16[j];
    }
    int tot;
    const int excl = block_scan<4>(s16, wsum, tot);
    if (excl < k && excl + s16 >= k) {
        int acc = excl, j = 0;
        for (; j < 15; ++j) {
            if (acc + c16[j] >= k) break;
            acc += c16[j];
        }
        s_tau = lo + ((uint32_t)(nb - 1 - (16 * tid + j)) << shift);
    }
    __syncthreads();
    const uint32_t tau = s_tau;
    const float2* v = lu + off * 64;
    int32_t* ul = ulist + off * 64 + p0;  // this slice's list
    int base = 0;
    for (int q0 = p0; q0 < p1; q0 += 4 * 256) {
        const int pb = q0 + 4 * tid;
        bool take[4];
        int tc = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            take[j] = pb + j < p1 && fkey(v[pb + j].y) >= tau;
            tc += take[j];
        }
        int pos = base + block_scan<4>(tc, wsum, tot);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (take[j]) ul[pos++] = pb + j;
        base += tot;
    }
    if (tid == 0) sc_out[blockIdx.x] = base;
}

// K3: canonical scores of the listed candidates of one slice.  Block = 32
// candidates x 8 head groups; each thread runs its heads' fma chains in
// element order, the head sum then runs in head order on one thread per
// candidate.
template <int KDT, int D, int H>
__global__ __launch_bounds__(256) void k_rescore(
    GeomDev g, const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt,
    const int32_t* __restrict__ ulist, const int32_t* __restrict__ scnt, int nslices, int k,
    const uint8_t* __restrict__ pages, int64_t page_bytes, int64_t ikey_off,
    const int32_t* __restrict__ page_table, const float* __restrict__ ikey_scale,
    const uint16_t* __restrict__ q, const float* __restrict__ w, float* __restrict__ exact) {
    constexpr int EB = KDT == LSA_BF16 ? 2 : 1;
    constexpr int ROWB = D * EB;
    constexpr int HPG = H / 8;  // heads per thread
    constexpr int GS = HPG * D + 4;  // head-group stride: the 8 groups hit distinct banks
    __shared__ __attribute__((aligned(16))) float qf[8 * GS];
    __shared__ float wf[H];
    __shared__ float rel[32][H + 1];
    const int r = blockIdx.y, tid = threadIdx.x;
    const int n = cnt[r] * 64;
    if (n <= k || blockIdx.x * kSlice >= n) return;
    const int m = scnt[(int64_t)r * nslices + blockIdx.x];
    if (m == 0) return;
    const uint32_t* qs = (const uint32_t*)(q + (int64_t)r * H * D);
#pragma unroll 4
    for (int e = tid; e < H * D / 8; e += 256) {
        const uint4 x = ((const uint4*)qs)[e];
        const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
        const int f0 = 8 * e;  // element index h*D + i; group h / HPG
        const int dst = (f0 / (HPG * D)) * GS + f0 % (HPG * D);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            qf[dst + 2 * j] = __uint_as_float(w4[j] << 16);
            qf[dst + 2 * j + 1] = __uint_as_float(w4[j] & 0xffff0000u);
        }
    }
    for (int e = tid; e < H; e += 256) wf[e] = w[(int64_t)r * H + e];
    __syncthreads();
    const int64_t off = g.chunk_off[r];
    const int32_t* ul = ulist + off * 64 + blockIdx.x * kSlice;
    float* ex = exact + off * 64 + blockIdx.x * kSlice;
    const int tok = tid >> 3, hg = tid & 7;
    for (int j0 = 0; j0 < m; j0 += 32) {
        const int j = j0 + tok;
        const bool valid = j < m;
        int p = 0;
        if (valid) {
            p = ul[j];
            const int c = sel[off + (p >> 6)];
            const int64_t pg = page_table ? (int64_t)page_table[off + c] : off + c;
            const uint8_t* row = pages + pg * page_bytes + ikey_off + (int64_t)(p & 63) * ROWB;
            float kf[D];
#pragma unroll
            for (int x = 0; x < ROWB / 16; ++x) {
                const uint4 v = *(const uint4*)(row + 16 * x);
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (KDT == LSA_BF16) {
                        kf[8 * x + 2 * e] = __uint_as_float(w4[e] << 16);
                        kf[8 * x + 2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
                    } else {
                        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w4[e], false);
                        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w4[e], true);
                        kf[16 * x + 4 * e + 0] = lo[0];
                        kf[16 * x + 4 * e + 1] = lo[1];
                        kf[16 * x + 4 * e + 2] = hi[0];
                        kf[16 * x + 4 * e + 3] = hi[1];
                    }
                }
            }
            float a[HPG];
#pragma unroll
            for (int u = 0; u < HPG; ++u) a[u] = 0.0f;
#pragma unroll
            for (int e = 0; e < D; e += 4) {
#pragma unroll
                for (int u = 0; u < HPG; ++u) {
                    const float4 x = *(const float4*)&qf[hg * GS + u * D + e];
                    a[u] = __builtin_fmaf(x.x, kf[e], a[u]);
                    a[u] = __builtin_fmaf(x.y, kf[e + 1], a[u]);
                    a[u] = __builtin_fmaf(x.z, kf[e + 2], a[u]);
                    a[u] = __builtin_fmaf(x.w, kf[e + 3], a[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < HPG; ++u) rel[tok][hg * HPG + u] = a[u] > 0.0f ? a[u] : 0.0f;
        }
        __syncthreads();
        if (valid && hg == 0) {
            float I = 0.0f;
            for (int h = 0; h < H; ++h) I = __builtin_fmaf(wf[h], rel[tok][h], I);
            if constexpr (KDT == LSA_FP8_E4M3FN) I = I * ikey_scale[off + sel[off + (p >> 6)]];
            ex[j] = I;
        }
        __syncthreads();
    }
}

// K4: exact top-k among the listed candidates of one request (one block).
// The slice lists are gathered in order into LDS (up to kListCap entries),
// the k-th largest key is found by 12/12/8-bit radix select on LDS, then the
// emit keeps keys above it and the lowest-index ties.  Larger lists (only
// with massive ties) take the same steps reading global memory.
constexpr int kListCap = 8192;

__global__ __launch_bounds__(kT) void k_topk_list(GeomDev g, const int32_t* __restrict__ sel,
                                                  const int32_t* __restrict__ cnt,
                                                  const int32_t* __restrict__ ulist,
                                                  const int32_t* __restrict__ scnt, int nslices,
                                                  const float* __restrict__ exact, int k,
                                                  int32_t* __restrict__ topk,
                                                  int32_t* __restrict__ tcnt) {
    __shared__ uint32_t hist[4096];
    __shared__ uint32_t lkey[kListCap];
    __shared__ int32_t lpos[kListCap];
    __shared__ int soff[1024 + 1];
    __shared__ int wsum[kTW];
    __shared__ uint32_t s_prefix;
    __shared__ int s_remaining, s_eq;
    const int r = blockIdx.x, tid = threadIdx.x;
    const int n = cnt[r] * 64;
    if (n <= k) return;  // k_band_list already wrote the result
    const int64_t off = g.chunk_off[r];
    const int ns = (n + kSlice - 1) / kSlice;
    // slice offsets (ns <= nslices <= 1024)
    int cnt_t = tid < ns ? scnt[(int64_t)r * nslices + tid] : 0;
    int tot;
    const int ex0 = block_scan<kTW>(cnt_t, wsum, tot);
    if (tid < ns) soff[tid] = ex0;
    if (tid == 0) soff[ns] = tot;
    __syncthreads();
    const int m = soff[ns];
    const bool in_lds = m <= kListCap;
    // position j of the ordered list -> (slice, index)
    auto at = [&](int j, uint32_t& key, int32_t& pos) {
        if (in_lds) {
            key = lkey[j];
            pos = lpos[j];
            return;
        }
        int lo = 0, hi = ns - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (soff[mid] <= j) lo = mid;
            else hi = mid - 1;
        }
        const int64_t e = off * 64 + (int64_t)lo * kSlice + (j - soff[lo]);
        key = fkey(exact[e]);
        pos = ulist[e];
    };
    if (in_lds) {
        for (int sidx = 0; sidx < ns; ++sidx) {
            const int c = soff[sidx + 1] - soff[sidx];
            const int64_t e0 = off * 64 + (int64_t)sidx * kSlice;
            for (int j = tid; j < c; j += kT) {
                lkey[soff[sidx] + j] = fkey(exact[e0 + j]);
                lpos[soff[sidx] + j] = ulist[e0 + j];
            }
        }
        __syncthreads();
    }
    uint32_t prefix = 0, mask = 0;
    int remaining = k;
    const int shifts[3] = {20, 8, 0}, widths[3] = {12, 12, 8};
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = shifts[pass], nb = 1 << widths[pass];
        for (int i = tid; i < nb; i += kT) hist[i] = 0;
        __syncthreads();
        for (int j = tid; j < m; j += kT) {
            uint32_t key;
            int32_t pos;
            at(j, key, pos);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
        }
        __syncthreads();
        int c4[4], s4 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = nb - 1 - (4 * tid + j);
            c4[j] = b >= 0 ? (int)hist[b] : 0;
            s4 += c4[j];
        }
        const int excl = block_scan<kTW>(s4, wsum, tot);
        if (excl < remaining && excl + s4 >= remaining) {
            int acc = excl, j = 0;
            for (; j < 3; ++j) {
                if (acc + c4[j] >= remaining) break;
                acc += c4[j];
            }
            s_prefix = prefix | ((uint32_t)(nb - 1 - (4 * tid + j)) << shift);
            s_remaining = remaining - acc;
            s_eq = c4[j];
        }
        __syncthreads();
        prefix = s_prefix;
        remaining = s_remaining;
        mask |= (uint32_t)(nb - 1) << shift;
    }
    const uint32_t K = prefix;
    const int need = remaining;
    const bool all_ties = (s_eq == need);
    const int32_t* sl = sel + off;
    int32_t* out = topk + (int64_t)r * k;
    int base = 0, eqbase = 0;
    for (int p0 = 0; p0 < m; p0 += 4 * kT) {
        const int pb = p0 + 4 * tid;
        uint32_t key[4];
        int32_t pos[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            key[j] = 0u;
            pos[j] = 0;
            if (pb + j < m) at(pb + j, key[j], pos[j]);
        }
        bool take[4];
        int tc = 0;
        if (all_ties) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                take[j] = pb + j < m && key[j] >= K;
                tc += take[j];
            }
        } else {
            int eqc = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) eqc += (pb + j < m && key[j] == K);
            int eqr = eqbase + block_scan<kTW>(eqc, wsum, tot);
            eqbase += tot;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool valid = pb + j < m;
                const bool eq = valid && key[j] == K;
                take[j] = valid && (key[j] > K || (eq && eqr < need));
                eqr += eq;
                tc += take[j];
            }
        }
        int o = base + block_scan<kTW>(tc, wsum, tot);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (take[j]) out[o++] = sl[pos[j] >> 6] * 64 + (pos[j] & 63);
        base += tot;
    }
    if (tid == 0) tcnt[r] = base;
}

}  // namespace

static int max_slices(const GeomDev& g);

bool band_fits(const GeomDev& g) { return max_slices(g) <= 1024; }

bool band_supported(lsa_dtype idx_dt, lsa_dtype q_dt, int H, int d) {
    // k_rescore keeps the queries (fp32) and the ReLU outputs in LDS
    const size_t lds = (size_t)H * d * 4 + 32 * (H + 1) * 4 + 1024;
    return (idx_dt == LSA_BF16 || idx_dt == LSA_FP8_E4M3FN) && q_dt == LSA_BF16 &&
           (d == 64 || d == 128) && (H == 16 || H == 32 || H == 64 || H == 128) &&
           lds <= 64 * 1024;
}

static int max_slices(const GeomDev& g) {
    int mx = 0;
    for (int r = 0; r < g.B; ++r) mx = g.nhist[r] > mx ? g.nhist[r] : mx;
    return (mx * 64 + kSlice - 1) / kSlice;
}

size_t band_ws_bytes(const GeomDev& g) {
    const size_t nc = (size_t)g.chunk_off[g.B] * 64 + 64;
    const size_t items = (size_t)g.chunk_off[g.B] / kBandWaves + g.B + 1;
    const size_t ns = (size_t)g.B * (max_slices(g) + 1);
    return align_up(nc * sizeof(float2), 256) + align_up(items * sizeof(uint2), 256) +
           2 * align_up(nc * 4, 256) + align_up(ns * 4, 256) +
           align_up((size_t)g.B * kBandBins * 4, 256);
}

hipError_t launch_refine_band(const GeomDev& g, const int32_t* sel, const int32_t* cnt,
                              const void* pages, int64_t page_bytes, int64_t ikey_off,
                              const int32_t* page_table, lsa_dtype idx_dt,
                              const float* ikey_scale, const void* q, const float* w, int H,
                              int d, int k, int32_t* topk, int32_t* tcnt, void* ws, int grid_hint,
                              hipStream_t s) {
    const size_t nc = (size_t)g.chunk_off[g.B] * 64 + 64;
    const size_t items = (size_t)g.chunk_off[g.B] / kBandWaves + g.B + 1;
    const int nslices = max_slices(g) > 0 ? max_slices(g) : 1;
    uint8_t* b = (uint8_t*)ws;
    float2* lu = (float2*)b;
    b += align_up(nc * sizeof(float2), 256);
    uint2* stats = (uint2*)b;
    b += align_up(items * sizeof(uint2), 256);
    int32_t* ulist = (int32_t*)b;
    b += align_up(nc * 4, 256);
    float* exact = (float*)b;
    b += align_up(nc * 4, 256);
    int32_t* scnt = (int32_t*)b;
    b += align_up((size_t)g.B * (max_slices(g) + 1) * 4, 256);
    uint32_t* bhist = (uint32_t*)b;
    const uint8_t* pg = (const uint8_t*)pages;
    const uint16_t* qq = (const uint16_t*)q;
    int grid = grid_hint;
    if (grid <= 0) grid = (int)(items < 4096 ? items : 4096);
    if (grid < 1) grid = 1;
    const int Hh = H;
    hipError_t e = hipErrorInvalidValue;
    timing_begin("k_refine_mfma", s);
#define LSA_K1(KDT, D, HH)                                                                        \
    if (idx_dt == KDT && d == D && Hh == HH) {                                                    \
        hipLaunchKernelGGL((k_refine_mfma<KDT, D, HH>), dim3(grid), dim3(64 * kBandWaves), 0, s, g, \
                           sel, cnt, pg, page_bytes, ikey_off, page_table, ikey_scale, qq, w, lu,  \
                           stats, bhist);                                                         \
        e = hipGetLastError();                                                                    \
    }
    LSA_K1(LSA_BF16, 128, 16) LSA_K1(LSA_BF16, 128, 32) LSA_K1(LSA_BF16, 128, 64)
    LSA_K1(LSA_BF16, 128, 128) LSA_K1(LSA_BF16, 64, 16) LSA_K1(LSA_BF16, 64, 32)
    LSA_K1(LSA_BF16, 64, 64) LSA_K1(LSA_BF16, 64, 128)
    LSA_K1(LSA_FP8_E4M3FN, 128, 16) LSA_K1(LSA_FP8_E4M3FN, 128, 32) LSA_K1(LSA_FP8_E4M3FN, 128, 64)
    LSA_K1(LSA_FP8_E4M3FN, 128, 128) LSA_K1(LSA_FP8_E4M3FN, 64, 16) LSA_K1(LSA_FP8_E4M3FN, 64, 32)
    LSA_K1(LSA_FP8_E4M3FN, 64, 64) LSA_K1(LSA_FP8_E4M3FN, 64, 128)
#undef LSA_K1
    timing_end("k_refine_mfma", s);
    if (e != hipSuccess) return e;
    const dim3 sg(nslices, g.B);
    timing_begin("k_band_hist", s);
    hipLaunchKernelGGL(k_band_hist, sg, dim3(256), 0, s, g, cnt, lu, stats, k, bhist);
    timing_end("k_band_hist", s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    timing_begin("k_band_list", s);
    hipLaunchKernelGGL(k_band_list, sg, dim3(256), 0, s, g, sel, cnt, lu, stats, k, bhist, ulist,
                       scnt, topk, tcnt, nslices);
    timing_end("k_band_list", s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = hipErrorInvalidValue;
    timing_begin("k_rescore", s);
#define LSA_K3(KDT, D, HH)                                                                        \
    if (idx_dt == KDT && d == D && Hh == HH) {                                                    \
        hipLaunchKernelGGL((k_rescore<KDT, D, HH>), sg, dim3(256), 0, s, g, sel, cnt, ulist, scnt, \
                           nslices, k, pg, page_bytes, ikey_off, page_table, ikey_scale, qq, w,   \
                           exact);                                                                \
        e = hipGetLastError();                                                                    \
    }
    LSA_K3(LSA_BF16, 128, 16) LSA_K3(LSA_BF16, 128, 32) LSA_K3(LSA_BF16, 128, 64)
    LSA_K3(LSA_BF16, 64, 16) LSA_K3(LSA_BF16, 64, 32) LSA_K3(LSA_BF16, 64, 64)
    LSA_K3(LSA_BF16, 64, 128)
    LSA_K3(LSA_FP8_E4M3FN, 128, 16) LSA_K3(LSA_FP8_E4M3FN, 128, 32) LSA_K3(LSA_FP8_E4M3FN, 128, 64)
    LSA_K3(LSA_FP8_E4M3FN, 64, 16) LSA_K3(LSA_FP8_E4M3FN, 64, 32) LSA_K3(LSA_FP8_E4M3FN, 64, 64)
    LSA_K3(LSA_FP8_E4M3FN, 64, 128)
#undef LSA_K3
    timing_end("k_rescore", s);
    if (e != hipSuccess) return e;
    timing_begin("k_topk_list", s);
    hipLaunchKernelGGL(k_topk_list, dim3(g.B), dim3(kT), 0, s, g, sel, cnt, ulist, scnt, nslices,
                       exact, k, topk, tcnt);
    timing_end("k_topk_list", s);
    return hipGetLastError();
}
