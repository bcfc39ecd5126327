// Per-head sigmoid chunk score (gfx950).
//
// The memory indexer is the lightning indexer with its ReLU replaced by a
// sigmoid, so that its score is a probability and a fixed 0.5 decides the
// fetch (cjcn.com.cn explainer, section 二).  Read per head, for history
// chunk c of request r:
//     a_h = q_h . k_c,   x_h = s_c a_h + b,   S_c = sum_h w_h sigmoid(x_h),
// fetched when S_c > theta (0.5).  The canonical fp32 order: per head an fma
// chain over i from +0, x_h = fma(s_c, a_h, b), S an fma chain over h from
// +0, and one written fp32 sigmoid (sigmoid_fp32).
//
// k_score_sig       the canonical order for every chunk, one lane per chunk
//                   (the path for fp32 queries or keys); fp32-vector-bound
//                   at H*d fma per chunk.
// k_score_sig_mfma  bf16 queries with bf16 or fp8 keys: a'_h for a tile of
//                   64 chunks and every head on the matrix cores as
//                   S^T = Q K^T (heads are the rows, so most of the head sum
//                   stays inside a lane), a fast sigmoid, and a bound E_c
//                   with |S'_c - S_c| <= E_c.  Chunks with |S'_c - theta| <=
//                   E_c get the canonical S_c, computed by the wave with one
//                   lane per head; every other chunk keeps S'_c, which lies
//                   on the same side of theta as S_c.  So S > theta decides
//                   exactly as the canonical order does, and S is within
//                   E_c of it everywhere.
//
// The bound.  The canonical chain and the MFMA sum each differ from the
// exact dot product by at most gamma(d) sum_i |q_i k_i| <= gamma(d) |q_h|
// |k_c| (Higham's bound for any summation order, with two ulps per
// operation; Cauchy-Schwarz); x adds one rounding on each side.  The
// sigmoid is 1/4-Lipschitz; the fast sigmoid (v_exp_f32, v_rcp_f32) and the
// canonical one are each within a few ulps of the exact function, far
// inside the allowance kSigAllow per head; each head sum adds
// gamma(H) sum_h |w_h|.  |k_c|^2 comes from the diagonal of the chunk
// block's Gram matrix on the matrix cores.
#include "lsa_internal.h"
#include "mfma_util.h"

#include <algorithm>

namespace {

using namespace lsa_dev;

__device__ __forceinline__ float bf16f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// The canonical sigmoid: 1 / (1 + 2^t), t = clamp(-x log2 e, -200, 200),
// 2^t = 2^n P(f) with n = rint(t), f = t - n and P the degree-7 Taylor
// polynomial of 2^f (coefficients (ln 2)^k / k!, nearest fp32) in Horner fma
// form; IEEE divide.
__device__ __forceinline__ float sigmoid_fp32(float x) {
    constexpr float kLog2e = 0x1.715476p+0f;
    constexpr float c0 = 0x1p+0f, c1 = 0x1.62e430p-1f, c2 = 0x1.ebfbe0p-3f, c3 = 0x1.c6b08ep-5f,
                    c4 = 0x1.3b2ab6p-7f, c5 = 0x1.5d87fep-10f, c6 = 0x1.430912p-13f, c7 = 0x1.ffcbfcp-17f;
    float t = -x * kLog2e;
    t = fminf(fmaxf(t, -200.0f), 200.0f);
    const float n = rintf(t);
    const float f = t - n;
    float p = __builtin_fmaf(c7, f, c6);
    p = __builtin_fmaf(p, f, c5);
    p = __builtin_fmaf(p, f, c4);
    p = __builtin_fmaf(p, f, c3);
    p = __builtin_fmaf(p, f, c2);
    p = __builtin_fmaf(p, f, c1);
    p = __builtin_fmaf(p, f, c0);
    return 1.0f / (1.0f + ldexpf(p, (int)n));
}

// Per head: the fast sigmoid's (1 / (1 + 2^t) with v_exp_f32 and v_rcp_f32)
// and the canonical one's distance from the exact function together (a few
// 1e-7 in fact).
constexpr float kSigAllow = 0x1p-14f;

// Waves per block of the one-lane-per-chunk kernel, so that its LDS tiles
// stay near 36 KB.
template <int KDT, int D>
constexpr int score_waves() {
    constexpr int rowb = D * (KDT == LSA_F32 ? 4 : (KDT == LSA_BF16 ? 2 : 1));
    return rowb <= 128 ? 4 : (rowb <= 256 ? 2 : 1);
}

// One lane per chunk: the lane decodes its key row once into registers; the
// request's queries and weights are decoded once per block into LDS (fp32)
// and read as broadcasts.  H * d <= 8192.
constexpr int kSigMaxHD = 8192;

template <int KDT, int D>
__global__ __launch_bounds__((64 * score_waves<KDT, D>())) void k_score_sig(
    GeomDev g, const uint8_t* __restrict__ kic, const float* __restrict__ kscale,
    const void* __restrict__ q, int q_dt, const float* __restrict__ w, int H,
    const float* __restrict__ bias, float* __restrict__ S) {
    constexpr int kScoreWaves = score_waves<KDT, D>();
    constexpr int EB = KDT == LSA_F32 ? 4 : (KDT == LSA_BF16 ? 2 : 1);
    constexpr int ROWB = D * EB;
    constexpr int PIECES = ROWB / 16;
    constexpr int STRIDE = ROWB + 16;
    __shared__ __attribute__((aligned(16))) uint8_t tile[kScoreWaves][64 * STRIDE];
    __shared__ __attribute__((aligned(16))) float qs[kSigMaxHD];
    __shared__ float ws_[kSigMaxHD / 64];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int r = blockIdx.y;
    const int nh = g.nhist[r];
    const int ntile = (nh + 63) >> 6;
    const int step = gridDim.x * kScoreWaves;
    if ((int)blockIdx.x * kScoreWaves >= ntile) return;  // uniform across the block
    for (int e = threadIdx.x; e < H * D; e += blockDim.x) {
        const size_t src = (size_t)r * H * D + e;
        qs[e] = q_dt == LSA_F32 ? ((const float*)q)[src] : bf16f(((const uint16_t*)q)[src]);
    }
    for (int h = threadIdx.x; h < H; h += blockDim.x) ws_[h] = w[(size_t)r * H + h];
    __syncthreads();
    int t = blockIdx.x * kScoreWaves + wv;
    if (t >= ntile) return;  // whole wave leaves together
    const int64_t off = g.chunk_off[r];
    const float br = bias[r];
    uint8_t* lt = tile[wv];
    for (; t < ntile; t += step) {
        const int nvalid = min(64, nh - t * 64);
        const uint4* src = (const uint4*)(kic + (off + (int64_t)t * 64) * ROWB);
#pragma unroll
        for (int j = 0; j < PIECES; ++j) {
            const int piece = j * 64 + lane;
            const uint4 v = (piece / PIECES < nvalid) ? src[piece] : make_uint4(0, 0, 0, 0);
            *(uint4*)(lt + (piece / PIECES) * STRIDE + (piece % PIECES) * 16) = v;
        }
        const float sc = (KDT == LSA_FP8_E4M3FN && lane < nvalid) ? kscale[off + (int64_t)t * 64 + lane] : 1.0f;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // this lane's key row, decoded once
        float kf[D];
        const uint4* row = (const uint4*)(lt + lane * STRIDE);
#pragma unroll
        for (int j = 0; j < PIECES; ++j) {
            const uint4 v = row[j];
            const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
            if constexpr (KDT == LSA_F32) {
#pragma unroll
                for (int e = 0; e < 4; ++e) kf[4 * j + e] = __uint_as_float(wd[e]);
            } else if constexpr (KDT == LSA_BF16) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kf[8 * j + 2 * e] = __uint_as_float(wd[e] << 16);
                    kf[8 * j + 2 * e + 1] = __uint_as_float(wd[e] & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[e], false);
                    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[e], true);
                    kf[16 * j + 4 * e] = lo[0];
                    kf[16 * j + 4 * e + 1] = lo[1];
                    kf[16 * j + 4 * e + 2] = hi[0];
                    kf[16 * j + 4 * e + 3] = hi[1];
                }
            }
        }
        float acc_s = 0.0f;
        for (int h = 0; h < H; ++h) {
            const float4* qh = (const float4*)(qs + h * D);
            float a = 0.0f;
#pragma unroll
            for (int i = 0; i < D / 4; ++i) {
                const float4 qv = qh[i];
                a = __builtin_fmaf(qv.x, kf[4 * i], a);
                a = __builtin_fmaf(qv.y, kf[4 * i + 1], a);
                a = __builtin_fmaf(qv.z, kf[4 * i + 2], a);
                a = __builtin_fmaf(qv.w, kf[4 * i + 3], a);
            }
            const float x = __builtin_fmaf(sc, a, br);
            acc_s = __builtin_fmaf(ws_[h], sigmoid_fp32(x), acc_s);
        }
        if (lane < nvalid) S[off + (int64_t)t * 64 + lane] = acc_s;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();  // the LDS tile is rewritten next round
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// ---------------------------------------------------------------------------
// Grid (X, B), kSigWaves waves per block: wave (x, wv) of request r takes
// tiles x*kSigWaves + wv, stepping by X*kSigWaves, and loads the next tile's
// key rows while the current one is on the matrix cores.  Queries (A
// operands and an LDS copy for the canonical re-score), weights and the
// bound's query terms are set up once per block.  Heads are padded to
// 16*HB with zero weight and zero query.
constexpr int kSigWaves = 4;

template <int KDT, int D, int HB>
__global__ __launch_bounds__(64 * kSigWaves, 2) void k_score_sig_mfma(
    GeomDev g, const uint8_t* __restrict__ kic, const float* __restrict__ kscale,
    const uint16_t* __restrict__ q, const float* __restrict__ w, int H,
    const float* __restrict__ bias, float theta, float* __restrict__ S) {
    constexpr int EB = KDT == LSA_BF16 ? 2 : 1;
    constexpr int ROWB = D * EB;
    constexpr int KS = D / 32;                          // MFMA k-steps
    constexpr int NR = KDT == LSA_BF16 ? KS : KS / 2;   // 16-byte key loads per row and lane
    constexpr int HP = HB * 16;                         // padded heads
    constexpr int QST = D + 8;                          // query row stride in LDS (bf16)
    __shared__ __attribute__((aligned(16))) uint16_t qsh[HP * QST];
    __shared__ __attribute__((aligned(16))) float wsh[HP];
    __shared__ __attribute__((aligned(16))) float sgw[kSigWaves][HP];
    __shared__ __attribute__((aligned(16))) uint8_t kbw[kSigWaves][4 * ROWB];  // band key rows

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, lq = lane >> 4;
    const int r = blockIdx.y;
    const int nh = g.nhist[r];
    const int ntile = (nh + 63) >> 6;
    if ((int)blockIdx.x * kSigWaves >= ntile) return;  // uniform across the block
    const int64_t off = g.chunk_off[r];
    const int stride = gridDim.x * kSigWaves;
    int t = blockIdx.x * kSigWaves + wv;
    const bool active = t < ntile;  // uniform across the wave

    // Loads in the order their results are needed (the memory counter
    // retires in order): queries and weights, then the first tile.  Heads
    // past H load head H-1 and are zeroed; rows past the end of the request
    // load its last row, whose results are never used.
    const uint16_t* qr = q + (int64_t)r * H * D;
    const float* wr = w + (int64_t)r * H;
    uint4 qb[HB][KS];   // A operands: head hb*16 + l16, dims kdim(ks, lq)
    float wl[HB][4];    // weights of the output rows held: heads hb*16 + 4*lq + e
    float wa[HB];       // |w| of head hb*16 + l16
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        const int h = hb * 16 + l16, hc = min(h, H - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qb[hb][ks] = *(const uint4*)(qr + hc * D + kdim<KDT>(ks, lq));
        wa[hb] = wr[hc];
#pragma unroll
        for (int e = 0; e < 4; ++e) wl[hb][e] = wr[min(hb * 16 + 4 * lq + e, H - 1)];
    }
    const float br = bias[r];

    // key rows of tile tt (B operands of chunks tb*16 + l16) and their
    // scales.  Where the registers allow, two sets take turns (one in flight
    // while the other is on the matrix cores); otherwise one set is copied
    // into operands before the next tile is fetched into it.
    constexpr bool kTwoSets = 2 * 4 * NR * 4 + HB * KS * 4 <= 160;
    uint4 rawA[4][NR], rawB[4][kTwoSets ? NR : 1];
    float scA[4], scB[4];
    auto fetch = [&](int tt, uint4 (&dst)[4][NR], float (&dsc)[4]) __attribute__((always_inline)) {
        const int last = min(64, nh - tt * 64) - 1;
        const uint8_t* base = kic + (off + (int64_t)tt * 64) * ROWB;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int row = min(tb * 16 + l16, last);
#pragma unroll
            for (int n = 0; n < NR; ++n) dst[tb][n] = *(const uint4*)(base + row * ROWB + n * 64 + lq * 16);
            if constexpr (KDT == LSA_FP8_E4M3FN) dsc[tb] = kscale[off + (int64_t)tt * 64 + row];
            else dsc[tb] = 1.0f;
        }
    };
    if (active) fetch(t, rawA, scA);

#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        const bool hv = hb * 16 + l16 < H;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) if (!hv) qb[hb][ks] = make_uint4(0, 0, 0, 0);
        wa[hb] = hv ? fabsf(wa[hb]) : 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) if (hb * 16 + 4 * lq + e >= H) wl[hb][e] = 0.0f;
    }
    // LDS copies for the canonical re-score, from the registers: wave 0's
    // operands cover every (head, dim); its lanes with l16 == 0 every weight
    if (wv == 0) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                *(uint4*)(qsh + (hb * 16 + l16) * QST + kdim<KDT>(ks, lq)) = qb[hb][ks];
            if (l16 == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) wsh[hb * 16 + 4 * lq + e] = wl[hb][e];
            }
        }
    }
    // Wq = sum_h |w_h| |q_h|_2 and W1 = sum_h |w_h|, rounded up
    float part = 0.0f, pw = 0.0f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        float ss = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ss += sumsq_bf16x8(qb[hb][ks]);
        ss = add_xor32(add_xor16(ss));
        part += wa[hb] * sqrtf(ss * (1.0f + gam(D + 8))) * (1.0f + 4 * kU2);
        pw += wa[hb];
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        part += __shfl_xor(part, o);
        pw += __shfl_xor(pw, o);
    }
    const float wq = part * (1.0f + gam(HP + 8));
    const float w1 = pw * (1.0f + gam(HP + 8));
    __syncthreads();
    if (!active) return;

    float* sg = sgw[wv];
    uint8_t* kband = kbw[wv];
    const float btl = br * -0x1.715476p+0f;  // bias times -log2 e
    // one tile: S' and the bound for its 64 chunks, the canonical S where the
    // bound leaves the side of theta open, the results to S
    // cur holds tile tt; the next tile of this wave is fetched into nxt once
    // cur has been taken into operands (nxt may be cur itself)
    auto tile = [&](int tt, uint4 (&cur)[4][NR], float (&csc)[4], uint4 (&nxt)[4][NR], float (&nsc)[4])
        __attribute__((always_inline)) {
        const int nvalid = min(64, nh - tt * 64);
        uint4 ka[4][KS];
        float sct[4], scr[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            scr[tb] = csc[tb];
            sct[tb] = csc[tb] * -0x1.715476p+0f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if constexpr (KDT == LSA_BF16) ka[tb][ks] = cur[tb][ks];
                else ka[tb][ks] = (ks & 1) ? fp8x8_to_bf16x8(cur[tb][ks >> 1].z, cur[tb][ks >> 1].w)
                                           : fp8x8_to_bf16x8(cur[tb][ks >> 1].x, cur[tb][ks >> 1].y);
            }
        }
        if (tt + stride < ntile) fetch(tt + stride, nxt, nsc);
        // lane = chunk tb*16 + l16 with tb == lq: S', |k|^2, the scale
        float mS = 0.0f, kn2 = 0.0f, ms = 1.0f;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            // Gram block of chunks tb*16..: lane (l16, lq) holds rows
            // 4lq..4lq+3 of column l16; the diagonal entry of chunk j sits in
            // lane (j, j >> 2), register j & 3
            f32x4_t gm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                gm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka[tb][ks]),
                                                            __builtin_bit_cast(bf16x8_t, ka[tb][ks]), gm,
                                                            0, 0, 0);
            const int e3 = l16 & 3;
            const float dv = e3 == 0 ? gm[0] : (e3 == 1 ? gm[1] : (e3 == 2 ? gm[2] : gm[3]));
            const float dd = __shfl(dv, ((l16 >> 2) << 4) | l16);
            float sS = 0.0f;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                f32x4_t c4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qb[hb][ks]),
                                                                __builtin_bit_cast(bf16x8_t, ka[tb][ks]),
                                                                c4, 0, 0, 0);
                // c4[e] = a'[head hb*16 + 4lq + e][chunk tb*16 + l16]; the
                // sigmoid's argument -x' log2 e in one fma
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float tx = __builtin_fmaf(sct[tb], c4[e], btl);
                    sS = __builtin_fmaf(wl[hb][e],
                                        __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(tx)), sS);
                }
            }
            sS = add_xor32(add_xor16(sS));
            if (lq == tb) {
                mS = sS;
                kn2 = dd;
                ms = scr[tb];
            }
        }
        // |x'_h| <= s |q_h| |k| + |b|, so sum_h |w_h| |x'_h| <= xs
        const float kn = sqrtf(kn2 * (1.0f + gam(D + 8))) * (1.0f + 4 * kU2);
        const float skw = fabsf(ms) * kn * wq;
        const float xs = (skw * (1.0f + gam(D)) + w1 * fabsf(br)) * (1.0f + 4 * kU2);
        const float da = 2.0f * gam(D) * skw;  // sum_h |w_h| s |a'_h - a_h|
        const float dx = da * (1.0f + 4 * kU2) + 3.0f * kU2 * (xs + da);
        float E = 0.25f * dx + w1 * (kSigAllow + 2.0f * gam(HP + 8));
        E = E * (1.0f + 16 * kU2) + 1e-30f;
        uint64_t bm = __ballot(lane < nvalid && fabsf(mS - theta) <= E);
        // canonical S for the chunks the bound leaves open, four at a time:
        // their key rows and scales come in one round of loads
        while (bm) {
            int cg[4];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                cg[g4] = bm ? (int)__builtin_ctzll(bm) : -1;
                bm &= bm - 1;
            }
            const int gi = lane >> 4, pc = lane & 15;
            const int cme = gi == 0 ? cg[0] : (gi == 1 ? cg[1] : (gi == 2 ? cg[2] : cg[3]));
            if (cme >= 0 && pc < ROWB / 16)
                *(uint4*)(kband + gi * ROWB + pc * 16) =
                    *(const uint4*)(kic + (off + (int64_t)tt * 64 + cme) * ROWB + pc * 16);
            float scg = 1.0f;
            if constexpr (KDT == LSA_FP8_E4M3FN) {
                const int cl = lane == 0 ? cg[0] : (lane == 1 ? cg[1] : (lane == 2 ? cg[2] : (lane == 3 ? cg[3] : -1)));
                if (cl >= 0) scg = kscale[off + (int64_t)tt * 64 + cl];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                if (cg[g4] < 0) break;
                const float s_c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(scg), g4));
                const uint8_t* kr = kband + g4 * ROWB;
#pragma unroll
                for (int hh = 0; hh < HP; hh += 64) {
                    const int h = hh + lane;
                    if (h < HP) {
                        const uint16_t* qh = qsh + h * QST;
                        float a = 0.0f;
#pragma unroll 4
                        for (int j = 0; j < D / 8; ++j) {
                            const uint4 qv = *(const uint4*)(qh + j * 8);
                            const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
                            float kf[8];
                            if constexpr (KDT == LSA_BF16) {
                                const uint4 kv = *(const uint4*)(kr + j * 16);
                                const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    kf[2 * e] = __uint_as_float(kw[e] << 16);
                                    kf[2 * e + 1] = __uint_as_float(kw[e] & 0xffff0000u);
                                }
                            } else {
                                const uint2 kv = *(const uint2*)(kr + j * 8);
                                const uint32_t kw[2] = {kv.x, kv.y};
#pragma unroll
                                for (int e = 0; e < 2; ++e) {
                                    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)kw[e], false);
                                    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)kw[e], true);
                                    kf[4 * e] = lo[0];
                                    kf[4 * e + 1] = lo[1];
                                    kf[4 * e + 2] = hi[0];
                                    kf[4 * e + 3] = hi[1];
                                }
                            }
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                a = __builtin_fmaf(__uint_as_float(qw[e] << 16), kf[2 * e], a);
                                a = __builtin_fmaf(__uint_as_float(qw[e] & 0xffff0000u), kf[2 * e + 1], a);
                            }
                        }
                        sg[h] = sigmoid_fp32(__builtin_fmaf(s_c, a, br));
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                // the head chain over the padded heads: a zero weight adds
                // fma(0, sigmoid, acc) = acc exactly
                float acc = 0.0f;
#pragma unroll
                for (int h4 = 0; h4 < HP / 4; ++h4) {
                    const float4 wv4 = *(const float4*)(wsh + 4 * h4);
                    const float4 sg4 = *(const float4*)(sg + 4 * h4);
                    acc = __builtin_fmaf(wv4.x, sg4.x, acc);
                    acc = __builtin_fmaf(wv4.y, sg4.y, acc);
                    acc = __builtin_fmaf(wv4.z, sg4.z, acc);
                    acc = __builtin_fmaf(wv4.w, sg4.w, acc);
                }
                if (lane == cg[g4]) mS = acc;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();  // sg[] is rewritten for the next chunk
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
        }
        if (lane < nvalid) S[off + (int64_t)tt * 64 + lane] = mS;
    };
    if constexpr (kTwoSets) {
        for (;;) {
            tile(t, rawA, scA, rawB, scB);
            t += stride;
            if (t >= ntile) break;
            tile(t, rawB, scB, rawA, scA);
            t += stride;
            if (t >= ntile) break;
        }
    } else {
        for (; t < ntile; t += stride) tile(t, rawA, scA, rawA, scA);
    }
}

}  // namespace

hipError_t launch_score_sig(const GeomDev& g, const void* kic, lsa_dtype kdt, const float* kscale,
                            const void* q, lsa_dtype q_dt, const float* w, int H, const float* bias,
                            float theta, int d, float* S, hipStream_t s) {
    const int tiles = g.tile_off[g.B];
    if (tiles == 0) return hipSuccess;
    int mt = 0;  // tiles of the longest request
    for (int r = 0; r < g.B; ++r) mt = g.tile_off[r + 1] - g.tile_off[r] > mt ? g.tile_off[r + 1] - g.tile_off[r] : mt;
    const uint8_t* k = (const uint8_t*)kic;
    const int hmax = d == 128 ? 64 : 128;
    if (q_dt == LSA_BF16 && kdt != LSA_F32 && H <= hmax) {
        // about two blocks per compute unit, each wave with at least one tile
        const int X = std::max(1, std::min((512 + g.B - 1) / g.B, (mt + kSigWaves - 1) / kSigWaves));
        const int hb = H <= 16 ? 1 : (H <= 32 ? 2 : (H <= 64 ? 4 : 8));
        const uint16_t* qq = (const uint16_t*)q;
#define LSA_SIGM_CASE(KDT, D, HB)                                                               \
        if (kdt == KDT && d == D && hb == HB) {                                                 \
            timing_begin("k_score_sig", s);                                                     \
            hipLaunchKernelGGL((k_score_sig_mfma<KDT, D, HB>), dim3(X, g.B), dim3(64 * kSigWaves), \
                               0, s, g, k, kscale, qq, w, H, bias, theta, S);                   \
            timing_end("k_score_sig", s);                                                       \
            return hipGetLastError();                                                           \
        }
        LSA_SIGM_CASE(LSA_BF16, 128, 1)
        LSA_SIGM_CASE(LSA_BF16, 128, 2)
        LSA_SIGM_CASE(LSA_BF16, 128, 4)
        LSA_SIGM_CASE(LSA_BF16, 64, 1)
        LSA_SIGM_CASE(LSA_BF16, 64, 2)
        LSA_SIGM_CASE(LSA_BF16, 64, 4)
        LSA_SIGM_CASE(LSA_BF16, 64, 8)
        LSA_SIGM_CASE(LSA_FP8_E4M3FN, 128, 1)
        LSA_SIGM_CASE(LSA_FP8_E4M3FN, 128, 2)
        LSA_SIGM_CASE(LSA_FP8_E4M3FN, 128, 4)
        LSA_SIGM_CASE(LSA_FP8_E4M3FN, 64, 1)
        LSA_SIGM_CASE(LSA_FP8_E4M3FN, 64, 2)
        LSA_SIGM_CASE(LSA_FP8_E4M3FN, 64, 4)
        LSA_SIGM_CASE(LSA_FP8_E4M3FN, 64, 8)
#undef LSA_SIGM_CASE
        return hipErrorInvalidValue;
    }
    if (H * d > kSigMaxHD) return hipErrorInvalidValue;
#define LSA_SIG_CASE(KDT, D)                                                                    \
    if (kdt == KDT && d == D) {                                                                 \
        constexpr int nw = score_waves<KDT, D>();                                               \
        timing_begin("k_score_sig", s);                                                         \
        hipLaunchKernelGGL((k_score_sig<KDT, D>), dim3((mt + 2 * nw - 1) / (2 * nw), g.B),       \
                           dim3(64 * nw), 0, s, g, k, kscale, q, (int)q_dt, w, H, bias, S);     \
        timing_end("k_score_sig", s);                                                           \
        return hipGetLastError();                                                               \
    }
    LSA_SIG_CASE(LSA_F32, 64)
    LSA_SIG_CASE(LSA_F32, 128)
    LSA_SIG_CASE(LSA_BF16, 64)
    LSA_SIG_CASE(LSA_BF16, 128)
    LSA_SIG_CASE(LSA_FP8_E4M3FN, 64)
    LSA_SIG_CASE(LSA_FP8_E4M3FN, 128)
#undef LSA_SIG_CASE
    return hipErrorInvalidValue;
}
