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
//     U = I' + E as order-preserving 32-bit keys and adds to the request's
//     coarse histograms of L and U (top 10 key bits).
//  K2 k_band_fine    every block finds the coarse bins holding the k-th
//     largest L and the k-th largest U, then adds fine histograms (2048-key
//     bins) of the keys inside those two coarse bins.
//  K3 k_band_list    every block finds tau = lowest key of the fine bin
//     holding the k-th largest L and edge = first key above the fine bin
//     holding the k-th largest U.  Candidates with U >= tau form the band
//     (never fewer than k); each block lists its share in token order.
//     Those with L >= edge are certain to be in the top-k; the rest of the
//     band (uncertain) gets the canonical score, by the same block.
//  K4 k_topk_band    exact top-k over the band (certain ones rank first),
//     ties to the lower token, emitted in token order; clears the
//     histograms for the next launch.
// Why it is exact.  A candidate outside the band has I <= U < tau, and at
// least k candidates have I >= L >= tau: it is below k others.  A certain
// candidate s has L_s >= edge; any t with I_t >= I_s has U_t >= L_s >= edge,
// and fewer than k candidates (s included) have U >= edge: fewer than k
// others can rank above s.  So the top-k is the certain set plus the best
// of the uncertain ones, by canonical score and then by token.
//
// The bound.  Both the canonical chain and the MFMA sum differ from the exact
// dot product by at most gamma(n) * sum_i |q_i k_i| (any summation order,
// one rounding per operation, Higham's bound), taken here with two ulps per
// operation (u = 2^-22) to cover truncating accumulation;
// sum_i |q_i k_i| <= |q_h| |key| (Cauchy-Schwarz).  ReLU is 1-Lipschitz and
// the head sums add gamma(H) * sum_h |w_h| (ReLU(a'_h) + eps_h).
#include "lsa_internal.h"
#include "mfma_util.h"

#include <type_traits>

namespace {

using namespace lsa_dev;

// max(x, +0) with +0 for every negative value and for -0: as a signed
// integer the bit pattern of a negative float is negative (one instruction,
// where fmaxf also quiets NaNs)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ uint32_t fkey(float f) {
    const uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kWaves = 4;         // waves per block of K1 and K3
constexpr int kCoarse = 1024;     // coarse bins: key >> 22
constexpr int kFine = 2048;       // fine bins inside one coarse bin: (key >> 11) & 2047
constexpr int kHist = 2 * kCoarse + 2 * kFine;  // per request: coarse L, U, then fine L, U
constexpr int kT = 1024, kTW = kT / 64;
constexpr int kMaxSeg = 1024;     // band list segments (K3 blocks) per request, at most
constexpr int kListCap = 8192;    // band entries K4 keeps in LDS
constexpr int kUncCap = 1024;     // uncertain entries K4 ranks directly
constexpr int kPgCap = 256;       // chunks per K3 block whose pages K3 keeps in LDS
constexpr int kUclCap = 512;      // uncertain entries per K3 block kept in LDS
constexpr int kRs = 64;           // uncertain entries K3 re-scores per round
constexpr int kSelCap = 8192;     // selected chunk ids K4 keeps in LDS

// ---------------------------------------------------------------------------
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
    lds_barrier();
    int wpre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int x = wsum[i];
        wpre += (i < wv) ? x : 0;
        tot += x;
    }
    lds_barrier();
    total = tot;
    return wpre + incl - v;
}

// Bin holding the k-th largest entry of hist[0, NB) -> out[0], and the
// number of entries in higher bins -> out[1].  Thread t owns the BPT bins
// below NB - t*BPT.  Every thread of the block (NW waves) must call; the
// caller guarantees at least k entries.
template <int NB, int NW>
__device__ __forceinline__ void kth_bin(const uint32_t* hist, int k, int* wsum, int* out) {
    constexpr int BPT = NB / (64 * NW);
    const int tid = threadIdx.x;
    int c[BPT], sum = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        c[j] = (int)hist[NB - 1 - (tid * BPT + j)];
        sum += c[j];
    }
    int tot;
    const int excl = block_scan<NW>(sum, wsum, tot);
    if (excl < k && excl + sum >= k) {
        int acc = excl, j = 0;
        for (; j < BPT - 1; ++j) {
            if (acc + c[j] >= k) break;
            acc += c[j];
        }
        out[0] = NB - 1 - (tid * BPT + j);
        out[1] = acc;
    }
    lds_barrier();
}

// Copies N words of a histogram into LDS (16 bytes per load, every load of
// the block's NT threads in flight at once; both pointers 16-byte aligned).
template <int N, int NT>
__device__ __forceinline__ void load_hist(const uint32_t* gh, uint32_t* lds) {
    constexpr int PER = N / 4 / NT;
    static_assert(PER * 4 * NT == N, "histogram words must split evenly");
    uint4 v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = ((const uint4*)gh)[threadIdx.x + NT * j];
#pragma unroll
    for (int j = 0; j < PER; ++j) ((uint4*)lds)[threadIdx.x + NT * j] = v[j];
    lds_barrier();
}

// ---------------------------------------------------------------------------
// K1.  Grid (X, B): wave x*4 + v of request r takes the whole chunks
// x*4 + v + j*4X below 4X * floor(n / 4X), n the request's selection count,
// and a run of at most four 16-token parts of the remaining chunks.  The query rows are the A operands (rows = heads), a chunk's key rows
// the B operands (columns = tokens), so D = Q K^T leaves each lane four heads
// of one token: the weighted head sum runs inside the lane and across the
// four lane groups by two permlane swaps, with no trip through LDS.  Key rows
// stay in flight ahead of the chunk being computed: each 16-token part of a
// key buffer is refilled with the next chunk's part (or the wave's remainder
// part) as soon as it has been converted.  The block's coarse histograms go to the request's (hist, zero on
// entry) with one atomic per nonzero bin.
template <int KDT, int D, int H>
__global__ __launch_bounds__(64 * kWaves, (H * D > 64 * 128 ? 1 : 2)) void k_refine_mfma(
    GeomDev g, const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt,
    const uint8_t* __restrict__ pages, int64_t page_bytes, int64_t ikey_off,
    const int32_t* __restrict__ page_table, const float* __restrict__ ikey_scale,
    const int32_t* __restrict__ sel_slot, const float* __restrict__ sel_scale,
    const float* __restrict__ kn2g, const uint16_t* __restrict__ q, const float* __restrict__ w,
    uint2* __restrict__ lu, uint32_t* __restrict__ hist) {
    constexpr int EB = KDT == LSA_BF16 ? 2 : 1;
    constexpr int ROWB = D * EB;
    constexpr int KS = D / 32;   // MFMA k-steps
    constexpr int HB = H / 16;   // head blocks
    constexpr int NR = KDT == LSA_BF16 ? KS : KS / 2;  // 16-byte key loads per token row and lane
    constexpr int QROW = D * 2 + 16;      // bytes per query row in LDS (padded: no bank conflicts)
    // One key buffer is in flight ahead of the chunk computed.  A second with
    // fp8 keys (8 registers per 16 tokens) kept the same occupancy (2 waves
    // per SIMD) and was slower: 20.5 against 19.4 us per step at 500K batch 8.
    __shared__ uint32_t hl[2 * kCoarse];  // coarse L bins, then coarse U bins
    __shared__ __attribute__((aligned(16))) uint8_t qs[H * QROW];

    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, lq = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = blockIdx.y, X = gridDim.x;
    const int64_t off = g.chunk_off[r];
    const int nhr = g.nhist[r];
    const int stride = X * kWaves;
    const int i0 = blockIdx.x * kWaves + wv;  // this wave's chunks: i0 + j * stride
    // chunk j0 + lane: page (slot) index and scale, 64 chunks at a time.  The
    // first window is requested together with the selection count, before
    // the count is known (bounded by the request's chunks, so in range); the
    // entries past the count are never used.  With sel_slot the pages of the
    // selected chunks come resolved (one load instead of two).
    int64_t pg_l = 0;
    float sc_l = 1.0f;
    // the scales sit beside the resolved pages, or by chunk (one array for
    // both cases: a choice of array per load puts the pointers in scratch)
    const float* __restrict__ scl = sel_slot ? sel_scale : ikey_scale;
    auto load_idx = [&](int j0, int nlim) __attribute__((always_inline)) {
        if (j0 + lane < nlim) {
            const int i = i0 + (j0 + lane) * stride;
            int64_t e;  // the chunk's entry in the page and scale arrays
            if (sel_slot) {
                e = off + i;
                pg_l = (int64_t)sel_slot[e];
            } else {
                e = off + min(max(sel[off + i], 0), nhr - 1);
                pg_l = page_table ? (int64_t)page_table[e] : e;
            }
            if constexpr (KDT == LSA_FP8_E4M3FN) sc_l = scl[e];
        }
    };
    const int nj_max = i0 < nhr ? (nhr - i0 + stride - 1) / stride : 0;
    load_idx(0, nj_max);
    const int nc = cnt[r];
    // Work: every wave takes nj = nc / stride whole chunks (i0 + j * stride);
    // the 16-token parts of the remaining chunks (selection indices
    // nj * stride ..) are spread over all the request's waves, at most four
    // consecutive parts a wave, so that no wave does a whole chunk more than
    // another.
    const int nj = nc / stride;
    const int rem = nc - nj * stride;
    const int pr0 = (int)((4LL * rem * i0) / stride), pr1 = (int)((4LL * rem * (i0 + 1)) / stride);
    // key rows: B operands of tokens tb*16 + l16, 16 bytes per load; slot tb
    // holds part tb of the chunk computed next (or a remainder part)
    uint4 buf[4][NR];
    auto load_part = [&](const uint8_t* base, int tb) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < NR; ++n)
            buf[tb][n] = *(const uint4*)(base + (tb * 16 + l16) * ROWB + n * 64 + lq * 16);
    };
    // page base and scale of the chunk with selection index j (of this
    // wave's whole chunks), from the index window
    auto win_chunk = [&](int j, const uint8_t*& base, float& scale) __attribute__((always_inline)) {
        const int src = j & 63;
        const int64_t pgo = (int64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)pg_l, src) |
                            ((int64_t)__builtin_amdgcn_readlane((int)(pg_l >> 32), src) << 32);
        base = pages + pgo * page_bytes + ikey_off;
        scale = 1.0f;
        if constexpr (KDT == LSA_FP8_E4M3FN)
            scale = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc_l), src));
    };
    // the same for a remainder chunk (selection index i), loaded directly
    auto rem_chunk = [&](int i, const uint8_t*& base, float& scale) __attribute__((always_inline)) {
        int64_t e, pg;
        if (sel_slot) {
            e = off + i;
            pg = (int64_t)sel_slot[e];
        } else {
            e = off + min(max(sel[off + i], 0), nhr - 1);
            pg = page_table ? (int64_t)page_table[e] : e;
        }
        base = pages + pg * page_bytes + ikey_off;
        scale = 1.0f;
        if constexpr (KDT == LSA_FP8_E4M3FN) scale = scl[e];
    };
    // the query rows load once per block into LDS (each wave takes its
    // operands from there)
    {
        const uint4* qr = (const uint4*)(q + (int64_t)r * H * D);
        for (int e = tid; e < H * D / 8; e += 64 * kWaves)
            *(uint4*)(qs + (e / (D / 8)) * QROW + (e % (D / 8)) * 16) = qr[e];
    }
    // weights of the heads this lane's accumulators hold: hb*16 + 4*lq + i;
    // and of head hb*16 + l16, whose query operands the lane holds (bound)
    float wl[HB][4], wq_own[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) wl[hb][e] = w[(int64_t)r * H + hb * 16 + 4 * lq + e];
        wq_own[hb] = w[(int64_t)r * H + hb * 16 + l16];
    }
    for (int i = tid; i < 2 * kCoarse; i += 64 * kWaves) hl[i] = 0;
    lds_barrier();
    if (nj > 0 || pr1 > pr0) {  // uniform per wave
        uint4 qa[HB][KS];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qa[hb][ks] = *(const uint4*)(qs + (hb * 16 + l16) * QROW + kdim<KDT>(ks, lq) * 2);
        // The remainder parts [pr0, pr1) lie in at most two chunks, rc0 and
        // rc0 + 1, and each has a slot of its own (part p sits in slot p % 4):
        // all of them load together, after the wave's last whole chunk.
        const int rc0 = nj * stride + (pr0 >> 2);
        const uint8_t *rb0 = nullptr, *rb1 = nullptr;
        float rs0 = 1.0f, rs1 = 1.0f;
        if (pr1 > pr0) rem_chunk(rc0, rb0, rs0);
        if (pr1 > pr0 && ((pr1 - 1) >> 2) != (pr0 >> 2)) rem_chunk(rc0 + 1, rb1, rs1);
        // the remainder part of slot tb, or -1
        auto rem_part = [&](int tb) __attribute__((always_inline)) {
            const int p = pr0 + ((tb - pr0) & 3);
            return p < pr1 ? p : -1;
        };
        auto load_rem = [&](int tb) __attribute__((always_inline)) {
            const int p = rem_part(tb);
            if (p >= 0) load_part((p >> 2) != (pr0 >> 2) ? rb1 : rb0, tb);
        };
        const uint8_t* cbase = nullptr;  // the whole chunk in the slots
        float cscale = 1.0f;
        if (nj > 0) {
            win_chunk(0, cbase, cscale);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) load_part(cbase, tb);
        } else {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) load_rem(tb);
        }
        // Wq = sum_h |w_h| * |q_h|_2 (rounded up), from the operands held:
        // lane (l16, lq) has dims lq*8.. of every k-step of head hb*16 + l16
        float part = 0.0f;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            float ss = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) ss += sumsq_bf16x8(qa[hb][ks]);
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
            part += fabsf(wq_own[hb]) * sqrtf(ss * (1.0f + gam(D + 8))) * (1.0f + 4 * kU2);
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) part += __shfl_xor(part, o);
        const float wq = part * (1.0f + gam(H + 8));

        // slot tb's key rows as bf16 operands
        auto operands = [&](int tb, uint4 (&ka)[KS]) __attribute__((always_inline)) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if constexpr (KDT == LSA_BF16) ka[ks] = buf[tb][ks];
                else ka[ks] = (ks & 1) ? fp8x8_to_bf16x8(buf[tb][ks >> 1].z, buf[tb][ks >> 1].w)
                                       : fp8x8_to_bf16x8(buf[tb][ks >> 1].x, buf[tb][ks >> 1].y);
            }
        };
        // the weighted ReLU sums and (unless given) |key|^2 of tokens
        // tb*16 + l16, kept by the lanes of group lq == tb
        auto sums = [&](int tb, const uint4 (&ka)[KS], float& mI, float& mW, float& mK)
            __attribute__((always_inline)) {
            // |key|^2 on the matrix cores (unless given): the diagonal of the
            // 16x16 Gram block; lane (l16, lq) holds rows 4lq..4lq+3 of
            // column l16, so the diagonal of column l16 sits in lane group
            // l16 / 4, element l16 % 4
            if (!kn2g) {  // uniform
                f32x4_t gm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    gm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka[ks]),
                                                                 __builtin_bit_cast(bf16x8_t, ka[ks]), gm, 0, 0, 0);
                const int e = l16 & 3;
                const float dv = e == 0 ? gm[0] : (e == 1 ? gm[1] : (e == 2 ? gm[2] : gm[3]));
                const float dg = __shfl(dv, (l16 >> 2) * 16 + l16);
                if (lq == tb) mK = dg;
            }
            // a'[head hb*16 + 4lq + e][token tb*16 + l16]; weighted ReLU sums
            // over the lane's heads, then over the four lane groups
            float sI = 0.0f, sW = 0.0f;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                f32x4_t c4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[hb][ks]),
                                                                 __builtin_bit_cast(bf16x8_t, ka[ks]), c4, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float rr = relu(c4[e]);
                    sI = __builtin_fmaf(wl[hb][e], rr, sI);
                    sW = __builtin_fmaf(fabsf(wl[hb][e]), rr, sW);
                }
            }
            sI = add_xor32(add_xor16(sI));
            sW = add_xor32(add_xor16(sW));
            if (lq == tb) {  // lane lq * 16 + l16 keeps token tb * 16 + l16
                mI = sI;
                mW = sW;
            }
        };
        // the (L, U) keys of the lane's token of chunk i, and its coarse bins
        auto emit = [&](int64_t i, float scale, float mI, float mW, float mK) __attribute__((always_inline)) {
            // |key|^2 of the lane's token, formed once per window when given
            const float kn2 = kn2g ? kn2g[(off + i) * 64 + lane] : mK;
            const float kn = sqrtf(kn2 * (1.0f + gam(D + 8))) * (1.0f + 4 * kU2);
            const float ek = gam(D) * 2.0f * kn * wq;  // sum_h |w_h| eps_h
            float E = ek + 2.0f * gam(H + 24) * (mW + ek);
            const float Is = mI * scale;
            E = (E * scale + 4 * kU2 * (fabsf(Is) + E * scale)) * (1.0f + 16 * kU2) + 1e-30f;
            const uint32_t kL = fkey(Is - E), kU = fkey(Is + E);
            lu[(off + i) * 64 + lane] = make_uint2(kL, kU);
            atomicAdd(&hl[kL >> 22], 1u);
            atomicAdd(&hl[kCoarse + (kU >> 22)], 1u);
        };
        // whole chunk j: each 16-token slot is refilled as soon as it is
        // converted, with chunk j + 1's part, or after the last whole chunk
        // with the wave's remainder part of that slot
        for (int j = 0; j < nj; ++j) {
            const int i = i0 + j * stride;
            const float scale = cscale;
            const bool more = j + 1 < nj;
            const uint8_t* nbase = nullptr;
            if (more) {
                // the index window moves 64 chunks at a time; the chunk in
                // flight already holds its page and scale
                if (((j + 1) & 63) == 0) load_idx(j + 1, nj);
                win_chunk(j + 1, nbase, cscale);
            }
            float mI = 0.0f, mW = 0.0f, mK = 0.0f;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                uint4 ka[KS];
                operands(tb, ka);
                if (more) load_part(nbase, tb);
                else load_rem(tb);
                sums(tb, ka, mI, mW, mK);
            }
            emit(i, scale, mI, mW, mK);
        }
        // the remainder parts: lanes of group lq == tb keep token tb*16 + l16
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int p = rem_part(tb);
            if (p < 0) continue;  // uniform
            const bool second = (p >> 2) != (pr0 >> 2);
            uint4 ka[KS];
            operands(tb, ka);
            float mI = 0.0f, mW = 0.0f, mK = 0.0f;
            sums(tb, ka, mI, mW, mK);
            if (lq == tb) emit(rc0 + (second ? 1 : 0), second ? rs1 : rs0, mI, mW, mK);
        }
    }
    lds_barrier();
    uint32_t* gh = hist + (int64_t)r * kHist;
    for (int i = tid; i < 2 * kCoarse; i += 64 * kWaves)
        if (hl[i]) atomicAdd(&gh[i], hl[i]);
}
// Pages (slots) and index-key scales of the selected chunks, in selection
// order: sel_slot[off + i] for i below the request's count, -1 from there to
// the request's chunk count.  The window pipeline forms them once per window
// so that K1 reaches the key rows with one dependent load instead of two.
__global__ __launch_bounds__(256) void k_resolve_sel(GeomDev g, const int32_t* __restrict__ sel,
                                                     const int32_t* __restrict__ cnt,
                                                     const int32_t* __restrict__ page_table,
                                                     const float* __restrict__ ikey_scale,
                                                     int32_t* __restrict__ sel_slot,
                                                     float* __restrict__ sel_scale) {
    const int r = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
    if (i >= g.nhist[r]) return;
    const int64_t off = g.chunk_off[r];
    int32_t slot = -1;
    float sc = 0.0f;
    if (i < cnt[r]) {
        const int c = sel[off + i];
        slot = page_table ? page_table[off + c] : (int32_t)(off + c);
        sc = ikey_scale ? ikey_scale[off + c] : 1.0f;
    }
    sel_slot[off + i] = slot;
    sel_scale[off + i] = sc;
}

// |key|^2 of every token of the selected chunks, in selection order:
// kn2[(off + i) * 64 + t] for i below the request's count.  Products of the
// (exactly converted) key values are exact in fp32 and the sum has error
// within gamma(D) of the exact one in any order, which is what the refine
// pass's bound allows for its own |key|^2.  One wave per chunk, lane = token.
template <int KDT, int D>
__global__ __launch_bounds__(256) void k_key_norm2(GeomDev g, const int32_t* __restrict__ cnt,
                                                   const int32_t* __restrict__ sel_slot,
                                                   const uint8_t* __restrict__ pages,
                                                   int64_t page_bytes, int64_t ikey_off,
                                                   float* __restrict__ kn2) {
    constexpr int ROWB = D * (KDT == LSA_BF16 ? 2 : 1);
    const int r = blockIdx.y, lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= cnt[r]) return;
    const int64_t off = g.chunk_off[r];
    const uint8_t* row = pages + (int64_t)sel_slot[off + i] * page_bytes + ikey_off + (int64_t)lane * ROWB;
    uint4 v[ROWB / 16];
#pragma unroll
    for (int n = 0; n < ROWB / 16; ++n) v[n] = *(const uint4*)(row + 16 * n);
    float s = 0.0f;
#pragma unroll
    for (int n = 0; n < ROWB / 16; ++n) {
        const uint32_t wd[4] = {v[n].x, v[n].y, v[n].z, v[n].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (KDT == LSA_BF16) {
                const float a = __uint_as_float(wd[e] << 16), b = __uint_as_float(wd[e] & 0xffff0000u);
                s = __builtin_fmaf(a, a, s);
                s = __builtin_fmaf(b, b, s);
            } else {
                const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[e], false);
                const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[e], true);
                s = __builtin_fmaf(lo[0], lo[0], s);
                s = __builtin_fmaf(lo[1], lo[1], s);
                s = __builtin_fmaf(hi[0], hi[0], s);
                s = __builtin_fmaf(hi[1], hi[1], s);
            }
        }
    }
    kn2[(off + i) * 64 + lane] = s;
}

// Chunks [c0, c1) of a request that block x of X takes in K2 and K3.
__device__ __forceinline__ void block_chunks(int nc, int X, int x, int& c0, int& c1) {
    const int C = (nc + X - 1) / X;
    c0 = min(nc, x * C);
    c1 = min(nc, c0 + C);
}

// K2.  Grid (X, B).  Requests with no more than k candidates keep them all
// here.  Otherwise every block finds the coarse bins cL, cU holding the k-th
// largest L and U (block 0 keeps them, with the counts above them, in
// cinfo), then, in one pass over its chunks' keys: adds the fine histograms
// of the keys that fall in those bins, and lists in token order (at
// (off + c0) * 64, count in pcnt[r][x]) the candidates whose U reaches the
// lower edge of bin cL.  No other candidate can be in the band (its
// U < (cL << 22) <= tau).
constexpr int kPre = 8;  // rounds of keys a K2 wave has in flight

__global__ __launch_bounds__(64 * kWaves) void k_band_fine(
    GeomDev g, const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt,
    const uint2* __restrict__ lu, int k, uint32_t* __restrict__ hist, int4* __restrict__ cinfo,
    int32_t* __restrict__ plist, int32_t* __restrict__ pcnt, int32_t* __restrict__ topk,
    int32_t* __restrict__ tcnt, AppendRow app) {
    __shared__ __attribute__((aligned(16))) uint32_t hf[2 * kFine];
    __shared__ int wsum[kWaves], s_out[4], s_np[kPre][kWaves];
    const int r = blockIdx.y, X = gridDim.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // a growing context's new row for the request (block 0): requested now,
    // stored at the end, so that its latency overlaps the block's work
    const bool app_on = app.rows && blockIdx.x == 0 && tid < app.n16;
    uint4 app_v = make_uint4(0u, 0u, 0u, 0u);
    if (app_on) app_v = ((const uint4*)(app.rows + (int64_t)r * app.n16 * 16))[tid];
    auto app_store = [&]() __attribute__((always_inline)) {
        if (app_on) ((uint4*)(app.recent + (g.rec_off[r] + g.nrec[r] - 1) * (int64_t)app.n16 * 16))[tid] = app_v;
    };
    const int nc = cnt[r], n = nc * 64;
    const int64_t off = g.chunk_off[r];
    if (n <= k) {  // every candidate is kept, already in token order
        for (int p = blockIdx.x * blockDim.x + tid; p < n; p += X * blockDim.x)
            topk[(int64_t)r * k + p] = sel[off + (p >> 6)] * 64 + (p & 63);
        if (blockIdx.x == 0 && tid == 0) tcnt[r] = n;
        app_store();
        return;
    }
    int c0, c1;
    block_chunks(nc, X, blockIdx.x, c0, c1);
    // this wave's keys for the first kPre rounds (round j: chunk c0 + 4j + wave)
    uint2 f[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        const int c = c0 + kWaves * u + wv;
        f[u] = c < c1 ? lu[(off + c) * 64 + lane] : make_uint2(0u, 0u);
    }
    uint32_t* gh = hist + (int64_t)r * kHist;
    load_hist<2 * kCoarse, 64 * kWaves>(gh, hf);
    kth_bin<kCoarse, kWaves>(hf, k, wsum, &s_out[0]);
    kth_bin<kCoarse, kWaves>(hf + kCoarse, k, wsum, &s_out[2]);
    const uint32_t cL = (uint32_t)s_out[0], cU = (uint32_t)s_out[2];
    const uint32_t tau_c = cL << 22;
    if (blockIdx.x == 0 && tid == 0) cinfo[r] = make_int4(s_out[0], s_out[1], s_out[2], s_out[3]);
    for (int i = tid; i < 2 * kFine; i += blockDim.x) hf[i] = 0;
    lds_barrier();
    const int64_t seg = (off + c0) * 64;
    const uint64_t lt = (1ull << lane) - 1;
    int np = 0;
    for (int cb0 = c0; cb0 < c1; cb0 += kWaves * kPre) {  // uniform
        // every round's ballot first, then one barrier for all their counts;
        // the list stays in token order (round-major, then wave)
        uint64_t mk[kPre];
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
            const int c = cb0 + kWaves * u + wv;
            const bool have = c < c1;
            const uint2 cur = f[u];
            if (have) {
                if ((cur.x >> 22) == cL) atomicAdd(&hf[(cur.x >> 11) & (kFine - 1)], 1u);
                if ((cur.y >> 22) == cU) atomicAdd(&hf[kFine + ((cur.y >> 11) & (kFine - 1))], 1u);
            }
            mk[u] = __ballot(have && cur.y >= tau_c);
            if (lane == 0) s_np[u][wv] = __popcll(mk[u]);
        }
        lds_barrier();
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
            int pb = np;
#pragma unroll
            for (int w2 = 0; w2 < kWaves; ++w2) {
                const int x = s_np[u][w2];
                pb += w2 < wv ? x : 0;
                np += x;
            }
            if ((mk[u] >> lane) & 1ull)
                plist[seg + pb + __popcll(mk[u] & lt)] = (cb0 + kWaves * u + wv) * 64 + lane;
        }
        lds_barrier();  // s_np is rewritten by the next rounds
        // next kPre rounds
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
            const int c = cb0 + kWaves * (kPre + u) + wv;
            f[u] = c < c1 ? lu[(off + c) * 64 + lane] : make_uint2(0u, 0u);
        }
    }
    if (tid == 0) pcnt[(int64_t)r * X + blockIdx.x] = np;
    lds_barrier();
    uint32_t* gf = gh + 2 * kCoarse;
    for (int i = tid; i < 2 * kFine; i += blockDim.x)
        if (hf[i]) atomicAdd(&gf[i], hf[i]);
    app_store();
}

// K3.  Grid (X, B).  Block x lists, in token order, the band candidates
// among its pre-band list at (off + c0) * 64 (positions p into the request's
// candidates; key 0xffffffff for certain ones) and its count at scnt[r][x];
// its uncertain ones get the canonical score as their key.  For the score each
// token is taken by TPT = min(H, 64) lanes, one or two heads per lane, with
// the lane's query rows held in registers (bf16 pairs); the key row goes
// through LDS as fp32, each head runs its fma chain in element order, then
// one lane runs the head sum in head order.
template <int KDT, int D, int H>
__global__ __launch_bounds__(64 * kWaves) void k_band_list(
    GeomDev g, const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt,
    const uint2* __restrict__ lu, const uint32_t* __restrict__ hist,
    const int4* __restrict__ cinfo, const int32_t* __restrict__ plist,
    const int32_t* __restrict__ pcnt, int k,
    const uint8_t* __restrict__ pages, int64_t page_bytes, int64_t ikey_off,
    const int32_t* __restrict__ page_table, const float* __restrict__ ikey_scale,
    const int32_t* __restrict__ sel_slot, const float* __restrict__ sel_scale,
    const uint16_t* __restrict__ q, const float* __restrict__ w, int32_t* __restrict__ bl,
    uint32_t* __restrict__ bk, int32_t* __restrict__ ul, int32_t* __restrict__ scnt) {
    constexpr int TPT = H < 64 ? H : 64;  // lanes per token
    constexpr int HPT = H / TPT;          // heads per lane
    constexpr int TPW = 64 / TPT;         // tokens per wave
    constexpr int EB = KDT == LSA_BF16 ? 2 : 1;
    constexpr int ROWB = D * EB;
    constexpr int G = 4;                  // tokens a lane scores at once (independent chains)
    constexpr int PPR = ROWB / 16;        // 16-byte pieces per key row
    constexpr int NPT = kRs * PPR / (64 * kWaves);  // row pieces per thread per round
    static_assert(NPT * 64 * kWaves == kRs * PPR, "key rows must split evenly");
    __shared__ __attribute__((aligned(16))) uint8_t krow[kRs][ROWB];  // key rows of a round
    __shared__ uint64_t rrow[kRs];        // their addresses
    __shared__ float rsc[kRs];            // their chunk scales
    __shared__ int rent[kRs];             // their band list slots
    __shared__ float rel[kWaves][TPW][G][H];
    __shared__ float wf[H];
    __shared__ __attribute__((aligned(16))) uint32_t hf[2 * kFine];
    __shared__ int wsum[kWaves], s_out[4];
    __shared__ int64_t pgb[kPgCap];  // page (slot) of chunk c0 + t
    __shared__ float psc[kPgCap];    // its index-key scale
    __shared__ int ucp[kUclCap], ucj[kUclCap];  // uncertain entries: position, list index
    const int r = blockIdx.y, X = gridDim.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nc = cnt[r];
    if (nc * 64 <= k) return;
    const int64_t off = g.chunk_off[r];
    int c0, c1;
    block_chunks(nc, X, blockIdx.x, c0, c1);
    const int nch = c1 - c0;
    const bool pg_lds = nch <= kPgCap;
    // The fine histograms, the coarse bins, the block's pre-band count and
    // the first pre-band entry of each thread load first (read with the
    // count unknown; within the block's list space); the loads that only
    // the re-score needs go out behind them.
    const int64_t seg = (off + c0) * 64;
    const int4 ci = cinfo[r];
    const int npre = pcnt[(int64_t)r * X + blockIdx.x];
    const int p_first = tid < nch * 64 ? plist[seg + tid] : 0;
    load_hist<2 * kFine, 64 * kWaves>(hist + (int64_t)r * kHist + 2 * kCoarse, hf);
    // page and scale of this block's chunks, the weights and the query rows:
    // held in registers until the lists are done, so that no barrier before
    // then waits for them (the pages are two dependent loads without sel_slot)
    int64_t pg_v = 0;
    float sc_v = 1.0f, w_v = 0.0f;
    if (pg_lds && tid < nch) {
        if (sel_slot) {
            pg_v = (int64_t)sel_slot[off + c0 + tid];
            sc_v = sel_scale[off + c0 + tid];
        } else {
            const int c = sel[off + c0 + tid];
            pg_v = page_table ? (int64_t)page_table[off + c] : off + c;
            if constexpr (KDT == LSA_FP8_E4M3FN) sc_v = ikey_scale[off + c];
        }
    }
    static_assert(H <= 64 * kWaves, "one weight per thread");
    if (tid < H) w_v = w[(int64_t)r * H + tid];
    const int lt2 = lane % TPT, ts = lane / TPT;
    uint32_t qp[HPT][D / 2];
#pragma unroll
    for (int j = 0; j < HPT; ++j) {
        const uint4* src = (const uint4*)(q + ((int64_t)r * H + lt2 + TPT * j) * D);
#pragma unroll
        for (int x = 0; x < D / 8; ++x) {
            const uint4 v = src[x];
            qp[j][4 * x] = v.x;
            qp[j][4 * x + 1] = v.y;
            qp[j][4 * x + 2] = v.z;
            qp[j][4 * x + 3] = v.w;
        }
    }
    // tau: lowest key of the fine bin holding the k-th largest L; edge: first
    // key above the fine bin holding the k-th largest U
    kth_bin<kFine, kWaves>(hf, k - ci.y, wsum, &s_out[0]);
    kth_bin<kFine, kWaves>(hf + kFine, k - ci.w, wsum, &s_out[2]);
    const uint32_t tau = ((uint32_t)ci.x << 22) | ((uint32_t)s_out[0] << 11);
    const uint64_t edge = ((uint64_t)(uint32_t)ci.z << 22) + ((uint64_t)(s_out[2] + 1) << 11);
    const uint2* lur = lu + off * 64;
    // ordered lists over the pre-band entries, one per thread per round
    int nb = 0, nu = 0;
    for (int b0 = 0; b0 < npre; b0 += 64 * kWaves) {  // uniform
        const int idx = b0 + tid;
        const bool have = idx < npre;
        const int p = have ? (b0 == 0 ? p_first : plist[seg + idx]) : 0;
        const uint2 cur = have ? lur[p] : make_uint2(0u, 0u);
        const bool band = have && cur.y >= tau;
        const bool sure = band && (uint64_t)cur.x >= edge;
        const bool unc = band && !sure;
        int tb_, tu_;
        const int j = nb + block_scan<kWaves>(band ? 1 : 0, wsum, tb_);
        const int u = nu + block_scan<kWaves>(unc ? 1 : 0, wsum, tu_);
        if (band) {
            bl[seg + j] = p;
            bk[seg + j] = sure ? 0xffffffffu : 0u;
            if (unc) {
                ul[seg + u] = j;
                if (u < kUclCap) {
                    ucp[u] = p;
                    ucj[u] = j;
                }
            }
        }
        nb += tb_;
        nu += tu_;
    }
    if (tid == 0) scnt[(int64_t)r * X + blockIdx.x] = nb;
    if (nu == 0) return;  // uniform
    if (pg_lds && tid < nch) {
        pgb[tid] = pg_v;
        psc[tid] = sc_v;
    }
    if (tid < H) wf[tid] = w_v;
    // canonical scores of this block's uncertain entries, kRs at a time:
    // every entry's key row comes into LDS in one round of loads, then each
    // lane runs the element-order chains of its heads for G tokens at once
    // (independent accumulators), and one lane per token the head sum.
    // The lists in global memory written above are read by other threads
    // below (past the LDS copies): a full block barrier.
    __threadfence_block();
    __syncthreads();
    for (int u0 = 0; u0 < nu; u0 += kRs) {  // uniform
        const int n = min(kRs, nu - u0);
        if (tid < n) {
            const int u = u0 + tid;
            int p, j;
            if (u < kUclCap) {
                p = ucp[u];
                j = ucj[u];
            } else {
                j = ul[seg + u];
                p = bl[seg + j];
            }
            int64_t pg;
            float scale = 1.0f;
            if (pg_lds) {
                pg = pgb[(p >> 6) - c0];
                scale = psc[(p >> 6) - c0];
            } else {
                if (sel_slot) {
                    pg = (int64_t)sel_slot[off + (p >> 6)];
                    scale = sel_scale[off + (p >> 6)];
                } else {
                    const int c = sel[off + (p >> 6)];
                    pg = page_table ? (int64_t)page_table[off + c] : off + c;
                    if constexpr (KDT == LSA_FP8_E4M3FN) scale = ikey_scale[off + c];
                }
            }
            rrow[tid] = (uint64_t)(pages + pg * page_bytes + ikey_off + (int64_t)(p & 63) * ROWB);
            rsc[tid] = scale;
            rent[tid] = (int)(seg + j - off * 64);
        }
        lds_barrier();
        {
            // every thread loads (rows past the round's count repeat row 0)
            typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
            typedef const __attribute__((address_space(1))) u32x4v gu32x4;
            uint4 v[NPT];
#pragma unroll
            for (int m = 0; m < NPT; ++m) {
                const int e = tid + 64 * kWaves * m, x = e / PPR;
                v[m] = __builtin_bit_cast(uint4, *(gu32x4*)(rrow[x < n ? x : 0] + (e % PPR) * 16));
            }
#pragma unroll
            for (int m = 0; m < NPT; ++m) {
                const int e = tid + 64 * kWaves * m, x = e / PPR;
                if (x < n) *(uint4*)&krow[x][(e % PPR) * 16] = v[m];
            }
        }
        lds_barrier();
        for (int x0 = 0; x0 < n; x0 += kWaves * TPW * G) {  // uniform
            // token of group g: x0 + (wv * TPW + ts) + kWaves * TPW * g
            float a[G][HPT];
#pragma unroll
            for (int gg = 0; gg < G; ++gg)
#pragma unroll
                for (int jh = 0; jh < HPT; ++jh) a[gg][jh] = 0.0f;
            int xs[G];
#pragma unroll
            for (int gg = 0; gg < G; ++gg) xs[gg] = min(x0 + wv * TPW + ts + kWaves * TPW * gg, kRs - 1);
#pragma unroll
            for (int i = 0; i < D; i += 4) {
#pragma unroll
                for (int gg = 0; gg < G; ++gg) {
                    float k4[4];
                    if constexpr (KDT == LSA_BF16) {
                        const uint2 bb = *(const uint2*)&krow[xs[gg]][2 * i];
                        k4[0] = __uint_as_float(bb.x << 16);
                        k4[1] = __uint_as_float(bb.x & 0xffff0000u);
                        k4[2] = __uint_as_float(bb.y << 16);
                        k4[3] = __uint_as_float(bb.y & 0xffff0000u);
                    } else {
                        const uint32_t bb = *(const uint32_t*)&krow[xs[gg]][i];
                        const auto lo2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)bb, false);
                        const auto hi2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)bb, true);
                        k4[0] = lo2[0];
                        k4[1] = lo2[1];
                        k4[2] = hi2[0];
                        k4[3] = hi2[1];
                    }
#pragma unroll
                    for (int jh = 0; jh < HPT; ++jh) {
                        const uint32_t q01 = qp[jh][i / 2], q23 = qp[jh][i / 2 + 1];
                        a[gg][jh] = __builtin_fmaf(__uint_as_float(q01 << 16), k4[0], a[gg][jh]);
                        a[gg][jh] = __builtin_fmaf(__uint_as_float(q01 & 0xffff0000u), k4[1], a[gg][jh]);
                        a[gg][jh] = __builtin_fmaf(__uint_as_float(q23 << 16), k4[2], a[gg][jh]);
                        a[gg][jh] = __builtin_fmaf(__uint_as_float(q23 & 0xffff0000u), k4[3], a[gg][jh]);
                    }
                }
            }
#pragma unroll
            for (int gg = 0; gg < G; ++gg)
#pragma unroll
                for (int jh = 0; jh < HPT; ++jh) rel[wv][ts][gg][lt2 + TPT * jh] = a[gg][jh] > 0.0f ? a[gg][jh] : 0.0f;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // head sums, in head order: lane lt2 = g of the slot takes token g
            if (lt2 < G) {
                const int x = x0 + wv * TPW + ts + kWaves * TPW * lt2;
                if (x < n) {
                    float I = 0.0f;
#pragma unroll 8
                    for (int h = 0; h < H; ++h) I = __builtin_fmaf(wf[h], rel[wv][ts][lt2][h], I);
                    if constexpr (KDT == LSA_FP8_E4M3FN) I = I * rsc[x];
                    bk[off * 64 + rent[x]] = fkey(I);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();  // rel is rewritten by the next tokens
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        lds_barrier();  // krow and the entry arrays are rewritten by the next round
    }
}

// K4.  Exact top-k over the band of one request (one block); also clears
// the request's histograms.  The block lists of K3 are gathered in order
// into LDS (up to kListCap entries).  Usually few entries are uncertain:
// each is ranked against the others by (score desc, token asc) and the best
// k - #certain join the certain ones, emitted in token order.  Otherwise (only
// with massive ties) the k-th largest key is found by 12/12/8-bit radix
// select and the emit keeps keys above it and the lowest-index ties, reading
// global memory when the band does not fit in LDS.
__global__ __launch_bounds__(kT) void k_topk_band(GeomDev g, const int32_t* __restrict__ sel,
                                                  const int32_t* __restrict__ cnt,
                                                  const int32_t* __restrict__ scnt, int X,
                                                  const int32_t* __restrict__ bl,
                                                  const uint32_t* __restrict__ bk, int k,
                                                  int32_t* __restrict__ topk,
                                                  int32_t* __restrict__ tcnt,
                                                  uint32_t* __restrict__ bhist) {
    __shared__ uint32_t hist[4096];
    __shared__ uint32_t lkey[kListCap];
    __shared__ int32_t lpos[kListCap];
    __shared__ __attribute__((aligned(16))) uint64_t uval[kUncCap];  // (key, ~position): larger ranks first
    __shared__ int32_t uj[kUncCap];
    __shared__ int boff[kMaxSeg + 1];
    __shared__ int32_t ssel[kSelCap];  // the request's selected chunk ids
    __shared__ int wsum[kTW];
    __shared__ uint32_t s_prefix;
    __shared__ int s_remaining, s_eq, s_u;
    const int r = blockIdx.x, tid = threadIdx.x;
    const int64_t off = g.chunk_off[r];
    // the count, the K3 block counts and the selected chunk ids (all the
    // request's chunk slots, before the count is known) load at once
    const int nc = cnt[r];
    const int v_scnt = tid < X ? scnt[(int64_t)r * X + tid] : 0;
    const int nsl = min(g.nhist[r], kSelCap);
    for (int i = tid; i < nsl; i += kT) ssel[i] = sel[g.chunk_off[r] + i];
    // the request's histograms were last read by the previous kernel: clear
    // them for the next launch
    for (int i = tid; i < kHist; i += kT) bhist[(int64_t)r * kHist + i] = 0;
    if (nc * 64 <= k) return;  // k_band_fine already wrote the result
    const int C = (nc + X - 1) / X;  // chunks per K3 block
    int tot;
    {
        const int v = v_scnt;
        const int ex = block_scan<kTW>(v, wsum, tot);
        if (tid < X) boff[tid] = ex;
        if (tid == 0) boff[X] = tot;
    }
    lds_barrier();
    const int m = boff[X];
    const bool in_lds = m <= kListCap;
    auto gidx = [&](int j) -> int64_t {  // list position j -> workspace index
        int lo = 0, hi = X - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (boff[mid] <= j) lo = mid;
            else hi = mid - 1;
        }
        return (off + (int64_t)lo * C) * 64 + (j - boff[lo]);
    };
    auto at = [&](int j, uint32_t& key, int32_t& pos) {
        if (in_lds) {
            key = lkey[j];
            pos = lpos[j];
            return;
        }
        const int64_t e = gidx(j);
        key = bk[e];
        pos = bl[e];
    };
    const int32_t* sl = sel + off;
    auto sel_of = [&](int i) -> int32_t { return i < kSelCap ? ssel[i] : sl[i]; };
    int32_t* out = topk + (int64_t)r * k;
    if (in_lds) {
        if (tid == 0) s_u = 0;
        // every entry's loads in flight before any is stored (kGB per thread)
        constexpr int kGB = 8;
        for (int j0 = 0; j0 < m; j0 += kT * kGB) {
            uint32_t kk[kGB];
            int32_t pp[kGB];
#pragma unroll
            for (int u = 0; u < kGB; ++u) {
                const int j = j0 + tid + kT * u;
                if (j < m) {
                    const int64_t e = gidx(j);
                    kk[u] = bk[e];
                    pp[u] = bl[e];
                }
            }
#pragma unroll
            for (int u = 0; u < kGB; ++u) {
                const int j = j0 + tid + kT * u;
                if (j < m) {
                    lkey[j] = kk[u];
                    lpos[j] = pp[u];
                }
            }
        }
        lds_barrier();
        // The certain entries (key 0xffffffff) are all in; the uncertain ones
        // (few) are ranked against each other by (score desc, token asc) and
        // the best k - #certain are taken.
        const int lane = tid & 63;
        const uint64_t lt = (1ull << lane) - 1;
        for (int j0 = 0; j0 < m; j0 += kT) {  // uniform trip count
            const int j = j0 + tid;
            const bool unc = j < m && lkey[j] != 0xffffffffu;
            const uint64_t mk = __ballot(unc);
            int base = 0;
            if (lane == 0 && mk) base = atomicAdd(&s_u, __popcll(mk));
            base = __shfl(base, 0);
            const int t = base + __popcll(mk & lt);
            if (unc && t < kUncCap) {
                uval[t] = ((uint64_t)lkey[j] << 32) | (uint32_t)~(uint32_t)lpos[j];
                uj[t] = j;
            }
        }
        lds_barrier();
        const int u = s_u;
        if (u <= kUncCap) {
            const int need = k - (m - u);
            if (u & 1) {  // pad to an even count with an entry below every other
                if (tid == 0) uval[u] = 0ull;
                lds_barrier();
            }
            const int u2 = (u + 1) & ~1;
            // kRP neighbouring lanes rank one entry, each over every kRP-th pair
            constexpr int kRP = 4;
            for (int t0 = 0; t0 < u; t0 += kT / kRP) {  // uniform trip count
                const int t = t0 + tid / kRP, q = tid % kRP;
                int rank = 0;
                if (t < u) {
                    const uint64_t vt = uval[t];
#pragma unroll 4
                    for (int s2 = 2 * q; s2 < u2; s2 += 2 * kRP) {
                        const ulonglong2 v2 = *(const ulonglong2*)&uval[s2];
                        rank += (v2.x > vt) + (v2.y > vt);
                    }
                }
                rank += __shfl_xor(rank, 1);
                rank += __shfl_xor(rank, 2);
                if (t < u && q == 0) lkey[uj[t]] = rank < need ? 0xffffffffu : 0u;
            }
            lds_barrier();
            // emit the taken entries in list (token) order: thread t takes a
            // contiguous run of the list
            const int per = (m + kT - 1) / kT;
            const int j0 = min(m, tid * per), j1 = min(m, j0 + per);
            int tc = 0;
            for (int j = j0; j < j1; ++j) tc += lkey[j] == 0xffffffffu;
            int o = block_scan<kTW>(tc, wsum, tot);
            for (int j = j0; j < j1; ++j)
                if (lkey[j] == 0xffffffffu) out[o++] = sel_of(lpos[j] >> 6) * 64 + (lpos[j] & 63);
            if (tid == 0) tcnt[r] = tot;
            return;
        }
    }
    uint32_t prefix = 0, mask = 0;
    int remaining = k;
    const int shifts[3] = {20, 8, 0}, widths[3] = {12, 12, 8};
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = shifts[pass], nb = 1 << widths[pass];
        for (int i = tid; i < nb; i += kT) hist[i] = 0;
        lds_barrier();
        for (int j = tid; j < m; j += kT) {
            uint32_t key;
            int32_t pos;
            at(j, key, pos);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
        }
        lds_barrier();
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
        lds_barrier();
        prefix = s_prefix;
        remaining = s_remaining;
        mask |= (uint32_t)(nb - 1) << shift;
    }
    const uint32_t K = prefix;
    const int need = remaining;
    const bool all_ties = (s_eq == need);
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
            if (take[j]) out[o++] = sel_of(pos[j] >> 6) * 64 + (pos[j] & 63);
        base += tot;
    }
    if (tid == 0) tcnt[r] = base;
}

__global__ void k_zero_u32(uint32_t* __restrict__ p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

}  // namespace

bool band_supported(lsa_dtype idx_dt, lsa_dtype q_dt, int H, int d) {
    return (idx_dt == LSA_BF16 || idx_dt == LSA_FP8_E4M3FN) && q_dt == LSA_BF16 &&
           (d == 64 || d == 128) && (H == 16 || H == 32 || H == 64 || H == 128);
}

static int max_hist(const GeomDev& g) {
    int mx = 0;
    for (int r = 0; r < g.B; ++r) mx = g.nhist[r] > mx ? g.nhist[r] : mx;
    return mx;
}

// K1 blocks per request: about two blocks per CU over the whole batch, no
// more than the longest history needs.
static int k1_blocks(const GeomDev& g) {
    const int forced = tune_get(LSA_TUNE_REFINE_BLOCKS);
    if (forced >= 1) return forced;
    int x = (512 + g.B - 1) / g.B;
    const int need = (max_hist(g) + kWaves - 1) / kWaves;
    if (x > need) x = need;
    return x < 1 ? 1 : x;
}

// K2 / K3 blocks per request: about one per CU over the batch, at least one
// chunk each, no more than K4 gathers.
static int k23_blocks(const GeomDev& g) {
    int x = (256 + g.B - 1) / g.B;
    const int mh = max_hist(g);
    if (x > mh) x = mh;
    if (x > kMaxSeg) x = kMaxSeg;
    return x < 1 ? 1 : x;
}

// Workspace: the histograms first (zero on entry unless the caller knows
// they are; every launch leaves them zero), then the rest.
static size_t clean_words(const GeomDev& g) { return (size_t)g.B * kHist; }

size_t band_ws_bytes(const GeomDev& g) {
    const size_t nc = (size_t)g.chunk_off[g.B] * 64 + 64;
    return align_up(clean_words(g) * 4, 256) + align_up((size_t)g.B * sizeof(int4), 256) +
           align_up(nc * sizeof(uint2), 256) + 4 * align_up(nc * 4, 256) +
           2 * align_up((size_t)g.B * k23_blocks(g) * 4, 256);
}

hipError_t launch_band_clear(const GeomDev& g, void* ws, hipStream_t s) {
    const int n = (int)clean_words(g);
    hipLaunchKernelGGL(k_zero_u32, dim3((n + 255) / 256), dim3(256), 0, s, (uint32_t*)ws, n);
    return hipGetLastError();
}

hipError_t launch_refine_band(const GeomDev& g, const int32_t* sel, const int32_t* cnt,
                              const void* pages, int64_t page_bytes, int64_t ikey_off,
                              const int32_t* page_table, lsa_dtype idx_dt,
                              const float* ikey_scale, const int32_t* sel_slot,
                              const float* sel_scale, const float* kn2, const void* q,
                              const float* w, int H, int d, int k, int32_t* topk, int32_t* tcnt,
                              void* ws, bool ws_clean, hipStream_t s, const AppendRow& app) {
    const size_t nc = (size_t)g.chunk_off[g.B] * 64 + 64;
    const int X1 = k1_blocks(g), X2 = k23_blocks(g);
    hipError_t e;
    if (!ws_clean && (e = launch_band_clear(g, ws, s)) != hipSuccess) return e;
    uint8_t* b = (uint8_t*)ws;
    uint32_t* hist = (uint32_t*)b;
    b += align_up(clean_words(g) * 4, 256);
    int4* cinfo = (int4*)b;
    b += align_up((size_t)g.B * sizeof(int4), 256);
    uint2* lu = (uint2*)b;
    b += align_up(nc * sizeof(uint2), 256);
    int32_t* bl = (int32_t*)b;
    b += align_up(nc * 4, 256);
    uint32_t* bk = (uint32_t*)b;
    b += align_up(nc * 4, 256);
    int32_t* ul = (int32_t*)b;
    b += align_up(nc * 4, 256);
    int32_t* plist = (int32_t*)b;
    b += align_up(nc * 4, 256);
    int32_t* scnt = (int32_t*)b;
    b += align_up((size_t)g.B * X2 * 4, 256);
    int32_t* pcnt = (int32_t*)b;
    const uint8_t* pg = (const uint8_t*)pages;
    const uint16_t* qq = (const uint16_t*)q;
    const int Hh = H;
    e = hipErrorInvalidValue;
    timing_begin("k_refine_mfma", s);
#define LSA_K1(KDT, D, HH)                                                                        \
    if (idx_dt == KDT && d == D && Hh == HH) {                                                    \
        hipLaunchKernelGGL((k_refine_mfma<KDT, D, HH>), dim3(X1, g.B), dim3(64 * kWaves), 0, s, g, \
                           sel, cnt, pg, page_bytes, ikey_off, page_table, ikey_scale, sel_slot,  \
                           sel_scale, kn2, qq, w, lu, hist);                                      \
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
    timing_begin("k_band_fine", s);
    hipLaunchKernelGGL(k_band_fine, dim3(X2, g.B), dim3(64 * kWaves), 0, s, g, sel, cnt, lu, k,
                       hist, cinfo, plist, pcnt, topk, tcnt, app);
    timing_end("k_band_fine", s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = hipErrorInvalidValue;
    timing_begin("k_band_list", s);
#define LSA_K3(KDT, D, HH)                                                                        \
    if (idx_dt == KDT && d == D && Hh == HH) {                                                    \
        hipLaunchKernelGGL((k_band_list<KDT, D, HH>), dim3(X2, g.B), dim3(64 * kWaves), 0, s, g,   \
                           sel, cnt, lu, hist, cinfo, plist, pcnt, k, pg, page_bytes, ikey_off,   \
                           page_table, ikey_scale, sel_slot, sel_scale, qq, w, bl, bk, ul, scnt); \
        e = hipGetLastError();                                                                    \
    }
    LSA_K3(LSA_BF16, 128, 16) LSA_K3(LSA_BF16, 128, 32) LSA_K3(LSA_BF16, 128, 64)
    LSA_K3(LSA_BF16, 128, 128) LSA_K3(LSA_BF16, 64, 16) LSA_K3(LSA_BF16, 64, 32)
    LSA_K3(LSA_BF16, 64, 64) LSA_K3(LSA_BF16, 64, 128)
    LSA_K3(LSA_FP8_E4M3FN, 128, 16) LSA_K3(LSA_FP8_E4M3FN, 128, 32) LSA_K3(LSA_FP8_E4M3FN, 128, 64)
    LSA_K3(LSA_FP8_E4M3FN, 128, 128) LSA_K3(LSA_FP8_E4M3FN, 64, 16) LSA_K3(LSA_FP8_E4M3FN, 64, 32)
    LSA_K3(LSA_FP8_E4M3FN, 64, 64) LSA_K3(LSA_FP8_E4M3FN, 64, 128)
#undef LSA_K3
    timing_end("k_band_list", s);
    if (e != hipSuccess) return e;
    timing_begin("k_topk_band", s);
    hipLaunchKernelGGL(k_topk_band, dim3(g.B), dim3(kT), 0, s, g, sel, cnt, scnt, X2, bl, bk, k,
                       topk, tcnt, hist);
    timing_end("k_topk_band", s);
    return hipGetLastError();
}

hipError_t launch_resolve_sel(const GeomDev& g, const int32_t* sel, const int32_t* cnt,
                              const int32_t* page_table, const float* ikey_scale,
                              int32_t* sel_slot, float* sel_scale, hipStream_t s) {
    const int mh = max_hist(g);
    if (mh == 0) return hipSuccess;
    timing_begin("k_resolve_sel", s);
    hipLaunchKernelGGL(k_resolve_sel, dim3((mh + 255) / 256, g.B), dim3(256), 0, s, g, sel, cnt,
                       page_table, ikey_scale, sel_slot, sel_scale);
    timing_end("k_resolve_sel", s);
    return hipGetLastError();
}

hipError_t launch_key_norm2(const GeomDev& g, const int32_t* cnt, const int32_t* sel_slot,
                            const void* pages, int64_t page_bytes, int64_t ikey_off,
                            lsa_dtype idx_dt, int d, float* kn2, hipStream_t s) {
    const int mh = max_hist(g);
    if (mh == 0) return hipSuccess;
    const dim3 grid((mh + 3) / 4, g.B);
    const uint8_t* pg = (const uint8_t*)pages;
    if ((idx_dt != LSA_BF16 && idx_dt != LSA_FP8_E4M3FN) || (d != 64 && d != 128))
        return hipErrorInvalidValue;
    timing_begin("k_key_norm2", s);
    if (idx_dt == LSA_BF16 && d == 128)
        hipLaunchKernelGGL((k_key_norm2<LSA_BF16, 128>), grid, dim3(256), 0, s, g, cnt, sel_slot, pg,
                           page_bytes, ikey_off, kn2);
    else if (idx_dt == LSA_BF16 && d == 64)
        hipLaunchKernelGGL((k_key_norm2<LSA_BF16, 64>), grid, dim3(256), 0, s, g, cnt, sel_slot, pg,
                           page_bytes, ikey_off, kn2);
    else if (idx_dt == LSA_FP8_E4M3FN && d == 128)
        hipLaunchKernelGGL((k_key_norm2<LSA_FP8_E4M3FN, 128>), grid, dim3(256), 0, s, g, cnt, sel_slot, pg,
                           page_bytes, ikey_off, kn2);
    else
        hipLaunchKernelGGL((k_key_norm2<LSA_FP8_E4M3FN, 64>), grid, dim3(256), 0, s, g, cnt, sel_slot, pg,
                           page_bytes, ikey_off, kn2);
    timing_end("k_key_norm2", s);
    return hipGetLastError();
}
