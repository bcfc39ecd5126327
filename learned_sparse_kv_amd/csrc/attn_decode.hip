// Sparse decode attention over the top-k tokens plus the recent window (gfx950).
//
// Core attention runs on the tokens the staged selection keeps (gist.science
// summary, section 2.1 "Gestufte Selektion") together with the most recent
// window, which always stays on the GPU (cjcn.com.cn explainer, section 二
// last paragraph; section 五: every scheme keeps the recent 8K).  All query
// heads share one KV row per token (MQA); the latent row holds 576 values and
// the value is its first 512.
//
// Positions of request r (bf16 latent kernel): the R_r recent tokens first,
// then the filled top-k slots, so empty slots are never visited.  Positions
// are cut into splits; each split keeps a reference max m, sum l and
// unnormalised output (online softmax, base 2) and writes them to a
// workspace; k_attn_merge combines the splits of each (request, head).
//
// k_attn_mla (bf16, Dk 576 / Dv 512): one block per (request, split, group
// of 64 or 32 heads), 32-token tiles, MFMA 16x16x32 bf16; every KV byte is
// read from HBM once per head group and feeds both products.
// Algorithmic bytes per attended token: 1,152 (HBM-bound).
//
// k_attn_f32: fp32 rows, VALU, for small head counts (fp32 path).
#include "lsa_internal.h"

#include <atomic>
#include <mutex>
#include <type_traits>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;

struct PosMap {
    const uint8_t* pages;
    int64_t page_bytes, row_bytes;
    const int32_t* pt;
    const uint8_t* recent;
    const int32_t* topk;
    int k;
};

// Row address of position p of request r, or nullptr for an empty slot.
__device__ __forceinline__ const uint8_t* pos_row(const GeomDev& g, const PosMap& m, int r,
                                                  int kcnt, int p) {
    if (p < m.k) {
        if (p >= kcnt) return nullptr;
        const int s = m.topk[(int64_t)r * m.k + p];
        const int64_t c = g.chunk_off[r] + (s >> 6);
        const int64_t slot = m.pt ? (int64_t)m.pt[c] : c;
        return m.pages + slot * m.page_bytes + (int64_t)(s & 63) * m.row_bytes;
    }
    const int qi = p - m.k;
    if (qi < g.nrec[r]) return m.recent + (g.rec_off[r] + qi) * m.row_bytes;
    return nullptr;
}

__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ----------------------------------------------------------------------------
// bf16 latent MQA (Dk 576, Dv 512), MFMA 16x16x32 bf16.
//
// A block takes one (request, split, head group) with NW waves; the wave
// pair (2 hq, 2 hq + 1) owns 32 heads.  In the pair, wave vh = 0 takes the
// first half of the 576 key dimensions and value dimensions 0..255, wave
// vh = 1 the second half and values 256..511.  Per 32-token tile:
//   S^T = K Q^T  partial over the wave's 9 k-steps (A = key rows from LDS,
//                B = the wave's query slice, held in registers all along);
//   the two partials are swapped through LDS and added in a fixed order, so
//   both waves hold the same S^T and run the same softmax;
//   O^T += V^T P^T for the wave's 256 value dims (A = V^T from LDS transpose
//                reads, B = P^T straight from the softmax registers).
// The output and the softmax state stay in registers; only the partial S
// goes through LDS.  The running reference m of a head is raised only when
// a tile's max exceeds it by more than 8 (log2 units): the probabilities
// exp2(s - m) then stay below 256 and the rescale of O^T is rare.  Since O
// and l share the reference, the result is the same softmax.
//
// KV tiles: 32 rows land in LDS by direct global->LDS loads (16 bytes per
// lane), three tiles deep; the loads of tile t + 2 are spread over the score
// products of tile t.  The tile is kept in the operand layout of the
// matrix core: block (token half tb, k-step ks) holds 64 slots of 16 bytes,
// slot lq*16 + t = key row 16 tb + t, dims 32 ks + 8 lq .. +8, so the S
// operand read of a wave is one contiguous 1 KB.  ds_read_b64_tr_b16 turns
// 4 rows x 4 dims per lane group into the V^T operand.
//
// Positions of request r are [recent window (nrec) | top-k (kcnt)]: the
// recent tokens first, then the filled top-k slots; splits cut this list.
// The tail of the last tile repeats its last row and is masked to -inf.
// ----------------------------------------------------------------------------
constexpr int MT = 32;                        // tokens per tile
constexpr int MDK = 576, MDV = 512;
constexpr int kKSteps = MDK / 32;             // 18
constexpr int kBlk = 1024;                    // bytes per (tb, ks) operand block
constexpr int kTileB = 2 * kKSteps * kBlk;    // 36,864
constexpr int kNBuf = 3;                      // tiles in LDS
constexpr int kMaxSplitPos = 1024;
constexpr float kRescaleSlack = 8.0f;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint2 lds_tr16(const uint8_t* base_lds, int byte_off) {
    const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16_t*)((__attribute__((address_space(3))) uint8_t*)base_lds +
                                                      byte_off));
    return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from gptr to LDS (M0 + 16 * lane).  Written as asm so
// that the compiler does not wait for these loads before every LDS read;
// the kernel waits for them itself (vmcnt) before the tile barrier.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_off) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "{m0}"(__builtin_amdgcn_readfirstlane(lds_off))
                 : "memory");
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }  // lgkmcnt(0)

// reductions over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane rows)
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const __bf16 x = (__bf16)a, y = (__bf16)b;  // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// NW waves per block, HPW blocks of 16 heads per wave; the block covers
// 16 * HPW * NW / 2 heads.
template <int NW, int HPW>
__global__ __launch_bounds__(64 * NW, 1) void k_attn_mla(GeomDev g, PosMap pm,
                                                        const int32_t* __restrict__ tcnt,
                                                        const uint16_t* __restrict__ q, int Hq,
                                                        int n_splits, int per_split, int hgroups,
                                                        float sm_log2e, uint16_t* __restrict__ part_o,
                                                        float* __restrict__ part_ml, int polls,
                                                        uint32_t* __restrict__ err) {
    constexpr int NB = 2 * kKSteps;                   // operand blocks per tile (36)
    constexpr int NLmax = (NB + NW - 1) / NW;         // tile loads per wave (the first NB % NW waves)
    __shared__ __attribute__((aligned(1024))) uint8_t tiles[kNBuf][kTileB];
    __shared__ __attribute__((aligned(16))) float sx[NW][64 * 8 * HPW];
    __shared__ uint64_t rowp[kMaxSplitPos];
    __shared__ int pflag[NW];  // tiles whose partial scores wave w has published

    const int bi = blockIdx.x;
    const int xcd = bi & 7, jb = bi >> 3;
    const int hg = jb % hgroups;
    const int unit = (jb / hgroups) * 8 + xcd;
    if (unit >= g.B * n_splits) return;
    const int r = unit / n_splits, split = unit % n_splits;
    const int tid = threadIdx.x, w = tid >> 6, L = tid & 63, l16 = L & 15, lq = L >> 4;
    const int vh = w & 1;
    const int h0 = hg * (8 * HPW * NW) + 16 * HPW * (w >> 1);  // first head of the pair
    const int nl = (NB % NW == 0 || w < NB % NW) ? NLmax : NLmax - 1;  // this wave's tile loads

    // query slices (B operands): head h0 + 16 hb + l16, k-steps 9 vh .. 9 vh + 8
    u32x4_t Qb[HPW][9];
    {
        const uint16_t* qr = q + ((int64_t)r * Hq + h0) * MDK + (9 * vh) * 32 + lq * 8;
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb)
#pragma unroll
            for (int j = 0; j < 9; ++j) Qb[hb][j] = *(const u32x4_t*)(qr + (hb * 16 + l16) * MDK + j * 32);
    }
    const int nrec = g.nrec[r];
    const int p_begin = split * per_split;
    // A split inside the recent window needs neither the top-k count nor the
    // list.  The others request the count and their share of the list (up to
    // k entries, before the count is known) at once, then the page of each
    // valid entry.
    const bool rec_only = p_begin + per_split <= nrec;  // uniform
    constexpr int kPT = kMaxSplitPos / (64 * NW);      // positions per thread, at most
    int sl[kPT];
    int tc = 0;
#pragma unroll
    for (int u = 0; u < kPT; ++u) sl[u] = 0;
    if (!rec_only) {
        const int32_t* tk = pm.topk + (int64_t)r * pm.k;
        tc = tcnt[r];
#pragma unroll
        for (int u = 0; u < kPT; ++u) {
            const int i = tid + 64 * NW * u, p = p_begin + i;
            if (i < per_split && p >= nrec && p < nrec + pm.k) sl[u] = tk[p - nrec];
        }
    }
    const int kcnt = min(max(tc, 0), pm.k);
    const int npos = rec_only ? per_split : max(0, min(per_split, nrec + kcnt - p_begin));
    const int ntiles = (npos + MT - 1) / MT;
    // row address of every valid position of the split (the loads of the
    // last tile's tail repeat position npos - 1)
    {
        const uint8_t* rec0 = pm.recent + g.rec_off[r] * pm.row_bytes;
        const int64_t coff = g.chunk_off[r];
#pragma unroll
        for (int u = 0; u < kPT; ++u) {
            const int i = tid + 64 * NW * u, p = p_begin + i;
            if (i < npos) {
                const uint8_t* row;
                if (p < nrec) {
                    row = rec0 + (int64_t)p * pm.row_bytes;
                } else {
                    const int64_t c = coff + (sl[u] >> 6);
                    const int64_t slot = pm.pt ? (int64_t)pm.pt[c] : c;
                    row = pm.pages + slot * pm.page_bytes + (int64_t)(sl[u] & 63) * pm.row_bytes;
                }
                rowp[i] = (uint64_t)row;
            }
        }
    }
    if (L == 0) pflag[w] = 0;
    // every load of the compiler's own is done before the tile loads start,
    // so that the vmcnt waits in the loop count tile loads only (the uses of
    // the query slices make the compiler wait for them here, not in the loop)
#pragma unroll
    for (int hb = 0; hb < HPW; ++hb)
#pragma unroll
        for (int j = 0; j < 9; ++j) asm volatile("" : : "v"(Qb[hb][j]));
    wait_vm<0>();
    wait_lds();
    __builtin_amdgcn_s_barrier();

    // wave w loads blocks w, w + NW, ... of a tile: slot L of block (tb, ks) is
    // key row 16 tb + (l16 ^ 8 (lq & 1)), bytes 64 ks + 16 lq .. +16.  The
    // XOR puts the two 8-dim groups a transposed V read takes together (256 B
    // apart, the same banks) on different halves of the banks.
    const int l16x = l16 ^ ((lq & 1) << 3);
    // the two row addresses a lane loads from for tile t (read from LDS one
    // tile ahead of their use, so the loads issue without waiting on LDS)
    auto tile_rows = [&](int t, uint64_t& a0, uint64_t& a1) __attribute__((always_inline)) {
        a0 = rowp[min(t * MT + l16x, npos - 1)];
        a1 = rowp[min(t * MT + 16 + l16x, npos - 1)];
    };
    auto load_tile = [&](uint64_t a0, uint64_t a1, int buf) __attribute__((always_inline)) {
        const uint8_t* ra0 = (const uint8_t*)a0;
        const uint8_t* ra1 = (const uint8_t*)a1;
        const uint32_t dst = lds_u32(tiles[buf]);
#pragma unroll
        for (int m = 0; m < NLmax; ++m) {
            const int b = w + NW * m;
            if (b < NB) {
                const int tb = b >= kKSteps ? 1 : 0, ks = b - kKSteps * tb;
                lds_dma16((tb ? ra1 : ra0) + ks * 64 + lq * 16, dst + b * kBlk);
            }
        }
    };
    // the wave's m-th block of a tile (the loop spreads these over its k-steps)
    auto load_block = [&](uint64_t a0, uint64_t a1, int buf, int m) __attribute__((always_inline)) {
        const int b = w + NW * m;
        if (b < NB) {
            const int tb = b >= kKSteps ? 1 : 0, ks = b - kKSteps * tb;
            lds_dma16((const uint8_t*)(tb ? a1 : a0) + ks * 64 + lq * 16, lds_u32(tiles[buf]) + b * kBlk);
        }
    };
    uint64_t na0 = 0, na1 = 0;  // row addresses of the next tile to load
    if (ntiles > 0) {
        tile_rows(0, na0, na1);
        load_tile(na0, na1, 0);
    }
    if (ntiles > 1) {
        tile_rows(1, na0, na1);
        load_tile(na0, na1, 1);
    }
    if (ntiles > 2) tile_rows(2, na0, na1);

    f32x4_t acc[HPW][16];
#pragma unroll
    for (int hb = 0; hb < HPW; ++hb)
#pragma unroll
        for (int vb = 0; vb < 16; ++vb) acc[hb][vb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_ref[HPW], l_lane[HPW];
#pragma unroll
    for (int hb = 0; hb < HPW; ++hb) {
        m_ref[hb] = -INFINITY;
        l_lane[hb] = 0.0f;
    }

    // V^T operand read offsets inside a tile (token half 0; half 1 is + 18 KB)
    // lane (n = l16, lq) points at row 4 lq + n / 4, dims 16 vbg + 4 (n % 4)
    const int tr_lqp_lo = (l16 & 3) >> 1, tr_sub = 8 * (l16 & 1);
    const int tr_slot_row = (4 * lq + (l16 >> 2)) ^ (tr_lqp_lo << 3);  // swizzled slot of the row

    float s[HPW][8], mx[HPW];  // s[hb][tb * 4 + i]: token 16 tb + 4 lq + i of head h0 + 16 hb + l16
    // scores of tile `it` (pair sum, scaled, masked) and their per-head max
    auto score_tile = [&](int it) __attribute__((always_inline)) {
        if (it + 1 < ntiles) {  // the loads of tile it + 1 may still be in flight
            if (nl == NLmax)
                wait_vm<NLmax>();
            else
                wait_vm<NLmax - 1>();
        } else {
            wait_vm<0>();
        }
        __builtin_amdgcn_s_barrier();  // tile `it` in LDS; tile it - 1 released
        // tile it + 2 goes into the buffer tile it - 1 released at the barrier;
        // its loads issue one per k-step below: issued together right after
        // the barrier, every wave's loads queue at once and hold the waves up
        const bool more = it + 2 < ntiles;  // uniform
        const int nbuf = (it + 2) % kNBuf;
        const uint8_t* tile = tiles[it % kNBuf];
        f32x4_t c[2][HPW];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int hb = 0; hb < HPW; ++hb) c[tb][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 9; ++j)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const uint4 a = *(const uint4*)(tile + (tb * kKSteps + 9 * vh + j) * kBlk + (l16x + 16 * lq) * 16);
#pragma unroll
                for (int hb = 0; hb < HPW; ++hb)
                    c[tb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(Qb[hb][j]),
                                                                        c[tb][hb], 0, 0, 0);
                if (tb == 1 && j < NLmax && more) load_block(na0, na1, nbuf, j);
            }
        if (more && it + 3 < ntiles) tile_rows(it + 3, na0, na1);
        // swap the partials with the other wave of the pair; both waves add
        // first-half + second-half, so they hold the same S^T
        {
            float4* mine = (float4*)sx[w];  // [tb * HPW + hb][lane]: lane-contiguous, no bank conflicts
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int hb = 0; hb < HPW; ++hb)
                    mine[(tb * HPW + hb) * 64 + L] = make_float4(c[tb][hb][0], c[tb][hb][1], c[tb][hb][2], c[tb][hb][3]);
        }
        // publish them (the release orders the data writes before the flag)
        // and wait for the partner's: only the pair meets here, not the
        // block.  The partner runs the same tile loop, so it always
        // publishes; the wait is still bounded (polls), and one that runs
        // out is recorded in the device's error word, so the output it
        // spoils is reported instead of returned silently.
        __hip_atomic_store(&pflag[w], it + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        {
            int seen = -1;
            for (int spin = 0; spin < polls; ++spin) {
                seen = __builtin_amdgcn_readfirstlane(
                    __hip_atomic_load(&pflag[w ^ 1], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
                if (seen > it) break;
                __builtin_amdgcn_s_sleep(1);
            }
            if (seen <= it && L == 0 && err)
                __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const float4* other = (const float4*)sx[w ^ 1];
        const int t0 = it * MT;
        // the sum of two terms is the same in either order, so both waves of
        // the pair get the same scores; only a last, partial tile is masked
        const bool partial = t0 + MT > npos;  // uniform
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const float4 o = other[(tb * HPW + hb) * 64 + L];
                const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) s[hb][tb * 4 + i] = (c[tb][hb][i] + ov[i]) * sm_log2e;
            }
            if (partial) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (t0 + 16 * (e >> 2) + 4 * lq + (e & 3) >= npos) s[hb][e] = -INFINITY;
            }
            float m = s[hb][0];
#pragma unroll
            for (int e = 1; e < 8; ++e) m = fmaxf(m, s[hb][e]);
            mx[hb] = max_xor32(max_xor16(m));
        }
    };
    // probabilities against the reference, row sums, O^T += V^T P^T over this
    // wave's 256 value dims
    auto accumulate = [&](int it) __attribute__((always_inline)) {
        const uint8_t* tile = tiles[it % kNBuf];
        uint4 pb[HPW];
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(s[hb][e] - m_ref[hb]);
            pb[hb] = make_uint4(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                                pack_bf16(p[6], p[7]));
            // the sum uses the rounded weights the products use
            float ls = 0.0f;
            ls += bf16_lo(pb[hb].x) + bf16_hi(pb[hb].x);
            ls += bf16_lo(pb[hb].y) + bf16_hi(pb[hb].y);
            ls += bf16_lo(pb[hb].z) + bf16_hi(pb[hb].z);
            ls += bf16_lo(pb[hb].w) + bf16_hi(pb[hb].w);
            l_lane[hb] += ls;
        }
#pragma unroll
        for (int vb = 0; vb < 16; ++vb) {
            const int vbg = 16 * vh + vb;
            const int off = (vbg >> 1) * kBlk + ((2 * (vbg & 1) + tr_lqp_lo) * 16 + tr_slot_row) * 16 + tr_sub;
            const uint2 lo = lds_tr16(tile, off);
            const uint2 hi = lds_tr16(tile, off + kKSteps * kBlk);
            const bf16x8_t va = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
            for (int hb = 0; hb < HPW; ++hb)
                acc[hb][vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, as_bf16x8(pb[hb]), acc[hb][vb], 0, 0, 0);
        }
    };

    // The inner loop runs while no head's tile max exceeds its reference by
    // more than the slack; such a tile (always the first) leaves it, the
    // reference is raised and O^T, l rescaled outside, and the tile finished.
    int it = 0;
    while (it < ntiles) {
        for (; it < ntiles; ++it) {
            score_tile(it);
            bool need = false;
#pragma unroll
            for (int hb = 0; hb < HPW; ++hb) need |= mx[hb] > m_ref[hb] + kRescaleSlack;
            if (__builtin_amdgcn_ballot_w64(need) != 0) break;  // same in both waves of the pair
            accumulate(it);
        }
        if (it == ntiles) break;
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) {
            const float m_new = fmaxf(m_ref[hb], mx[hb]);
            const float alpha = m_new == -INFINITY ? 1.0f : exp2f(m_ref[hb] - m_new);
            m_ref[hb] = m_new;
            l_lane[hb] *= alpha;
#pragma unroll
            for (int vb = 0; vb < 16; ++vb) acc[hb][vb] *= alpha;
        }
        accumulate(it);
        ++it;
    }

    // ---- partial outputs: O^T lane (head l16, lq) holds dims 16 vbg + 4 lq .. +4;
    // rows are stored in bf16 (the output's own precision), m and l in fp32 ----
    const int64_t hbase = ((int64_t)r * n_splits + split) * Hq + h0;
#pragma unroll
    for (int hb = 0; hb < HPW; ++hb) {
        uint16_t* dst = part_o + (hbase + hb * 16 + l16) * MDV + 256 * vh + 4 * lq;
#pragma unroll
        for (int vb = 0; vb < 16; ++vb)
            *(uint2*)(dst + 16 * vb) = make_uint2(pack_bf16(acc[hb][vb][0], acc[hb][vb][1]),
                                                  pack_bf16(acc[hb][vb][2], acc[hb][vb][3]));
        const float l = add_xor32(add_xor16(l_lane[hb]));
        if (vh == 0 && lq == 0) {
            part_ml[(hbase + hb * 16 + l16) * 2 + 0] = m_ref[hb];
            part_ml[(hbase + hb * 16 + l16) * 2 + 1] = l;
        }
    }
}

// ----------------------------------------------------------------------------
// fp32 rows, VALU (small head counts)
// ----------------------------------------------------------------------------
constexpr int FT = 16;        // tokens per tile
constexpr int FMAXH = 16, FMAXD = 256;

__global__ __launch_bounds__(256) void k_attn_f32(GeomDev g, PosMap pm, const int32_t* __restrict__ tcnt,
                                                  const float* __restrict__ q, int Hq, int Dk,
                                                  int Dv, int v_off, int n_splits, int per_split,
                                                  float sm_log2e, float* __restrict__ part_o,
                                                  float* __restrict__ part_ml) {
    __shared__ __attribute__((aligned(16))) float Ks[FT][FMAXD + 4];
    __shared__ __attribute__((aligned(16))) float Vs[FT][FMAXD + 4];
    __shared__ __attribute__((aligned(16))) float qs[FMAXH][FMAXD];
    __shared__ float Sl[FMAXH][FT];
    __shared__ float m_s[FMAXH], l_s[FMAXH], a_s[FMAXH];
    __shared__ const uint8_t* rowt[FT];

    const int r = blockIdx.x / n_splits, split = blockIdx.x % n_splits;
    const int tid = threadIdx.x;
    const int kcnt = tcnt[r];
    const int p_begin = split * per_split;
    const int P = pm.k + g.nrec[r];
    const int npos = max(0, min(per_split, P - p_begin));

    for (int e = tid; e < Hq * Dk; e += 256) qs[e / Dk][e % Dk] = q[(int64_t)r * Hq * Dk + e];
    if (tid < Hq) {
        m_s[tid] = -INFINITY;
        l_s[tid] = 0.0f;
    }
    constexpr int NA = FMAXH * FMAXD / 256;
    float acc[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) acc[i] = 0.0f;
    const int nel = Hq * Dv;

    for (int t0 = 0; t0 < npos; t0 += FT) {
        if (tid < FT) rowt[tid] = (t0 + tid < npos) ? pos_row(g, pm, r, kcnt, p_begin + t0 + tid) : nullptr;
        __syncthreads();
        for (int e = tid; e < FT * (Dk / 4); e += 256) {
            const int t = e / (Dk / 4), c4 = e % (Dk / 4);
            const uint8_t* row = rowt[t];
            const float4 v = row ? *(const float4*)(row + c4 * 16) : make_float4(0.f, 0.f, 0.f, 0.f);
            *(float4*)&Ks[t][c4 * 4] = v;
        }
        for (int e = tid; e < FT * (Dv / 4); e += 256) {
            const int t = e / (Dv / 4), c4 = e % (Dv / 4);
            const uint8_t* row = rowt[t];
            const float4 v = row ? *(const float4*)(row + v_off * 4 + c4 * 16) : make_float4(0.f, 0.f, 0.f, 0.f);
            *(float4*)&Vs[t][c4 * 4] = v;
        }
        __syncthreads();
        for (int e = tid; e < Hq * FT; e += 256) {
            const int h = e / FT, t = e % FT;
            float x = -INFINITY;
            if (rowt[t] != nullptr) {
                float a = 0.0f;
                for (int i = 0; i < Dk; ++i) a = __builtin_fmaf(qs[h][i], Ks[t][i], a);
                x = a * sm_log2e;
            }
            Sl[h][t] = x;
        }
        __syncthreads();
        if (tid < Hq) {
            float mt = -INFINITY;
            for (int t = 0; t < FT; ++t) mt = fmaxf(mt, Sl[tid][t]);
            const float m_old = m_s[tid];
            const float m_new = fmaxf(m_old, mt);
            const bool none = (m_new == -INFINITY);
            const float alpha = none ? 1.0f : exp2f(m_old - m_new);
            float ls = 0.0f;
            for (int t = 0; t < FT; ++t) {
                const float p = none ? 0.0f : exp2f(Sl[tid][t] - m_new);
                Sl[tid][t] = p;
                ls += p;
            }
            l_s[tid] = l_s[tid] * alpha + ls;
            m_s[tid] = m_new;
            a_s[tid] = alpha;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int e = tid + 256 * i;
            if (e < nel) {
                const int h = e / Dv, v = e % Dv;
                float a = acc[i] * a_s[h];
                for (int t = 0; t < FT; ++t) a = __builtin_fmaf(Sl[h][t], Vs[t][v], a);
                acc[i] = a;
            }
        }
        __syncthreads();
    }
    const int64_t hbase = ((int64_t)r * n_splits + split) * Hq;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int e = tid + 256 * i;
        if (e < nel) part_o[(hbase + e / Dv) * Dv + e % Dv] = acc[i];
    }
    if (tid < Hq) {
        part_ml[(hbase + tid) * 2 + 0] = m_s[tid];
        part_ml[(hbase + tid) * 2 + 1] = l_s[tid];
    }
}

// ----------------------------------------------------------------------------
// merge of the splits: one block per (request, head, 64 * VPL value columns),
// VPL = 16 bytes of a partial row per lane (8 bf16 columns on the bf16 latent
// path, 4 fp32 columns on the f32 path), so a load reads a whole 1 KB
// partial row.  The block's kMergeWaves waves take contiguous ranges of the
// splits and have all their rows in flight at once (the merge is bound by
// the load latency, not the bytes).  Every wave forms the split weights
// 2^(m_s - m) and the total sum in the same fixed order; each lane combines
// its columns over its range in split order, and the ranges are added in
// wave order.
// ----------------------------------------------------------------------------
constexpr int kMergeMaxSplits = 1024;
constexpr int kMergeWaves = 4;   // waves per block (split ranges)
constexpr int kMergeBatch = 8;   // partial rows in flight per lane

template <typename PT>
__host__ __device__ inline int merge_col_blocks(int Dv) {
    constexpr int VPL = 16 / (int)sizeof(PT);
    return (Dv + 64 * VPL - 1) / (64 * VPL);
}

template <int ODT, typename PT>
__global__ __launch_bounds__(64 * kMergeWaves) void k_attn_merge(const PT* __restrict__ part_o,
                                                               const float* __restrict__ part_ml,
                                                               int B, int Hq, int Dv, int n_splits,
                                                               void* __restrict__ out,
                                                               float* __restrict__ lse) {
    constexpr int VPL = 16 / (int)sizeof(PT);
    __shared__ float fac[kMergeMaxSplits];
    __shared__ float red[kMergeWaves][VPL][64];
    const int w = threadIdx.x >> 6, L = threadIdx.x & 63;
    const int ncb = merge_col_blocks<PT>(Dv);
    const int unit = blockIdx.x;  // (r * Hq + h) * ncb + cb
    if (unit >= B * Hq * ncb) return;  // uniform per block
    const int rh = unit / ncb, cb = unit % ncb;
    const int r = rh / Hq, h = rh % Hq;
    const int64_t b0 = (int64_t)r * n_splits * Hq + h;  // split s: (b0 + s*Hq)
    const int v = (cb * 64 + L) * VPL;                  // first column of the lane
    const bool col = v < Dv;                            // Dv is a multiple of VPL
    const PT* src = part_o + b0 * Dv + v;
    const int64_t stride = (int64_t)Hq * Dv;
    const int per = (n_splits + kMergeWaves - 1) / kMergeWaves;
    const int s_lo = min(w * per, n_splits), s_hi = min(s_lo + per, n_splits);
    // the first batch of partial rows is requested before the split weights
    // are formed, so both latencies overlap
    uint4 x[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
        if (col && s_lo + u < s_hi) x[u] = *(const uint4*)(src + (int64_t)(s_lo + u) * stride);
    float m = -INFINITY;
    for (int s = L; s < n_splits; s += 64) m = fmaxf(m, part_ml[(b0 + (int64_t)s * Hq) * 2]);
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float part = 0.0f;
    for (int s = L; s < n_splits; s += 64) {
        const float ms = part_ml[(b0 + (int64_t)s * Hq) * 2];
        const float f = (ms == -INFINITY) ? 0.0f : exp2f(ms - m);
        if (w == 0) fac[s] = f;
        part += part_ml[(b0 + (int64_t)s * Hq) * 2 + 1] * f;
    }
    // fixed-order tree over the lanes
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    // an empty attended set (no recent token, no top-k entry) has no
    // softmax: its output is zero and its lse -inf
    const float Lsum = part, inv = part > 0.0f ? 1.0f / part : 0.0f;
    __syncthreads();  // fac complete
    float o[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) o[i] = 0.0f;
    if (col) {
        for (int s0 = s_lo; s0 < s_hi; s0 += kMergeBatch) {
            if (s0 > s_lo) {
#pragma unroll
                for (int u = 0; u < kMergeBatch; ++u)
                    if (s0 + u < s_hi) x[u] = *(const uint4*)(src + (int64_t)(s0 + u) * stride);
            }
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u) {
                if (s0 + u < s_hi) {
                    const float f = fac[s0 + u];
                    if (f != 0.0f) {
                        const uint32_t wd[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
                        for (int i = 0; i < VPL; ++i) {
                            float xv;
                            if constexpr (sizeof(PT) == 4) xv = __uint_as_float(wd[i]);
                            else xv = (i & 1) ? bf16_hi(wd[i >> 1]) : bf16_lo(wd[i >> 1]);
                            o[i] += xv * f;
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) red[w][i][L] = o[i];
    __syncthreads();
    if (w == 0 && col) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            float t = red[0][i][L];
#pragma unroll
            for (int k = 1; k < kMergeWaves; ++k) t += red[k][i][L];
            o[i] = t;
        }
        const int64_t ob = (int64_t)rh * Dv + v;
        if constexpr (ODT == LSA_F32) {
            float* dst = (float*)out + ob;
            if (((uintptr_t)dst & 15) == 0) {
                *(float4*)dst = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
            } else {
#pragma unroll
                for (int i = 0; i < VPL; ++i) dst[i] = o[i] * inv;
            }
        } else {
            uint16_t* dst = (uint16_t*)out + ob;
            uint16_t y[VPL];
#pragma unroll
            for (int i = 0; i < VPL; ++i) y[i] = f2bf(o[i] * inv);
            if (VPL == 8 && ((uintptr_t)dst & 15) == 0) {
                uint32_t pk[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) pk[i] = (uint32_t)y[2 * i] | ((uint32_t)y[2 * i + 1] << 16);
                *(uint4*)dst = make_uint4(pk[0], pk[1], pk[2], pk[3]);
            } else {
#pragma unroll
                for (int i = 0; i < VPL; ++i) dst[i] = y[i];
            }
        }
    }
    if (lse && cb == 0 && w == 0 && L == 0) lse[rh] = Lsum > 0.0f ? (m + __log2f(Lsum)) * kLn2 : -INFINITY;
}

}  // namespace

lsa_status attn_plan(const GeomDev& g, const lsa_kv_layout* kv, int Hq, int k, int n_splits,
                     AttnPlan* plan) {
    int max_rec = 0;
    for (int r = 0; r < g.B; ++r) max_rec = g.nrec[r] > max_rec ? g.nrec[r] : max_rec;
    const int P = k + max_rec;
    AttnPlan p{};
    p.P_max = P;
    if (kv->kv_dtype == LSA_BF16) {
        if (kv->Dk != MDK || kv->Dv != MDV || kv->v_off != 0 || Hq % 32 != 0 ||
            kv->row_bytes % 16 != 0 || kv->page_bytes % 16 != 0)
            return LSA_ERR_UNSUPPORTED;
        p.mode = 1;
        p.waves = Hq % 64 == 0 ? 8 : 4;  // 16 heads per wave: 64 or 32 heads per block
        p.head_groups = Hq / (8 * p.waves);
        const int tile = MT;
        int S = n_splits;
        if (S <= 0) {
            // one block per CU over 256 CUs, at least 2 tiles per split
            const int want = (256 + g.B * p.head_groups - 1) / (g.B * p.head_groups);
            const int max_by_len = (P + 2 * tile - 1) / (2 * tile);
            S = want < max_by_len ? want : max_by_len;
            if (S < 1) S = 1;
        }
        int per = (P + S - 1) / S;
        per = (per + tile - 1) / tile * tile;
        if (per > kMaxSplitPos) per = kMaxSplitPos;
        p.n_splits = (P + per - 1) / per;
        p.per_split = per;
    } else if (kv->kv_dtype == LSA_F32) {
        if (Hq > FMAXH || kv->Dk > FMAXD || kv->Dv > FMAXD || kv->Dk % 4 || kv->Dv % 4 ||
            kv->v_off % 4 || kv->row_bytes % 16 || kv->page_bytes % 16)
            return LSA_ERR_UNSUPPORTED;
        p.mode = 0;
        p.head_groups = 1;
        int S = n_splits;
        if (S <= 0) {
            const int want = (256 + g.B - 1) / g.B;
            const int max_by_len = (P + 4 * FT - 1) / (4 * FT);
            S = want < max_by_len ? want : max_by_len;
            if (S < 1) S = 1;
        }
        int per = (P + S - 1) / S;
        per = (per + FT - 1) / FT * FT;
        p.n_splits = (P + per - 1) / per;
        p.per_split = per;
    } else {
        return LSA_ERR_UNSUPPORTED;
    }
    if (p.n_splits > kMergeMaxSplits) return LSA_ERR_UNSUPPORTED;
    // partial rows: bf16 on the bf16 latent path, fp32 on the f32 path
    p.part_o_bytes = align_up((size_t)g.B * p.n_splits * Hq * kv->Dv * (p.mode == 1 ? 2 : 4), 256);
    p.part_ml_bytes = align_up((size_t)g.B * p.n_splits * Hq * 2 * sizeof(float), 256);
    *plan = p;
    return LSA_OK;
}

// Each GPU holds its own copy of the error word; its address is looked up
// once per device (with that device current) and kept.
__device__ uint32_t g_lsa_err_word;

// The split partials of lsa_sparse_decode_attn_noalloc, for callers that
// cannot allocate: a device array of fixed size that each GPU holds from the
// library's load until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in); it uses the device
// address that attn_scratch() looks up once per device.
constexpr size_t kAttnScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kAttnScratchBytes];

size_t attn_scratch_bytes() { return kAttnScratchBytes; }

void* attn_scratch() {
    constexpr int kMaxDev = 64;
    static std::atomic<void*> addr[kMaxDev];
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
    void* a = addr[dev].load(std::memory_order_acquire);
    if (a) return a;
    std::lock_guard<std::mutex> lk(mu);
    a = addr[dev].load(std::memory_order_relaxed);
    if (!a) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        a = p;
        addr[dev].store(a, std::memory_order_release);
    }
    return a;
}

uint32_t* dev_err_word() {
    constexpr int kMaxDev = 64;
    static std::atomic<uint32_t*> addr[kMaxDev];
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
    uint32_t* a = addr[dev].load(std::memory_order_acquire);
    if (a) return a;
    std::lock_guard<std::mutex> lk(mu);
    a = addr[dev].load(std::memory_order_relaxed);
    if (!a) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_lsa_err_word)) != hipSuccess || !p) return nullptr;
        a = (uint32_t*)p;
        addr[dev].store(a, std::memory_order_release);
    }
    return a;
}

hipError_t launch_attn(const GeomDev& g, const AttnPlan& plan, const void* q, int Hq,
                       const lsa_kv_layout& kv, const void* pages, const int32_t* page_table,
                       const void* recent, const int32_t* topk, const int32_t* tcnt, int k,
                       float sm_scale, void* out, float* lse, void* ws, hipStream_t s) {
    PosMap pm{(const uint8_t*)pages, kv.page_bytes, kv.row_bytes, page_table,
              (const uint8_t*)recent, topk, k};
    float* part_o = (float*)ws;  // fp32 rows (f32 path) or bf16 rows (latent path)
    float* part_ml = (float*)((uint8_t*)ws + plan.part_o_bytes);
    const float sm_log2e = sm_scale * 1.44269504088896340736f;
    if (plan.mode == 1) {
        uint32_t* err = dev_err_word();
        if (!err) return hipErrorInvalidSymbol;
        const int tp = tune_get(LSA_TUNE_ATTN_PAIR_POLLS);
        const int polls = tp >= 0 ? tp : (1 << 20);
        const int units = g.B * plan.n_splits;
        const int grid = (units + 7) / 8 * 8 * plan.head_groups;
        timing_begin("k_attn_mla", s);
        if (plan.waves == 8)
            hipLaunchKernelGGL((k_attn_mla<8, 1>), dim3(grid), dim3(512), 0, s, g, pm, tcnt,
                               (const uint16_t*)q, Hq, plan.n_splits, plan.per_split,
                               plan.head_groups, sm_log2e, (uint16_t*)part_o, part_ml, polls, err);
        else
            hipLaunchKernelGGL((k_attn_mla<4, 1>), dim3(grid), dim3(256), 0, s, g, pm, tcnt,
                               (const uint16_t*)q, Hq, plan.n_splits, plan.per_split,
                               plan.head_groups, sm_log2e, (uint16_t*)part_o, part_ml, polls, err);
        timing_end("k_attn_mla", s);
    } else {
        timing_begin("k_attn_f32", s);
        hipLaunchKernelGGL(k_attn_f32, dim3(g.B * plan.n_splits), dim3(256), 0, s, g, pm, tcnt,
                           (const float*)q, Hq, kv.Dk, kv.Dv, kv.v_off, plan.n_splits,
                           plan.per_split, sm_log2e, part_o, part_ml);
        timing_end("k_attn_f32", s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int mblocks = g.B * Hq * (plan.mode == 1 ? merge_col_blocks<uint16_t>(kv.Dv)
                                                   : merge_col_blocks<float>(kv.Dv));
    timing_begin("k_attn_merge", s);
    if (plan.mode != 1)
        hipLaunchKernelGGL((k_attn_merge<LSA_F32, float>), dim3(mblocks), dim3(64 * kMergeWaves), 0,
                           s, (const float*)part_o, part_ml, g.B, Hq, kv.Dv, plan.n_splits, out, lse);
    else
        hipLaunchKernelGGL((k_attn_merge<LSA_BF16, uint16_t>), dim3(mblocks), dim3(64 * kMergeWaves),
                           0, s, (const uint16_t*)part_o, part_ml, g.B, Hq, kv.Dv, plan.n_splits,
                           out, lse);
    timing_end("k_attn_merge", s);
    return hipGetLastError();
}
