// Sparse decode attention over the top-k tokens plus the recent window (gfx950).
//
// Core attention runs on the tokens the staged selection keeps (gist.science
// summary, section 2.1 "Gestufte Selektion") together with the most recent
// window, which always stays on the GPU (cjcn.com.cn explainer, section 二
// last paragraph; section 五: every scheme keeps the recent 8K).  All query
// heads share one KV row per token (MQA); the latent row holds 576 values and
// the value is its first 512.
//
// Positions of request r: p in [0, k) is top-k slot p (valid below the
// top-k count), p in [k, k + R_r) is recent token rs + (p - k).  Positions
// are cut into splits; each split keeps a running max m, sum l and
// unnormalised output (online softmax, base 2) and writes them to a
// workspace; k_attn_merge combines the splits of each (request, head).
//
// k_attn_mla (bf16, Dk 576 / Dv 512): one block per (request, split, group
// of 32 heads), 4 waves, 32-token tiles, MFMA 16x16x32 bf16; every KV byte
// is read from HBM once per head group and feeds both products.
// Algorithmic bytes per attended token: 1,152 (HBM-bound).
//
// k_attn_f32: fp32 rows, VALU, for small head counts (fp32 path).
#include "lsa_internal.h"

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
// bf16 latent MQA (Dk 576, Dv 512), MFMA
// ----------------------------------------------------------------------------
constexpr int MT = 32;           // tokens per tile
constexpr int MH = 32;           // heads per block
constexpr int MDK = 576, MDV = 512;
constexpr int PLS = 40;          // pl row stride (bf16)
constexpr int kMaxSplitPos = 1024;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }


// ----------------------------------------------------------------------------
// bf16 latent MQA, second form: the 32-token KV tile sits row-major in LDS
// (rows padded to 1168 bytes), filled from registers that prefetch the next
// tile.  S = Q K^T splits the 576-wide contraction over the 4 waves as
// above; O += P V takes its V operands with LDS transpose reads
// (ds_read_b64_tr_b16: lane n of each 16-lane group, pointing at
// V[t0 + n/4][v0 + 4(n%4)], receives V[t0..t0+3][v0 + n]), so no transposed
// copy of V is written.  Softmax is spread over all waves, one head per 8
// lanes.  About 66 KB of LDS: two blocks per CU.
// ----------------------------------------------------------------------------
constexpr int RB = 1152, RBP = 1168;    // KV row bytes, padded LDS row bytes
constexpr int SPT = 36;                 // sp row stride (floats), head-major [h][t]
constexpr int kPieces = MT * RB / 16;   // 16-byte pieces per tile (2304)
constexpr int kPPT = kPieces / 256;     // pieces per thread (9)

typedef short v4i16_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 lds_tr16(const uint8_t* base_lds, int byte_off) {
    const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16_t*)((__attribute__((address_space(3))) uint8_t*)base_lds +
                                                      byte_off));
    return __builtin_bit_cast(uint2, r);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4_t gu32x4_t;

__global__ __launch_bounds__(256, 2) void k_attn_mla(GeomDev g, PosMap pm,
                                                     const int32_t* __restrict__ tcnt,
                                                     const uint16_t* __restrict__ q, int Hq,
                                                     int n_splits, int per_split, int hgroups,
                                                     float sm_log2e, float* __restrict__ part_o,
                                                     float* __restrict__ part_ml) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[MT * RBP];
    __shared__ __attribute__((aligned(16))) float sp[4][MH * SPT];
    __shared__ __attribute__((aligned(16))) uint16_t pl[MH][PLS];
    __shared__ __attribute__((aligned(16))) float alpha_s[MH];
    // row address per position; bit 0 set: empty position (the address is then
    // a valid row of finite values, whose probability is forced to 0)
    __shared__ uint64_t rowp[kMaxSplitPos];

    const int bi = blockIdx.x;
    const int xcd = bi & 7, j = bi >> 3;
    const int hg = j % hgroups;
    const int unit = (j / hgroups) * 8 + xcd;
    if (unit >= g.B * n_splits) return;
    const int r = unit / n_splits, split = unit % n_splits;

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, lq = l >> 4;
    const int kcnt = tcnt[r];
    const int p_begin = split * per_split;
    const int P = pm.k + g.nrec[r];
    const int npos = max(0, min(per_split, P - p_begin));
    const int ntiles = (npos + MT - 1) / MT;
    const uint64_t dummy = (uint64_t)(pm.recent + g.rec_off[r] * pm.row_bytes) | 1ull;

    for (int i = tid; i < ntiles * MT; i += 256) {
        const uint8_t* row = (i < npos) ? pos_row(g, pm, r, kcnt, p_begin + i) : nullptr;
        rowp[i] = row ? (uint64_t)row : dummy;
    }

    // Q slices as MFMA A operands: k-steps 4w..4w+3 and the rope k-step 16+w
    // (waves 2 and 3 have no rope k-step: a zero slice)
    uint4 Qa[2][5];
    const uint16_t* qr = q + ((int64_t)r * Hq + hg * MH) * MDK;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            Qa[hb][jj] = *(const uint4*)(qr + (hb * 16 + l16) * MDK + (4 * w + jj) * 32 + lq * 8);
        Qa[hb][4] = (w < 2) ? *(const uint4*)(qr + (hb * 16 + l16) * MDK + (16 + w) * 32 + lq * 8)
                            : make_uint4(0, 0, 0, 0);
    }
    const int ks4 = 16 + (w & 1);  // rope k-step read by this wave (harmless for w >= 2)
    __syncthreads();  // rowp ready

    // tile loader: 8 threads per row; thread t copies the 16-byte columns
    // (t%8) + 8k, k = 0..8, of row t/8 (coalesced 128-byte runs per row)
    const int ld_row = tid >> 3, ld_col = (tid & 7) * 16;
    uint8_t* const ld_dst = tile + ld_row * RBP + ld_col;

    f32x4_t acc[2][8];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int vb = 0; vb < 8; ++vb) acc[hb][vb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;  // head 8w + l/8

    u32x4_t R0[kPPT];  // the next tile, in flight while this one is computed
    if (ntiles > 0) {
        const int T0_ = 0;
        {
            gu32x4_t* src_ = (gu32x4_t*)((rowp[T0_ + ld_row] & ~15ull) + ld_col);
            R0[0] = src_[0]; R0[1] = src_[8]; R0[2] = src_[16]; R0[3] = src_[24];
            R0[4] = src_[32]; R0[5] = src_[40]; R0[6] = src_[48]; R0[7] = src_[56];
            R0[8] = src_[64];
        }
        {
            u32x4_t* d_ = (u32x4_t*)ld_dst;
            d_[0] = R0[0]; d_[8] = R0[1]; d_[16] = R0[2]; d_[24] = R0[3]; d_[32] = R0[4];
            d_[40] = R0[5]; d_[48] = R0[6]; d_[56] = R0[7]; d_[64] = R0[8];
        }
    }
    if (ntiles > 1) {
        const int T0_ = MT;
        {
            gu32x4_t* src_ = (gu32x4_t*)((rowp[T0_ + ld_row] & ~15ull) + ld_col);
            R0[0] = src_[0]; R0[1] = src_[8]; R0[2] = src_[16]; R0[3] = src_[24];
            R0[4] = src_[32]; R0[5] = src_[40]; R0[6] = src_[48]; R0[7] = src_[56];
            R0[8] = src_[64];
        }
    }

    for (int it = 0; it < ntiles; ++it) {
        const int t0 = it * MT;
        __syncthreads();  // tile `it` is in LDS
        // ---- partial S over this wave's dims: sp[w][h][t] ----
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const uint8_t* krow = tile + (tb * 16 + l16) * RBP + lq * 16;
            uint4 kb[5];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) kb[jj] = *(const uint4*)(krow + (4 * w + jj) * 64);
            kb[4] = *(const uint4*)(krow + ks4 * 64);
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int jj = 0; jj < 5; ++jj)
                    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Qa[hb][jj]),
                                                                as_bf16x8(kb[jj]), c, 0, 0, 0);
                float* dst = &sp[w][(hb * 16 + lq * 4) * SPT + tb * 16 + l16];
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i * SPT] = c[i];
            }
        }
        __syncthreads();
        // ---- online softmax: head h = 8w + l/8, tokens 4*(l%8) .. +4 ----
        {
            const int h = 8 * w + (l >> 3), tq = 4 * (l & 7);
            const float4 a = *(const float4*)&sp[0][h * SPT + tq];
            const float4 b = *(const float4*)&sp[1][h * SPT + tq];
            const float4 c = *(const float4*)&sp[2][h * SPT + tq];
            const float4 d = *(const float4*)&sp[3][h * SPT + tq];
            float x[4] = {((a.x + b.x) + c.x) + d.x, ((a.y + b.y) + c.y) + d.y,
                          ((a.z + b.z) + c.z) + d.z, ((a.w + b.w) + c.w) + d.w};
            float mloc = -INFINITY;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = (rowp[t0 + tq + e] & 1ull) ? -INFINITY : x[e] * sm_log2e;
                mloc = fmaxf(mloc, x[e]);
            }
            mloc = fmaxf(mloc, __shfl_xor(mloc, 1));
            mloc = fmaxf(mloc, __shfl_xor(mloc, 2));
            mloc = fmaxf(mloc, __shfl_xor(mloc, 4));
            const float m_new = fmaxf(m_run, mloc);
            const bool none = (m_new == -INFINITY);
            const float alpha = none ? 1.0f : exp2f(m_run - m_new);
            float p[4], lsum = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] = none ? 0.0f : exp2f(x[e] - m_new);
                lsum += p[e];
            }
            lsum += __shfl_xor(lsum, 1);
            lsum += __shfl_xor(lsum, 2);
            lsum += __shfl_xor(lsum, 4);
            l_run = l_run * alpha + lsum;
            m_run = m_new;
            *(uint2*)&pl[h][tq] = make_uint2((uint32_t)f2bf(p[0]) | ((uint32_t)f2bf(p[1]) << 16),
                                             (uint32_t)f2bf(p[2]) | ((uint32_t)f2bf(p[3]) << 16));
            if ((l & 7) == 0) alpha_s[h] = alpha;
        }
        __syncthreads();
        // ---- O[:, 128w .. 128w+128) = O * alpha + P V ----
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const float4 a4 = *(const float4*)&alpha_s[hb * 16 + lq * 4];
            const bf16x8_t pa = as_bf16x8(*(const uint4*)&pl[hb * 16 + l16][lq * 8]);
#pragma unroll
            for (int vb = 0; vb < 8; ++vb) {
                acc[hb][vb][0] *= a4.x;
                acc[hb][vb][1] *= a4.y;
                acc[hb][vb][2] *= a4.z;
                acc[hb][vb][3] *= a4.w;
                const int off0 = (lq * 8 + (l16 >> 2)) * RBP + (128 * w + vb * 16 + 4 * (l16 & 3)) * 2;
                const uint2 lo = lds_tr16(tile, off0);
                const uint2 hi = lds_tr16(tile, off0 + 4 * RBP);
                const bf16x8_t vb8 = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
                acc[hb][vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb8, acc[hb][vb], 0, 0, 0);
            }
        }
        __syncthreads();  // every wave is done with tile `it`
        if (it + 1 < ntiles) {
            {
            u32x4_t* d_ = (u32x4_t*)ld_dst;
            d_[0] = R0[0]; d_[8] = R0[1]; d_[16] = R0[2]; d_[24] = R0[3]; d_[32] = R0[4];
            d_[40] = R0[5]; d_[48] = R0[6]; d_[56] = R0[7]; d_[64] = R0[8];
        }
            if (it + 2 < ntiles) {
                const int T0_ = t0 + 2 * MT;
                {
            gu32x4_t* src_ = (gu32x4_t*)((rowp[T0_ + ld_row] & ~15ull) + ld_col);
            R0[0] = src_[0]; R0[1] = src_[8]; R0[2] = src_[16]; R0[3] = src_[24];
            R0[4] = src_[32]; R0[5] = src_[40]; R0[6] = src_[48]; R0[7] = src_[56];
            R0[8] = src_[64];
        }
            }
        }
    }

    const int64_t hbase = ((int64_t)r * n_splits + split) * Hq + hg * MH;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int vb = 0; vb < 8; ++vb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                part_o[(hbase + hb * 16 + lq * 4 + i) * MDV + 128 * w + vb * 16 + l16] = acc[hb][vb][i];
    if ((l & 7) == 0) {
        const int h = 8 * w + (l >> 3);
        part_ml[(hbase + h) * 2 + 0] = m_run;
        part_ml[(hbase + h) * 2 + 1] = l_run;
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
// merge of the splits: one block per (request, head).  The split weights
// 2^(m_s - m) and the total sum are formed once per block in a fixed order;
// then each thread combines four columns at a time.
// ----------------------------------------------------------------------------
constexpr int kMergeMaxSplits = 1024;

template <int ODT>
__global__ __launch_bounds__(128) void k_attn_merge(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml, int Hq,
                                                    int Dv, int n_splits, void* __restrict__ out,
                                                    float* __restrict__ lse) {
    __shared__ float fac[kMergeMaxSplits];
    __shared__ float s_m, s_inv, s_L;
    const int rh = blockIdx.x;  // r * Hq + h
    const int r = rh / Hq, h = rh % Hq;
    const int64_t b0 = (int64_t)r * n_splits * Hq + h;  // split s: (b0 + s*Hq)
    // split weights in parallel; max and sum by a fixed-order tree
    __shared__ float red[128];
    float m = -INFINITY;
    for (int s = threadIdx.x; s < n_splits; s += blockDim.x)
        m = fmaxf(m, part_ml[(b0 + (int64_t)s * Hq) * 2]);
    red[threadIdx.x] = m;
    __syncthreads();
    for (int w = 64; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
        __syncthreads();
    }
    m = red[0];
    __syncthreads();
    float part = 0.0f;
    for (int s = threadIdx.x; s < n_splits; s += blockDim.x) {
        const float ms = part_ml[(b0 + (int64_t)s * Hq) * 2];
        const float f = (ms == -INFINITY) ? 0.0f : exp2f(ms - m);
        fac[s] = f;
        part += part_ml[(b0 + (int64_t)s * Hq) * 2 + 1] * f;
    }
    red[threadIdx.x] = part;
    __syncthreads();
    for (int w = 64; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        s_m = m;
        s_L = red[0];
        s_inv = 1.0f / red[0];
    }
    __syncthreads();
    const float inv = s_inv;
    for (int v = 4 * threadIdx.x; v < Dv; v += 4 * blockDim.x) {
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
        for (int s = 0; s < n_splits; ++s) {
            const float f = fac[s];
            const float4 x = *(const float4*)&part_o[(b0 + (int64_t)s * Hq) * Dv + v];
            o.x += f == 0.0f ? 0.0f : x.x * f;
            o.y += f == 0.0f ? 0.0f : x.y * f;
            o.z += f == 0.0f ? 0.0f : x.z * f;
            o.w += f == 0.0f ? 0.0f : x.w * f;
        }
        const float ov[4] = {o.x * inv, o.y * inv, o.z * inv, o.w * inv};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (ODT == LSA_F32)
                ((float*)out)[(int64_t)rh * Dv + v + e] = ov[e];
            else
                ((uint16_t*)out)[(int64_t)rh * Dv + v + e] = f2bf(ov[e]);
        }
    }
    if (lse && threadIdx.x == 0) lse[rh] = (s_m + __log2f(s_L)) * kLn2;
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
        if (kv->Dk != MDK || kv->Dv != MDV || kv->v_off != 0 || Hq % MH != 0 ||
            kv->row_bytes % 16 != 0 || kv->page_bytes % 16 != 0)
            return LSA_ERR_UNSUPPORTED;
        p.mode = 1;
        p.head_groups = Hq / MH;
        const int tile = MT;
        int S = n_splits;
        if (S <= 0) {
            // about two blocks per CU over 256 CUs, at least 2 tiles per split
            const int want = (512 + g.B * p.head_groups - 1) / (g.B * p.head_groups);
            const int max_by_len = (P + 2 * tile - 1) / (2 * tile);
            S = want < max_by_len ? want : max_by_len;
            if (S < 1) S = 1;
        }
        int per = (P + S - 1) / S;
        per = (per + tile - 1) / tile * tile;
        if (per > kMaxSplitPos) {
            per = kMaxSplitPos;
            S = (P + per - 1) / per;
        }
        S = (P + per - 1) / per;
        p.n_splits = S;
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
    p.part_o_bytes = align_up((size_t)g.B * p.n_splits * Hq * kv->Dv * sizeof(float), 256);
    p.part_ml_bytes = align_up((size_t)g.B * p.n_splits * Hq * 2 * sizeof(float), 256);
    *plan = p;
    return LSA_OK;
}

hipError_t launch_attn(const GeomDev& g, const AttnPlan& plan, const void* q, int Hq,
                       const lsa_kv_layout& kv, const void* pages, const int32_t* page_table,
                       const void* recent, const int32_t* topk, const int32_t* tcnt, int k,
                       float sm_scale, void* out, float* lse, void* ws, hipStream_t s) {
    PosMap pm{(const uint8_t*)pages, kv.page_bytes, kv.row_bytes, page_table,
              (const uint8_t*)recent, topk, k};
    float* part_o = (float*)ws;
    float* part_ml = (float*)((uint8_t*)ws + plan.part_o_bytes);
    const float sm_log2e = sm_scale * 1.44269504088896340736f;
    if (plan.mode == 1) {
        const int units = g.B * plan.n_splits;
        const int grid = (units + 7) / 8 * 8 * plan.head_groups;
        timing_begin("k_attn_mla", s);
        hipLaunchKernelGGL(k_attn_mla, dim3(grid), dim3(256), 0, s, g, pm, tcnt,
                           (const uint16_t*)q, Hq, plan.n_splits, plan.per_split,
                           plan.head_groups, sm_log2e, part_o, part_ml);
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
    timing_begin("k_attn_merge", s);
    if (kv.kv_dtype == LSA_F32)
        hipLaunchKernelGGL(k_attn_merge<LSA_F32>, dim3(g.B * Hq), dim3(128), 0, s, part_o,
                           part_ml, Hq, kv.Dv, plan.n_splits, out, lse);
    else
        hipLaunchKernelGGL(k_attn_merge<LSA_BF16>, dim3(g.B * Hq), dim3(128), 0, s, part_o,
                           part_ml, Hq, kv.Dv, plan.n_splits, out, lse);
    timing_end("k_attn_merge", s);
    return hipGetLastError();
}
