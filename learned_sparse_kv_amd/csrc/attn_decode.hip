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
// of 32 heads), 4 waves, 32-token tiles, MFMA 16x16x32 bf16.
//   S = Q K^T: the 576-wide contraction is split over the waves (wave w owns
//   dims [128w, 128w+128) plus one 32-wide slice of the 64 rope dims), Q
//   stays in registers, K comes straight from HBM into the MFMA operand
//   layout (one tile ahead), partial S goes through LDS.
//   O += P V: wave w owns value columns [128w, 128w+128) for all 32 heads;
//   its own V slice is the K slice it loaded, written transposed to LDS.
// So every KV byte is read from HBM once per head group and feeds both
// products.  Algorithmic bytes per attended token: 1,152 (HBM-bound).
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
constexpr int SPS = 36;          // sp row stride (floats)
constexpr int VTS = 40;          // vt row stride (bf16)
constexpr int PLS = 40;          // pl row stride (bf16)
constexpr int kMaxSplitPos = 1024;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__global__ __launch_bounds__(256) void k_attn_mla(GeomDev g, PosMap pm, const int32_t* __restrict__ tcnt,
                                                  const uint16_t* __restrict__ q, int Hq,
                                                  int n_splits, int per_split, int hgroups,
                                                  float sm_log2e, float* __restrict__ part_o,
                                                  float* __restrict__ part_ml) {
    __shared__ __attribute__((aligned(16))) float sp[4][MH][SPS];
    __shared__ __attribute__((aligned(16))) uint16_t vt[MDV][VTS];
    __shared__ __attribute__((aligned(16))) uint16_t pl[MH][PLS];
    __shared__ float alpha_s[MH];
    __shared__ const uint8_t* rowp[kMaxSplitPos];

    // block -> (request, split, head group); the head groups of one
    // (request, split) land on the same XCD one after another (blocks are
    // dispatched round-robin over the 8 XCDs), so their shared K/V tiles
    // are read from HBM once and from that XCD's L2 after.
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

    for (int i = tid; i < per_split; i += 256)
        rowp[i] = (i < npos) ? pos_row(g, pm, r, kcnt, p_begin + i) : nullptr;

    // Q in registers as MFMA A operands: Qa[hb][jj] = q[h = hb*16 + l16][ks*32 + lq*8 .. +8]
    const int nks = (w < 2) ? 5 : 4;
    uint4 Qa[2][5];
    const uint16_t* qr = q + ((int64_t)r * Hq + hg * MH) * MDK;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int jj = 0; jj < 5; ++jj) {
            const int ks = jj < 4 ? 4 * w + jj : 16 + w;
            Qa[hb][jj] = (jj < nks) ? *(const uint4*)(qr + (hb * 16 + l16) * MDK + ks * 32 + lq * 8)
                                    : make_uint4(0, 0, 0, 0);
        }
    __syncthreads();

    f32x4_t acc[2][8];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int vb = 0; vb < 8; ++vb) acc[hb][vb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;  // waves 0, 1: head w*16 + l16

    const int ntiles = (npos + MT - 1) / MT;
    uint4 Kb[2][5], Kn[2][5];
    auto load_tile = [&](int t0, uint4 (&dst)[2][5]) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const uint8_t* row = rowp[t0 + tb * 16 + l16];
#pragma unroll
            for (int jj = 0; jj < 5; ++jj) {
                const int ks = jj < 4 ? 4 * w + jj : 16 + w;
                dst[tb][jj] = (row != nullptr && jj < nks)
                                  ? *(const uint4*)(row + (ks * 32 + lq * 8) * 2)
                                  : make_uint4(0, 0, 0, 0);
            }
        }
    };
    if (ntiles > 0) load_tile(0, Kb);

    for (int it = 0; it < ntiles; ++it) {
        const int t0 = it * MT;
        if (it + 1 < ntiles) load_tile(t0 + MT, Kn);

        // ---- partial S over this wave's dims ----
        f32x4_t S[2][2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int jj = 0; jj < 5; ++jj)
                    if (jj < nks)
                        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Qa[hb][jj]),
                                                                    as_bf16x8(Kb[tb][jj]), c, 0, 0, 0);
                S[hb][tb] = c;
            }
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int i = 0; i < 4; ++i) sp[w][hb * 16 + lq * 4 + i][tb * 16 + l16] = S[hb][tb][i];
        // ---- this wave's value columns, transposed: vt[v][token] ----
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const uint4 v = Kb[tb][jj];
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                const int v0 = (4 * w + jj) * 32 + lq * 8;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vt[v0 + 2 * e][tb * 16 + l16] = (uint16_t)(w4[e] & 0xffffu);
                    vt[v0 + 2 * e + 1][tb * 16 + l16] = (uint16_t)(w4[e] >> 16);
                }
            }
        __syncthreads();

        // ---- online softmax for heads w*16 + l16 (waves 0 and 1) ----
        if (w < 2) {
            const int h = w * 16 + l16;
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; e += 4) {
                const float4 a = *(const float4*)&sp[0][h][lq * 8 + e];
                const float4 b = *(const float4*)&sp[1][h][lq * 8 + e];
                const float4 c = *(const float4*)&sp[2][h][lq * 8 + e];
                const float4 d = *(const float4*)&sp[3][h][lq * 8 + e];
                x[e + 0] = ((a.x + b.x) + c.x) + d.x;
                x[e + 1] = ((a.y + b.y) + c.y) + d.y;
                x[e + 2] = ((a.z + b.z) + c.z) + d.z;
                x[e + 3] = ((a.w + b.w) + c.w) + d.w;
            }
            float mloc = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool valid = rowp[t0 + lq * 8 + e] != nullptr;
                x[e] = valid ? x[e] * sm_log2e : -INFINITY;
                mloc = fmaxf(mloc, x[e]);
            }
            mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
            const float m_new = fmaxf(m_run, mloc);
            const bool none = (m_new == -INFINITY);
            const float alpha = none ? 1.0f : exp2f(m_run - m_new);
            float lsum = 0.0f;
            uint32_t pk[4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float p0 = none ? 0.0f : exp2f(x[e] - m_new);
                const float p1 = none ? 0.0f : exp2f(x[e + 1] - m_new);
                lsum += p0 + p1;
                pk[e / 2] = (uint32_t)f2bf(p0) | ((uint32_t)f2bf(p1) << 16);
            }
            lsum += __shfl_xor(lsum, 16);
            lsum += __shfl_xor(lsum, 32);
            l_run = l_run * alpha + lsum;
            m_run = m_new;
            *(uint4*)&pl[h][lq * 8] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
            if (lq == 0) alpha_s[h] = alpha;
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
                const bf16x8_t vb8 = as_bf16x8(*(const uint4*)&vt[128 * w + vb * 16 + l16][lq * 8]);
                acc[hb][vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb8, acc[hb][vb], 0, 0, 0);
            }
        }
        __syncthreads();
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int jj = 0; jj < 5; ++jj) Kb[tb][jj] = Kn[tb][jj];
    }

    // ---- partial results ----
    const int64_t hbase = ((int64_t)r * n_splits + split) * Hq + hg * MH;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int vb = 0; vb < 8; ++vb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                part_o[(hbase + hb * 16 + lq * 4 + i) * MDV + 128 * w + vb * 16 + l16] = acc[hb][vb][i];
    if (w < 2 && lq == 0) {
        part_ml[(hbase + w * 16 + l16) * 2 + 0] = m_run;
        part_ml[(hbase + w * 16 + l16) * 2 + 1] = l_run;
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
