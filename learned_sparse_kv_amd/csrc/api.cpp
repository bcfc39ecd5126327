// C-ABI entry points: argument checks, workspace sizing and dispatch.
// Every check runs before anything is enqueued; on error nothing is.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "lsa_internal.h"

#define LSA_HIP(x)                                      \
    do {                                                \
        if ((x) != hipSuccess) return LSA_ERR_HIP;      \
    } while (0)

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static int64_t esize(lsa_dtype t) { return t == LSA_F32 ? 4 : (t == LSA_BF16 ? 2 : 1); }

static lsa_status check_kv(const lsa_kv_layout* kv) {
    if (!kv) return LSA_ERR_INVALID_ARG;
    if (kv->Dk < 1 || kv->Dv < 1 || kv->v_off < 0) return LSA_ERR_INVALID_ARG;
    const int64_t need = esize(kv->kv_dtype) * (kv->Dk > kv->v_off + kv->Dv ? kv->Dk : kv->v_off + kv->Dv);
    if (kv->row_bytes < need) return LSA_ERR_INVALID_ARG;
    if (kv->page_bytes < kv->row_bytes * LSA_CHUNK) return LSA_ERR_INVALID_ARG;
    return LSA_OK;
}

lsa_status geom_derive(const lsa_geom* g, GeomDev* d) {
    if (!g || !d || !g->seq_len) return LSA_ERR_INVALID_ARG;
    if (g->batch < 1 || g->batch > LSA_MAX_BATCH) return LSA_ERR_INVALID_ARG;
    if (g->chunk != LSA_CHUNK || g->window < 0) return LSA_ERR_INVALID_ARG;
    if (g->chunk_cap < 0 || g->recent_cap < 0) return LSA_ERR_INVALID_ARG;
    std::memset(d, 0, sizeof(*d));
    d->B = g->batch;
    d->W = g->window;
    int64_t co = 0, ro = 0;
    int64_t to = 0;
    for (int r = 0; r < g->batch; ++r) {
        const int32_t L = g->seq_len[r];
        if (L < 1) return LSA_ERR_INVALID_ARG;
        int64_t rs;
        if (g->hist_tokens) {
            rs = g->hist_tokens[r];
            if (rs < 0 || rs > L || rs % LSA_CHUNK != 0) return LSA_ERR_INVALID_ARG;
        } else {
            int64_t h = (int64_t)L - g->window;
            if (h < 0) h = 0;
            rs = (int64_t)LSA_CHUNK * (h / LSA_CHUNK);
        }
        d->L[r] = L;
        d->rs[r] = (int32_t)rs;
        d->nhist[r] = (int32_t)(rs / LSA_CHUNK);
        d->nrec[r] = (int32_t)(L - rs);
        if (g->chunk_cap > 0 && d->nhist[r] > g->chunk_cap) return LSA_ERR_INVALID_ARG;
        if (g->recent_cap > 0 && d->nrec[r] > g->recent_cap) return LSA_ERR_INVALID_ARG;
        d->chunk_off[r] = g->chunk_cap > 0 ? (int64_t)r * g->chunk_cap : co;
        d->rec_off[r] = g->recent_cap > 0 ? (int64_t)r * g->recent_cap : ro;
        d->tile_off[r] = (int32_t)to;
        co += d->nhist[r];
        ro += d->nrec[r];
        to += (d->nhist[r] + 63) / 64;
    }
    if (g->chunk_cap > 0) co = (int64_t)g->batch * g->chunk_cap;
    if (g->recent_cap > 0) ro = (int64_t)g->batch * g->recent_cap;
    d->chunk_off[g->batch] = co;
    d->rec_off[g->batch] = ro;
    d->tile_off[g->batch] = (int32_t)to;
    if (co * LSA_CHUNK > INT32_MAX) return LSA_ERR_INVALID_ARG;  // token ids are int32
    return LSA_OK;
}

void geom_retile(GeomDev* d) {
    int32_t to = 0;
    for (int r = 0; r < d->B; ++r) {
        d->tile_off[r] = to;
        to += (d->nhist[r] + 63) / 64;
    }
    d->tile_off[d->B] = to;
}

extern "C" {

const char* lsa_status_str(lsa_status s) {
    switch (s) {
        case LSA_OK: return "ok";
        case LSA_ERR_INVALID_ARG: return "invalid argument";
        case LSA_ERR_UNSUPPORTED: return "unsupported dtype or shape";
        case LSA_ERR_CAPACITY: return "slot pool capacity exceeded";
        case LSA_ERR_WORKSPACE: return "workspace too small";
        case LSA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

lsa_status lsa_device_status(void* stream, uint32_t* flags) {
    hipStream_t s = (hipStream_t)stream;
    uint32_t* word = dev_err_word();
    if (!word) return LSA_ERR_HIP;
    uint32_t v = 0;
    LSA_HIP(hipStreamSynchronize(s));
    LSA_HIP(hipMemcpyAsync(&v, word, sizeof(v), hipMemcpyDeviceToHost, s));
    LSA_HIP(hipStreamSynchronize(s));
    if (v) {
        const uint32_t zero = 0;
        LSA_HIP(hipMemcpyAsync(word, &zero, sizeof(zero), hipMemcpyHostToDevice, s));
        LSA_HIP(hipStreamSynchronize(s));
    }
    if (flags) *flags = v;
    return v ? LSA_ERR_HIP : LSA_OK;
}

size_t lsa_score_ws_bytes(const lsa_geom* g, int32_t d) {
    if (!g || g->batch < 1 || d < 1) return 0;
    return align_up((size_t)g->batch * d * sizeof(float), 256);
}

lsa_status lsa_score_chunks(const lsa_geom* g, const void* q, lsa_dtype q_dt, const float* w,
                            const float* bias, int32_t H, int32_t d, const void* kic,
                            lsa_dtype kic_dt, const float* kic_scale, float* z, void* ws,
                            size_t ws_bytes, void* stream) {
    GeomDev gd;
    lsa_status st = geom_derive(g, &gd);
    if (st != LSA_OK) return st;
    if (!q || !w || !bias || !ws || !aligned16(ws)) return LSA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LSA_ERR_UNSUPPORTED;
    if (H < 1 || H > 256) return LSA_ERR_INVALID_ARG;
    if (q_dt != LSA_F32 && q_dt != LSA_BF16) return LSA_ERR_UNSUPPORTED;
    if (kic_dt != LSA_F32 && kic_dt != LSA_BF16 && kic_dt != LSA_FP8_E4M3FN)
        return LSA_ERR_UNSUPPORTED;
    const int64_t n = gd.chunk_off[gd.B];
    if (n > 0 && (!kic || !z || !aligned16(kic))) return LSA_ERR_INVALID_ARG;
    if (n > 0 && kic_dt == LSA_FP8_E4M3FN && !kic_scale) return LSA_ERR_INVALID_ARG;
    if (ws_bytes < lsa_score_ws_bytes(g, d)) return LSA_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    float* qbar = (float*)ws;
    LSA_HIP(launch_fuse_query(gd, q, q_dt, w, H, d, qbar, s));
    LSA_HIP(launch_score(gd, kic, kic_dt, kic_scale, qbar, bias, d, z, s));
    return LSA_OK;
}

lsa_status lsa_score_chunks_union(const lsa_geom* g, int32_t n_layers, const void* const* q,
                                  lsa_dtype q_dt, const float* const* w, const float* const* bias,
                                  int32_t H, int32_t d, const void* const* kic, lsa_dtype kic_dt,
                                  const float* const* kic_scale, float* z, void* ws, size_t ws_bytes,
                                  void* stream) {
    GeomDev gd;
    lsa_status st = geom_derive(g, &gd);
    if (st != LSA_OK) return st;
    if (n_layers < 1 || n_layers > LSA_MAX_LAYERS || !q || !w || !bias || !kic || !ws ||
        !aligned16(ws))
        return LSA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LSA_ERR_UNSUPPORTED;
    if (H < 1 || H > 256) return LSA_ERR_INVALID_ARG;
    if (q_dt != LSA_F32 && q_dt != LSA_BF16) return LSA_ERR_UNSUPPORTED;
    if (kic_dt != LSA_F32 && kic_dt != LSA_BF16 && kic_dt != LSA_FP8_E4M3FN)
        return LSA_ERR_UNSUPPORTED;
    const int64_t n = gd.chunk_off[gd.B];
    if (n > 0 && !z) return LSA_ERR_INVALID_ARG;
    if (n > 0 && kic_dt == LSA_FP8_E4M3FN && !kic_scale) return LSA_ERR_INVALID_ARG;
    for (int l = 0; l < n_layers; ++l) {
        if (!q[l] || !w[l] || !bias[l]) return LSA_ERR_INVALID_ARG;
        if (n > 0 && (!kic[l] || !aligned16(kic[l]))) return LSA_ERR_INVALID_ARG;
        if (n > 0 && kic_dt == LSA_FP8_E4M3FN && !kic_scale[l]) return LSA_ERR_INVALID_ARG;
    }
    if (ws_bytes < lsa_score_ws_bytes(g, d)) return LSA_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    float* qbar = (float*)ws;  // reused by each layer in stream order
    for (int l = 0; l < n_layers; ++l) {
        LSA_HIP(launch_fuse_query(gd, q[l], q_dt, w[l], H, d, qbar, s));
        LSA_HIP(launch_score(gd, kic[l], kic_dt, kic_dt == LSA_FP8_E4M3FN ? kic_scale[l] : nullptr, qbar,
                             bias[l], d, z, s, l > 0));
    }
    return LSA_OK;
}

lsa_status lsa_score_chunks_sigmoid(const lsa_geom* g, const void* q, lsa_dtype q_dt, const float* w,
                                    const float* bias, float theta, int32_t H, int32_t d,
                                    const void* kic, lsa_dtype kic_dt, const float* kic_scale, float* S,
                                    void* stream) {
    GeomDev gd;
    lsa_status st = geom_derive(g, &gd);
    if (st != LSA_OK) return st;
    if (!q || !w || !bias) return LSA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LSA_ERR_UNSUPPORTED;
    if (H < 1 || H * d > 8192) return LSA_ERR_INVALID_ARG;
    if (q_dt != LSA_F32 && q_dt != LSA_BF16) return LSA_ERR_UNSUPPORTED;
    if (kic_dt != LSA_F32 && kic_dt != LSA_BF16 && kic_dt != LSA_FP8_E4M3FN)
        return LSA_ERR_UNSUPPORTED;
    const int64_t n = gd.chunk_off[gd.B];
    if (n > 0 && (!kic || !S || !aligned16(kic) || !aligned16(q))) return LSA_ERR_INVALID_ARG;
    if (n > 0 && kic_dt == LSA_FP8_E4M3FN && !kic_scale) return LSA_ERR_INVALID_ARG;
    if (!(theta == theta)) return LSA_ERR_INVALID_ARG;
    LSA_HIP(launch_score_sig(gd, kic, kic_dt, kic_scale, q, q_dt, w, H, bias, theta, d, S,
                             (hipStream_t)stream));
    return LSA_OK;
}

lsa_status lsa_select_threshold(const lsa_geom* g, const float* z, float theta, int32_t* sel_ids,
                                int32_t* sel_cnt, void* stream) {
    GeomDev gd;
    lsa_status st = geom_derive(g, &gd);
    if (st != LSA_OK) return st;
    if (!sel_cnt) return LSA_ERR_INVALID_ARG;
    if (gd.chunk_off[gd.B] > 0 && (!z || !sel_ids)) return LSA_ERR_INVALID_ARG;
    if (theta != theta) return LSA_ERR_INVALID_ARG;  // NaN threshold
    LSA_HIP(launch_select(gd, z, theta, sel_ids, sel_cnt, (hipStream_t)stream));
    return LSA_OK;
}

lsa_status lsa_append_kv(const lsa_geom* g, const lsa_kv_layout* kv, const void* rows,
                         void* recent, void* stream) {
    GeomDev gd;
    lsa_status st = geom_derive(g, &gd);
    if (st != LSA_OK) return st;
    st = check_kv(kv);
    if (st != LSA_OK) return st;
    if (g->recent_cap <= 0 || !rows || !recent || kv->row_bytes % 16 != 0) return LSA_ERR_INVALID_ARG;
    if (!aligned16(rows) || !aligned16(recent)) return LSA_ERR_INVALID_ARG;
    for (int r = 0; r < gd.B; ++r)
        if (gd.nrec[r] < 1) return LSA_ERR_INVALID_ARG;
    LSA_HIP(launch_append_kv(gd, rows, kv->row_bytes, recent, (hipStream_t)stream));
    return LSA_OK;
}

lsa_status lsa_commit_chunk(const lsa_geom* g, const lsa_kv_layout* kv, const void* recent_src,
                            void* recent_dst, void* cold, lsa_dtype idx_dt, int32_t d,
                            const void* new_ikeys, const float* new_ikey_scale,
                            float* ikey_scale, const void* new_kic,
                            const float* new_kic_scale, void* kic, float* kic_scale,
                            int32_t* hist_out, void* stream) {
    GeomDev gd;
    lsa_status st = geom_derive(g, &gd);
    if (st != LSA_OK) return st;
    st = check_kv(kv);
    if (st != LSA_OK) return st;
    if (g->recent_cap <= 0 || g->chunk_cap <= 0 || !hist_out) return LSA_ERR_INVALID_ARG;
    if (idx_dt != LSA_F32 && idx_dt != LSA_BF16 && idx_dt != LSA_FP8_E4M3FN) return LSA_ERR_INVALID_ARG;
    const int64_t krb = (int64_t)d * esize(idx_dt);
    if (d < 1 || krb % 16 != 0 || kv->row_bytes % 16 != 0 || kv->page_bytes % 16 != 0 ||
        kv->ikey_off % 16 != 0 || kv->ikey_off < kv->row_bytes * LSA_CHUNK ||
        kv->ikey_off + krb * LSA_CHUNK > kv->page_bytes)
        return LSA_ERR_INVALID_ARG;
    if (!recent_src || !recent_dst || !cold || !new_ikeys || !new_kic || !kic) return LSA_ERR_INVALID_ARG;
    const bool fp8 = idx_dt == LSA_FP8_E4M3FN;
    if (fp8 && (!new_ikey_scale || !new_kic_scale || !ikey_scale || !kic_scale)) return LSA_ERR_INVALID_ARG;
    const size_t rb = (size_t)g->batch * g->recent_cap * kv->row_bytes;
    const uint8_t *a = (const uint8_t*)recent_src, *b = (const uint8_t*)recent_dst;
    if (a < b + rb && b < a + rb) return LSA_ERR_INVALID_ARG;  // the two buffers overlap
    int32_t nh[LSA_MAX_BATCH];
    for (int r = 0; r < gd.B; ++r) {
        const bool commit = gd.nrec[r] >= gd.W + LSA_CHUNK;
        if (commit && gd.nhist[r] + 1 > g->chunk_cap) return LSA_ERR_CAPACITY;
        nh[r] = gd.rs[r] + (commit ? LSA_CHUNK : 0);
    }
    LSA_HIP(launch_commit_chunk(gd, kv->row_bytes, kv->page_bytes, kv->ikey_off, recent_src, recent_dst,
                                cold, krb, new_ikeys, new_ikey_scale, ikey_scale, new_kic, new_kic_scale,
                                kic, kic_scale, fp8, (hipStream_t)stream));
    for (int r = 0; r < gd.B; ++r) hist_out[r] = nh[r];
    return LSA_OK;
}

lsa_status lsa_select_ranked(const lsa_geom* g, const void* keys, lsa_rank_kind kind,
                             const int32_t* m, int32_t* sel_ids, int32_t* sel_cnt, void* stream) {
    GeomDev gd;
    lsa_status st = geom_derive(g, &gd);
    if (st != LSA_OK) return st;
    if (!m || !sel_cnt) return LSA_ERR_INVALID_ARG;
    if (kind != LSA_RANK_SMALLEST_U32 && kind != LSA_RANK_LARGEST_F32) return LSA_ERR_INVALID_ARG;
    if (gd.chunk_off[gd.B] > 0 && (!keys || !sel_ids)) return LSA_ERR_INVALID_ARG;
    RankCounts rc;
    for (int r = 0; r < gd.B; ++r) {
        if (m[r] < 0) return LSA_ERR_INVALID_ARG;
        rc.m[r] = m[r];
    }
    LSA_HIP(launch_select_ranked(gd, keys, (int)kind, rc, sel_ids, sel_cnt, (hipStream_t)stream));
    return LSA_OK;
}

static size_t mass_ws_layout(const GeomDev& gd, int Hq, int n_steps, MassGeom* mg, size_t* o_lse,
                             size_t* o_rec) {
    mass_geom(gd, Hq, n_steps, mg);
    size_t off = align_up((size_t)mg->ml_total * 8, 256);
    *o_lse = off;
    off += align_up((size_t)gd.B * n_steps * Hq * 4, 256);
    *o_rec = off;
    off += align_up((size_t)mg->rc_total * 4 + 4, 256);
    return off;
}

size_t lsa_chunk_mass_ws_bytes(const lsa_geom* g, int32_t Hq, int32_t n_steps) {
    GeomDev gd;
    if (geom_derive(g, &gd) != LSA_OK || Hq < 1 || n_steps < 1) return 0;
    MassGeom mg;
    size_t a, b;
    return mass_ws_layout(gd, Hq, n_steps, &mg, &a, &b);
}

lsa_status lsa_chunk_attn_mass(const lsa_geom* g, const void* q, int32_t Hq, int32_t n_steps,
                               const lsa_kv_layout* kv, const void* pages,
                               const int32_t* page_table, const void* recent, float sm_scale,
                               float* mass, float* rec_mass, void* ws, size_t ws_bytes,
                               void* stream) {
    GeomDev gd;
    lsa_status st = geom_derive(g, &gd);
    if (st != LSA_OK) return st;
    st = check_kv(kv);
    if (st != LSA_OK) return st;
    if (kv->kv_dtype != LSA_BF16 || kv->Dk != 576 || kv->v_off != 0 || kv->row_bytes % 16 != 0 ||
        kv->page_bytes % 16 != 0)
        return LSA_ERR_UNSUPPORTED;
    if (Hq < 64 || Hq % 64 != 0 || n_steps < 1 || (int64_t)n_steps * Hq > 16384)
        return LSA_ERR_UNSUPPORTED;
    if (!q || !recent || !rec_mass || !ws || !(sm_scale == sm_scale)) return LSA_ERR_INVALID_ARG;
    if (gd.chunk_off[gd.B] > 0 && (!pages || !mass)) return LSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(recent) || !aligned16(ws) || (pages && !aligned16(pages)))
        return LSA_ERR_INVALID_ARG;
    MassGeom mg;
    size_t o_lse, o_rec;
    if (ws_bytes < mass_ws_layout(gd, Hq, n_steps, &mg, &o_lse, &o_rec)) return LSA_ERR_WORKSPACE;
    uint8_t* w = (uint8_t*)ws;
    LSA_HIP(launch_chunk_mass(gd, mg, q, Hq, n_steps, pages, kv->page_bytes, page_table, recent,
                              kv->row_bytes, sm_scale, mass, rec_mass, (float2*)w, (float*)(w + o_lse),
                              (float*)(w + o_rec), (hipStream_t)stream));
    return LSA_OK;
}

size_t lsa_refine_ws_bytes(const lsa_geom* g, int32_t k) {
    GeomDev gd;
    (void)k;
    if (geom_derive(g, &gd) != LSA_OK) return 0;
    const size_t plain = align_up((size_t)gd.chunk_off[gd.B] * LSA_CHUNK * sizeof(float), 256) + 256;
    const size_t band = band_ws_bytes(gd);
    return plain > band ? plain : band;
}

lsa_status lsa_topk_refine(const lsa_geom* g, const int32_t* sel_ids, const int32_t* sel_cnt,
                           const void* pages, int64_t page_bytes, int64_t ikey_off,
                           const int32_t* page_table, lsa_dtype idx_dt, const float* ikey_scale,
                           const void* q, lsa_dtype q_dt, const float* w, int32_t H, int32_t d,
                           int32_t k, int32_t* topk_idx, int32_t* topk_cnt, void* ws,
                           size_t ws_bytes, void* stream) {
    GeomDev gd;
    lsa_status st = geom_derive(g, &gd);
    if (st != LSA_OK) return st;
    if (!sel_cnt || !q || !w || !topk_idx || !topk_cnt || !ws || !aligned16(ws)) return LSA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LSA_ERR_UNSUPPORTED;
    if (H < 1 || H > 128 || k < 1) return LSA_ERR_INVALID_ARG;
    // the VALU refine (every case the matrix-core path does not take) keeps the queries in LDS
    if (!band_supported(idx_dt, q_dt, H, d) && ((int64_t)H * d + H) * 4 > 65536)
        return LSA_ERR_UNSUPPORTED;
    if (q_dt != LSA_F32 && q_dt != LSA_BF16) return LSA_ERR_UNSUPPORTED;
    if (idx_dt != LSA_F32 && idx_dt != LSA_BF16 && idx_dt != LSA_FP8_E4M3FN)
        return LSA_ERR_UNSUPPORTED;
    const int64_t n = gd.chunk_off[gd.B];
    if (n > 0) {
        if (!sel_ids || !pages || !aligned16(pages)) return LSA_ERR_INVALID_ARG;
        if (page_bytes < ikey_off + (int64_t)LSA_CHUNK * d * esize(idx_dt)) return LSA_ERR_INVALID_ARG;
        if (page_bytes % 16 || ikey_off % 16 || ikey_off < 0) return LSA_ERR_INVALID_ARG;
        if (idx_dt == LSA_FP8_E4M3FN && !ikey_scale) return LSA_ERR_INVALID_ARG;
    }
    if (ws_bytes < lsa_refine_ws_bytes(g, k)) return LSA_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    if (n > 0 && band_supported(idx_dt, q_dt, H, d)) {
        LSA_HIP(launch_refine_band(gd, sel_ids, sel_cnt, pages, page_bytes, ikey_off, page_table,
                                   idx_dt, ikey_scale, nullptr, nullptr, nullptr, q, w, H, d, k,
                                   topk_idx, topk_cnt, ws, false, s));
        return LSA_OK;
    }
    float* scores = (float*)ws;
    if (n > 0)
        LSA_HIP(launch_refine(gd, sel_ids, sel_cnt, pages, page_bytes, ikey_off, page_table, idx_dt,
                              ikey_scale, q, q_dt, w, H, d, scores, 0, s));
    LSA_HIP(launch_topk(gd, sel_ids, sel_cnt, scores, k, topk_idx, topk_cnt, s));
    return LSA_OK;
}

size_t lsa_attn_ws_bytes(const lsa_geom* g, const lsa_kv_layout* kv, int32_t Hq, int32_t k,
                         int32_t n_splits) {
    GeomDev gd;
    AttnPlan p;
    if (geom_derive(g, &gd) != LSA_OK || check_kv(kv) != LSA_OK || k < 1 || Hq < 1) return 0;
    if (attn_plan(gd, kv, Hq, k, n_splits, &p) != LSA_OK) return 0;
    return p.part_o_bytes + p.part_ml_bytes;
}

// Argument checks and plan of both attention entry points (ws is checked
// by the caller).
static lsa_status attn_args(const lsa_geom* g, const void* q, int32_t Hq, const lsa_kv_layout* kv,
                            const void* pages, const void* recent, const int32_t* topk_idx,
                            const int32_t* topk_cnt, int32_t k, float sm_scale, void* out,
                            int32_t n_splits, GeomDev* gd, AttnPlan* plan) {
    lsa_status st = geom_derive(g, gd);
    if (st != LSA_OK) return st;
    st = check_kv(kv);
    if (st != LSA_OK) return st;
    if (!q || !recent || !topk_idx || !topk_cnt || !out || Hq < 1 || k < 1) return LSA_ERR_INVALID_ARG;
    if (gd->chunk_off[gd->B] > 0 && !pages) return LSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(recent) || (pages && !aligned16(pages))) return LSA_ERR_INVALID_ARG;
    if (!(sm_scale == sm_scale) || n_splits < 0) return LSA_ERR_INVALID_ARG;
    return attn_plan(*gd, kv, Hq, k, n_splits, plan);
}

lsa_status lsa_sparse_decode_attn(const lsa_geom* g, const void* q, int32_t Hq,
                                  const lsa_kv_layout* kv, const void* pages,
                                  const int32_t* page_table, const void* recent,
                                  const int32_t* topk_idx, const int32_t* topk_cnt, int32_t k,
                                  float sm_scale, void* out, float* lse, int32_t n_splits,
                                  void* ws, size_t ws_bytes, void* stream) {
    GeomDev gd;
    AttnPlan plan;
    lsa_status st = attn_args(g, q, Hq, kv, pages, recent, topk_idx, topk_cnt, k, sm_scale, out,
                              n_splits, &gd, &plan);
    if (st != LSA_OK) return st;
    if (!ws || !aligned16(ws)) return LSA_ERR_INVALID_ARG;
    if (ws_bytes < plan.part_o_bytes + plan.part_ml_bytes) return LSA_ERR_WORKSPACE;
    LSA_HIP(launch_attn(gd, plan, q, Hq, *kv, pages, page_table, recent, topk_idx, topk_cnt, k,
                        sm_scale, out, lse, ws, (hipStream_t)stream));
    return LSA_OK;
}

size_t lsa_attn_noalloc_max_bytes(void) { return attn_scratch_bytes(); }

lsa_status lsa_sparse_decode_attn_noalloc(const lsa_geom* g, const void* q, int32_t Hq,
                                          const lsa_kv_layout* kv, const void* pages,
                                          const int32_t* page_table, const void* recent,
                                          const int32_t* topk_idx, const int32_t* topk_cnt,
                                          int32_t k, float sm_scale, void* out, float* lse,
                                          int32_t n_splits, void* stream) {
    GeomDev gd;
    AttnPlan plan;
    lsa_status st = attn_args(g, q, Hq, kv, pages, recent, topk_idx, topk_cnt, k, sm_scale, out,
                              n_splits, &gd, &plan);
    if (st != LSA_OK) return st;
    if (plan.part_o_bytes + plan.part_ml_bytes > attn_scratch_bytes()) return LSA_ERR_WORKSPACE;
    void* ws = attn_scratch();  // the device address of this GPU's array
    if (!ws) return LSA_ERR_HIP;
    LSA_HIP(launch_attn(gd, plan, q, Hq, *kv, pages, page_table, recent, topk_idx, topk_cnt, k,
                        sm_scale, out, lse, ws, (hipStream_t)stream));
    return LSA_OK;
}

}  // extern "C"
