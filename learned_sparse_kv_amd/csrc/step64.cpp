// The window pipeline (lsa_step64).
//
// The memory indexer fires every 64 generation steps and predicts which
// history chunks the next 64 steps need; only those are moved from the CPU
// cold pool into GPU memory (cjcn.com.cn explainer, section 二; gist.science
// summary, section 2.1 "Periodische Triggerung").  Here the prediction runs
// one window ahead: while window m's decode steps run on the main stream,
// window m+1 is scored and selected (main stream, before the steps), its
// selection comes back to the host, and its missing chunks are copied on the
// copy stream into slots that window m does not read.  Window m+1 waits for
// that copy only when it starts.  Two page tables and two selection buffers
// alternate between windows.
#include <hip/hip_runtime.h>

#include <cstring>
#include <new>

#include "lsa_internal.h"

struct lsa_ctx {
    lsa_ctx_desc d;
    GeomDev g;
    AttnPlan plan;
    int64_t nh = 0;
    float* qbar = nullptr;
    uint64_t* tmask = nullptr;   // per tile of 64 chunks: the mask of z > theta
    int32_t* tcount = nullptr;   // and its count
    float* z = nullptr;
    int32_t* sel[2] = {nullptr, nullptr};
    int32_t* cnt[2] = {nullptr, nullptr};
    float* scores = nullptr;
    bool band_clean = false;  // band workspace histograms known to be zero
    int32_t* topk_tmp = nullptr;
    int32_t* tcnt_tmp = nullptr;
    void* attn_ws = nullptr;
    int32_t* pt[2] = {nullptr, nullptr};
    int32_t* sel_slot = nullptr;  // pages of the running window's selected chunks
    float* sel_scale = nullptr;   // and their index-key scales
    float* kn2 = nullptr;         // |key|^2 of their tokens
    int32_t* h_sel[2] = {nullptr, nullptr};
    int32_t* h_cnt[2] = {nullptr, nullptr};
    uint32_t* h_err = nullptr;   // pinned [3]: the device error word after each window, 0
    uint32_t* d_err = nullptr;   // the device error word
    hipEvent_t ev_sel = nullptr, ev_win[2] = {nullptr, nullptr}, ev_fetch[2] = {nullptr, nullptr};
    int cur = 0;
    bool primed = false;
    bool have_next = false;
    // growing context: request r's recent rows start at row rec_first[r] of
    // its recent_cap rows; no window holds more than rmax of them
    bool growing = false;
    int64_t recent_cap = 0;
    int32_t rmax = 0;
    int32_t rec_first[LSA_MAX_BATCH] = {};
};

namespace {

int64_t esz(lsa_dtype t) { return t == LSA_F32 ? 4 : (t == LSA_BF16 ? 2 : 1); }

struct Carve {
    size_t off = 0;
    size_t take(size_t bytes) {
        const size_t o = off;
        off += align_up(bytes ? bytes : 1, 256);
        return o;
    }
};

// Growing context: the most recent rows a request holds during a window.
// A window starts with at most max(W + 63, R_r) rows (a request at or past
// W + 64 at a window's end commits a chunk) and adds at most 64.
int32_t grow_rmax(const GeomDev& g) {
    int32_t a = g.W + 63;
    for (int r = 0; r < g.B; ++r) a = g.nrec[r] > a ? g.nrec[r] : a;
    return a + 64;
}

// The attention plan covers every recent length the context reaches.
lsa_status ctx_plan(const lsa_ctx_desc* d, const GeomDev& g, AttnPlan* plan) {
    if (!d->growing) return attn_plan(g, &d->kv, d->Hq, d->k, 0, plan);
    GeomDev gp = g;
    const int32_t rm = grow_rmax(g);
    for (int r = 0; r < g.B; ++r) gp.nrec[r] = rm;
    return attn_plan(gp, &d->kv, d->Hq, d->k, 0, plan);
}

// Tiles of 64 history chunks the scoring may cover: the requests' chunk
// capacities when the history grows, else their chunk counts.
size_t tile_cap(const GeomDev& g, const lsa_ctx_desc* d) {
    if (d->geom.chunk_cap > 0) return (size_t)g.B * ((d->geom.chunk_cap + 63) / 64);
    return (size_t)g.tile_off[g.B];
}

// Workspace layout; returns total bytes (0 on invalid description).
size_t layout(const lsa_ctx_desc* d, GeomDev* g, AttnPlan* plan, size_t offs[16]) {
    if (!d) return 0;
    if (geom_derive(&d->geom, g) != LSA_OK) return 0;
    if (ctx_plan(d, *g, plan) != LSA_OK) return 0;
    const int64_t nh = g->chunk_off[g->B];
    const int B = g->B;
    Carve c;
    offs[0] = c.take((tile_cap(*g, d) + 1) * 12);      // tile masks, then tile counts
    offs[1] = c.take((size_t)nh * 4);                   // z
    offs[2] = c.take((size_t)nh * 4);                   // sel[0]
    offs[3] = c.take((size_t)nh * 4);                   // sel[1]
    offs[4] = c.take((size_t)B * 4);                    // cnt[0]
    offs[5] = c.take((size_t)B * 4);                    // cnt[1]
    const size_t plain = (size_t)nh * LSA_CHUNK * 4, band = band_ws_bytes(*g);
    offs[6] = c.take(plain > band ? plain : band);      // refine scores / band scratch
    offs[7] = c.take((size_t)B * d->k * 4);             // top-k scratch
    offs[8] = c.take((size_t)B * 4);                    // top-k counts scratch
    offs[9] = c.take(plan->part_o_bytes + plan->part_ml_bytes);  // attention partials
    offs[10] = c.take((size_t)nh * 4);                  // page table 0
    offs[11] = c.take((size_t)nh * 4);                  // page table 1
    offs[12] = c.take((size_t)nh * 4);                  // pages of the selected chunks
    offs[13] = c.take((size_t)nh * 4);                  // their scales
    offs[14] = c.take((size_t)nh * LSA_CHUNK * 4);      // |key|^2 of their tokens
    offs[15] = c.take((size_t)B * d->d * 4);            // fused queries
    return c.off;
}

int n_layers_of(const lsa_ctx_desc& d) { return d.n_layers > 1 ? d.n_layers : 1; }

// Scores every indexer layer into z (later layers keep the per-chunk maximum,
// so z > theta exactly when some layer's logit is), then selects.
lsa_status score_select(lsa_ctx* x, const GeomDev& g, const lsa_trigger_in* t, int buf,
                        hipStream_t s) {
    const lsa_ctx_desc& d = x->d;
    const int nl = n_layers_of(d);
    if (!t) return LSA_ERR_INVALID_ARG;
    for (int l = 0; l < nl; ++l) {
        if (!t[l].q || !t[l].w || !t[l].bias) return LSA_ERR_INVALID_ARG;
        if (x->nh > 0 && !t[l].kic) return LSA_ERR_INVALID_ARG;
        if (x->nh > 0 && d.idx_dt == LSA_FP8_E4M3FN && !t[l].kic_scale) return LSA_ERR_INVALID_ARG;
    }
    // the last layer's launch records the tile masks of the union's logits
    for (int l = 0; l < nl; ++l) {
        const bool last = l == nl - 1;
        if (launch_fuse_query(g, t[l].q, d.q_dt, t[l].w, d.H, d.d, x->qbar, s) != hipSuccess)
            return LSA_ERR_HIP;
        if (launch_score(g, t[l].kic, d.idx_dt, t[l].kic_scale, x->qbar, t[l].bias, d.d, x->z, s,
                         l > 0, d.theta, last ? x->tmask : nullptr,
                         last ? x->tcount : nullptr) != hipSuccess)
            return LSA_ERR_HIP;
    }
    if (launch_select_tiles(g, x->tmask, x->tcount, x->sel[buf], x->cnt[buf], s) != hipSuccess)
        return LSA_ERR_HIP;
    if (x->nh > 0 && hipMemcpyAsync(x->h_sel[buf], x->sel[buf], (size_t)x->nh * 4,
                                    hipMemcpyDeviceToHost, s) != hipSuccess)
        return LSA_ERR_HIP;
    if (hipMemcpyAsync(x->h_cnt[buf], x->cnt[buf], (size_t)g.B * 4, hipMemcpyDeviceToHost, s) !=
        hipSuccess)
        return LSA_ERR_HIP;
    if (hipEventRecord(x->ev_sel, s) != hipSuccess) return LSA_ERR_HIP;
    return LSA_OK;
}

}  // namespace

extern "C" {

size_t lsa_ctx_ws_bytes(const lsa_ctx_desc* desc) {
    GeomDev g;
    AttnPlan p;
    size_t offs[16];
    return layout(desc, &g, &p, offs);
}

lsa_status lsa_ctx_create(lsa_ctx** ctx, const lsa_ctx_desc* desc) {
    if (!ctx || !desc) return LSA_ERR_INVALID_ARG;
    *ctx = nullptr;
    GeomDev g;
    AttnPlan plan;
    size_t offs[16];
    lsa_status st = geom_derive(&desc->geom, &g);
    if (st != LSA_OK) return st;
    if (desc->d != 64 && desc->d != 128) return LSA_ERR_UNSUPPORTED;
    if (desc->H < 1 || desc->H > 128 || desc->k < 1 || desc->Hq < 1) return LSA_ERR_INVALID_ARG;
    if (desc->n_layers < 0 || desc->n_layers > LSA_MAX_LAYERS) return LSA_ERR_INVALID_ARG;
    if (desc->q_dt != LSA_F32 && desc->q_dt != LSA_BF16) return LSA_ERR_UNSUPPORTED;
    if (!desc->pool || !desc->recent || !desc->ws || ((uintptr_t)desc->ws & 15u))
        return LSA_ERR_INVALID_ARG;
    if (desc->idx_dt == LSA_FP8_E4M3FN && !desc->ikey_scale && g.chunk_off[g.B] > 0)
        return LSA_ERR_INVALID_ARG;
    if (desc->kv.ikey_off % 16 || desc->kv.page_bytes % 16) return LSA_ERR_INVALID_ARG;
    if (!band_supported(desc->idx_dt, desc->q_dt, desc->H, desc->d) &&
        ((int64_t)desc->H * desc->d + desc->H) * 4 > 65536)
        return LSA_ERR_UNSUPPORTED;
    if (desc->kv.ikey_off < (int64_t)LSA_CHUNK * desc->kv.row_bytes ||
        desc->kv.page_bytes < desc->kv.ikey_off + (int64_t)LSA_CHUNK * desc->d * esz(desc->idx_dt))
        return LSA_ERR_INVALID_ARG;
    if (lsa_pool_page_bytes(desc->pool) != desc->kv.page_bytes ||
        lsa_pool_batch(desc->pool) != g.B)
        return LSA_ERR_INVALID_ARG;
    int32_t rmax = 0;
    if (desc->growing) {
        // fixed capacities per request, and room for the recent rows to
        // slide a whole window's length before they move back
        if (desc->geom.chunk_cap <= 0 || desc->geom.recent_cap <= 0) return LSA_ERR_INVALID_ARG;
        rmax = grow_rmax(g);
        if ((int64_t)desc->geom.recent_cap < 2 * (int64_t)rmax) return LSA_ERR_INVALID_ARG;
    }
    st = ctx_plan(desc, g, &plan);
    if (st != LSA_OK) return st;
    const size_t need = layout(desc, &g, &plan, offs);
    if (need == 0) return LSA_ERR_INVALID_ARG;
    if (desc->ws_bytes < need) return LSA_ERR_WORKSPACE;
    lsa_ctx* x = new (std::nothrow) lsa_ctx();
    if (!x) return LSA_ERR_INVALID_ARG;
    x->d = *desc;
    x->g = g;
    x->plan = plan;
    x->nh = g.chunk_off[g.B];
    x->growing = desc->growing != 0;
    x->recent_cap = desc->geom.recent_cap;
    x->rmax = rmax;
    uint8_t* base = (uint8_t*)desc->ws;
    x->qbar = (float*)(base + offs[15]);
    x->tmask = (uint64_t*)(base + offs[0]);
    x->tcount = (int32_t*)(base + offs[0] + (tile_cap(g, desc) + 1) * 8);
    x->z = (float*)(base + offs[1]);
    x->sel[0] = (int32_t*)(base + offs[2]);
    x->sel[1] = (int32_t*)(base + offs[3]);
    x->cnt[0] = (int32_t*)(base + offs[4]);
    x->cnt[1] = (int32_t*)(base + offs[5]);
    x->scores = (float*)(base + offs[6]);
    x->topk_tmp = (int32_t*)(base + offs[7]);
    x->tcnt_tmp = (int32_t*)(base + offs[8]);
    x->attn_ws = base + offs[9];
    x->pt[0] = (int32_t*)(base + offs[10]);
    x->pt[1] = (int32_t*)(base + offs[11]);
    x->sel_slot = (int32_t*)(base + offs[12]);
    x->sel_scale = (float*)(base + offs[13]);
    x->kn2 = (float*)(base + offs[14]);
    const size_t nhb = (size_t)(x->nh > 0 ? x->nh : 1) * 4;
    bool ok = true;
    for (int i = 0; i < 2 && ok; ++i) {
        ok = hipHostMalloc((void**)&x->h_sel[i], nhb, hipHostMallocDefault) == hipSuccess &&
             hipHostMalloc((void**)&x->h_cnt[i], (size_t)g.B * 4, hipHostMallocDefault) == hipSuccess &&
             hipEventCreateWithFlags(&x->ev_win[i], hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&x->ev_fetch[i], hipEventDisableTiming) == hipSuccess;
    }
    ok = ok && hipEventCreateWithFlags(&x->ev_sel, hipEventDisableTiming) == hipSuccess &&
         hipHostMalloc((void**)&x->h_err, 3 * sizeof(uint32_t), hipHostMallocDefault) == hipSuccess &&
         (x->d_err = dev_err_word()) != nullptr;
    if (ok) x->h_err[0] = x->h_err[1] = x->h_err[2] = 0;
    if (!ok) {
        lsa_ctx_destroy(x);
        return LSA_ERR_HIP;
    }
    *ctx = x;
    return LSA_OK;
}

void lsa_ctx_destroy(lsa_ctx* x) {
    if (!x) return;
    for (int i = 0; i < 2; ++i) {
        if (x->ev_win[i]) (void)hipEventSynchronize(x->ev_win[i]);
        if (x->ev_fetch[i]) (void)hipEventSynchronize(x->ev_fetch[i]);
    }
    for (int i = 0; i < 2; ++i) {
        if (x->h_sel[i]) (void)hipHostFree(x->h_sel[i]);
        if (x->h_cnt[i]) (void)hipHostFree(x->h_cnt[i]);
        if (x->ev_win[i]) (void)hipEventDestroy(x->ev_win[i]);
        if (x->ev_fetch[i]) (void)hipEventDestroy(x->ev_fetch[i]);
    }
    if (x->ev_sel) (void)hipEventDestroy(x->ev_sel);
    if (x->h_err) (void)hipHostFree(x->h_err);
    delete x;
}

lsa_status lsa_ctx_prime(lsa_ctx* x, const lsa_trigger_in* first, void* main_stream,
                         void* copy_stream, lsa_window_out* out) {
    if (!x || !first) return LSA_ERR_INVALID_ARG;
    hipStream_t ms = (hipStream_t)main_stream;
    x->cur = 0;
    lsa_status st = score_select(x, x->g, first, 0, ms);
    if (st != LSA_OK) return st;
    if (hipEventRecord(x->ev_win[0], ms) != hipSuccess || hipEventRecord(x->ev_win[1], ms) != hipSuccess)
        return LSA_ERR_HIP;
    if (hipEventSynchronize(x->ev_sel) != hipSuccess) return LSA_ERR_HIP;
    lsa_gather_stats gs{};
    st = lsa_gather_kv(x->d.pool, x->h_sel[0], x->h_cnt[0], nullptr, nullptr, x->pt[0],
                       copy_stream, nullptr, x->ev_fetch[0], &gs);
    if (st != LSA_OK) return st;
    if (out) {
        out->stats = gs;
        if (out->sel_cnt) std::memcpy(out->sel_cnt, x->h_cnt[0], (size_t)x->g.B * 4);
    }
    x->primed = true;
    x->have_next = true;
    return LSA_OK;
}

lsa_status lsa_step64(lsa_ctx* x, const lsa_window_in* in, lsa_window_out* out,
                      void* main_stream, void* copy_stream) {
    if (!x || !in || !out || !out->out) return LSA_ERR_INVALID_ARG;
    if (!x->primed || !x->have_next) return LSA_ERR_INVALID_ARG;  // no selected window to run
    if (in->steps < 1 || in->steps > 64 || !in->q_refine || !in->w_refine || !in->q_attn)
        return LSA_ERR_INVALID_ARG;
    const lsa_ctx_desc& d = x->d;
    GeomDev& g = x->g;
    hipStream_t ms = (hipStream_t)main_stream;
    const int cur = x->cur, nxt = cur ^ 1;
    const bool fp8 = d.idx_dt == LSA_FP8_E4M3FN;
    const int64_t key_row_bytes = (int64_t)d.d * esz(d.idx_dt);

    // growing context: who commits a chunk in this window (checked before
    // anything is launched), and the history the next trigger scores
    CommitSet commit{};
    GeomDev gs = g;
    if (x->growing) {
        if (!in->new_rows || !in->commit_ikeys || (fp8 && !in->commit_ikey_scale))
            return LSA_ERR_INVALID_ARG;
        for (int r = 0; r < g.B; ++r) {
            if (g.nrec[r] + in->steps > x->rmax) return LSA_ERR_INVALID_ARG;  // cannot happen
            commit.on[r] = g.nrec[r] + in->steps >= g.W + LSA_CHUNK;
            if (commit.on[r] && g.chunk_off[r] + g.nhist[r] + 1 > g.chunk_off[r + 1])
                return LSA_ERR_CAPACITY;
            gs.nhist[r] += commit.on[r];
        }
        geom_retile(&gs);
    }

    if (hipStreamWaitEvent(ms, x->ev_fetch[cur], 0) != hipSuccess) return LSA_ERR_HIP;
    if (x->growing) {
        // a window that would run past the end of a request's recent area
        // starts with its rows moved back to the area's start (the ranges do
        // not overlap: the area holds two windows' worth of rows)
        RecentMoves mv{};
        bool any_move = false, any_commit = false;
        for (int r = 0; r < g.B; ++r) {
            any_commit |= commit.on[r] != 0;
            if (x->rec_first[r] + g.nrec[r] + in->steps > x->recent_cap) {
                mv.src[r] = g.rec_off[r];
                mv.dst[r] = (int64_t)r * x->recent_cap;
                mv.n[r] = g.nrec[r];
                x->rec_first[r] = 0;
                g.rec_off[r] = mv.dst[r];
                any_move = true;
            }
        }
        if (any_move &&
            launch_compact_recent(g.B, mv, d.kv.row_bytes, (void*)d.recent, ms) != hipSuccess)
            return LSA_ERR_HIP;
        if (any_commit &&
            launch_commit_page(g, commit, d.kv.row_bytes, d.kv.page_bytes, d.kv.ikey_off, d.recent,
                               lsa_pool_cold(d.pool), key_row_bytes, in->commit_ikeys,
                               fp8 ? in->commit_ikey_scale : nullptr, (float*)d.ikey_scale,
                               ms) != hipSuccess)
            return LSA_ERR_HIP;
    }
    const bool band = band_supported(d.idx_dt, d.q_dt, d.H, d.d);
    if (band && (launch_resolve_sel(g, x->sel[cur], x->cnt[cur], x->pt[cur], d.ikey_scale,
                                    x->sel_slot, x->sel_scale, ms) != hipSuccess ||
                 launch_key_norm2(g, x->cnt[cur], x->sel_slot, lsa_pool_slots(d.pool),
                                  d.kv.page_bytes, d.kv.ikey_off, d.idx_dt, d.d, x->kn2,
                                  ms) != hipSuccess))
        return LSA_ERR_HIP;
    if (in->next) {
        lsa_status st = score_select(x, gs, in->next, nxt, ms);
        if (st != LSA_OK) return st;
    }
    int groups = 0;
    for (int r = 0; r < g.B; ++r) groups += (x->h_cnt[cur][r] + 3) / 4;
    const size_t qr_step = (size_t)g.B * d.H * d.d * esz(d.q_dt);
    const size_t qa_step = (size_t)g.B * d.Hq * d.kv.Dk * esz(d.kv.kv_dtype);
    const size_t o_step = (size_t)g.B * d.Hq * d.kv.Dv * esz(d.kv.kv_dtype);
    for (int j = 0; j < in->steps; ++j) {
        int32_t* tk = out->topk_idx ? out->topk_idx + (size_t)j * g.B * d.k : x->topk_tmp;
        int32_t* tc = out->topk_cnt ? out->topk_cnt + (size_t)j * g.B : x->tcnt_tmp;
        const uint8_t* qr = (const uint8_t*)in->q_refine + j * qr_step;
        const float* wr = in->w_refine + (size_t)j * g.B * d.H;
        // the step's token joins the recent region first: its row is written
        // by the band's fine-histogram pass (before attention reads the
        // recent rows), else by a copy kernel of its own
        AppendRow app;
        const bool app_band = x->growing && groups > 0 && band && d.kv.row_bytes % 16 == 0 &&
                              d.kv.row_bytes <= 16 * 256;
        if (x->growing) {
            for (int r = 0; r < g.B; ++r) {
                ++g.L[r];
                ++g.nrec[r];
            }
            const uint8_t* rows = (const uint8_t*)in->new_rows + (size_t)j * g.B * d.kv.row_bytes;
            if (app_band) {
                app.rows = rows;
                app.recent = (uint8_t*)d.recent;
                app.n16 = (int32_t)(d.kv.row_bytes / 16);
            } else if (launch_append_kv(g, rows, d.kv.row_bytes, (void*)d.recent, ms) != hipSuccess) {
                return LSA_ERR_HIP;
            }
        }
        if (groups > 0 && band) {
            const bool clean = x->band_clean;
            x->band_clean = false;  // until the chain is queued whole
            if (launch_refine_band(g, x->sel[cur], x->cnt[cur], lsa_pool_slots(d.pool),
                                   d.kv.page_bytes, d.kv.ikey_off, x->pt[cur], d.idx_dt,
                                   d.ikey_scale, x->sel_slot, x->sel_scale, x->kn2, qr, wr, d.H,
                                   d.d, d.k, tk, tc, x->scores, clean, ms, app) != hipSuccess)
                return LSA_ERR_HIP;
            x->band_clean = true;
        } else {
            if (groups > 0 &&
                launch_refine(g, x->sel[cur], x->cnt[cur], lsa_pool_slots(d.pool), d.kv.page_bytes,
                              d.kv.ikey_off, x->pt[cur], d.idx_dt, d.ikey_scale, qr, d.q_dt, wr,
                              d.H, d.d, x->scores, groups, ms) != hipSuccess)
                return LSA_ERR_HIP;
            if (launch_topk(g, x->sel[cur], x->cnt[cur], x->scores, d.k, tk, tc, ms) != hipSuccess)
                return LSA_ERR_HIP;
        }
        if (launch_attn(g, x->plan, (const uint8_t*)in->q_attn + j * qa_step, d.Hq, d.kv,
                        lsa_pool_slots(d.pool), x->pt[cur], d.recent, tk, tc, d.k, d.sm_scale,
                        (uint8_t*)out->out + j * o_step,
                        out->lse ? out->lse + (size_t)j * g.B * d.Hq : nullptr, x->attn_ws,
                        ms) != hipSuccess)
            return LSA_ERR_HIP;
    }
    // the device error word as this window leaves it, taken over (and
    // cleared) so that it reports this window only; the next call reads it
    // once its wait below has passed this window
    if (hipMemcpyAsync(&x->h_err[cur], x->d_err, sizeof(uint32_t), hipMemcpyDeviceToHost, ms) !=
            hipSuccess ||
        hipMemcpyAsync(x->d_err, &x->h_err[2], sizeof(uint32_t), hipMemcpyHostToDevice, ms) != hipSuccess)
        return LSA_ERR_HIP;
    if (hipEventRecord(x->ev_win[cur], ms) != hipSuccess) return LSA_ERR_HIP;
    if (x->growing) {
        // the committed chunks leave the recent region: from the next window
        // on they are history, attended when a trigger selects them
        for (int r = 0; r < g.B; ++r) {
            if (!commit.on[r]) continue;
            g.rs[r] += LSA_CHUNK;
            g.nhist[r] += 1;
            g.nrec[r] -= LSA_CHUNK;
            g.rec_off[r] += LSA_CHUNK;
            x->rec_first[r] += LSA_CHUNK;
        }
        geom_retile(&g);
    }
    bool dev_err = false;
    if (in->next) {
        if (hipEventSynchronize(x->ev_sel) != hipSuccess) return LSA_ERR_HIP;
        // ev_sel follows the previous window on the main stream
        dev_err = x->h_err[nxt] != 0;
        if (x->growing) {
            lsa_status st = pool_grow(x->d.pool, gs);
            if (st != LSA_OK) return st;
        }
        lsa_gather_stats fs{};
        lsa_status st = lsa_gather_kv(x->d.pool, x->h_sel[nxt], x->h_cnt[nxt], x->h_sel[cur],
                                      x->h_cnt[cur], x->pt[nxt], copy_stream, x->ev_win[nxt],
                                      x->ev_fetch[nxt], &fs);
        if (st != LSA_OK) return st;
        out->stats = fs;
        if (out->sel_cnt) std::memcpy(out->sel_cnt, x->h_cnt[nxt], (size_t)g.B * 4);
        x->cur = nxt;
        x->have_next = true;
    } else {
        x->have_next = false;
    }
    return dev_err ? LSA_ERR_HIP : LSA_OK;
}

lsa_status lsa_ctx_state(const lsa_ctx* x, int32_t* seq_len, int32_t* hist_tokens,
                         int32_t* recent_first) {
    if (!x) return LSA_ERR_INVALID_ARG;
    for (int r = 0; r < x->g.B; ++r) {
        if (seq_len) seq_len[r] = x->g.L[r];
        if (hist_tokens) hist_tokens[r] = x->g.rs[r];
        if (recent_first) recent_first[r] = x->rec_first[r];
    }
    return LSA_OK;
}

}  // extern "C"
