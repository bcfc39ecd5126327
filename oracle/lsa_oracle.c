/*
 * CPU oracle for the Lookahead Sparse Attention (LSA) decode hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code with the HIP library.
 *
 * It follows the method as the pages describe it ("FlashMemory-DeepSeek-V4:
 * Lightning Index Ultra-Long Context via Lookahead Sparse Attention"):
 *   - every 64 decode steps the memory indexer scores every history chunk's
 *     compressed index key against the current query state with a
 *     head-fused matching score passed through a sigmoid (gist.science
 *     summary, section 2.1 "Scoring-Mechanismus"; cjcn.com.cn explainer,
 *     section 二);
 *   - chunks whose score exceeds 0.5 are fetched (same passages: a fixed
 *     threshold replaces a fixed top-k, so the count varies);
 *   - inside that candidate set the lightning indexer (ReLU-weighted head
 *     sum) takes a top-k of tokens (gist.science 2.1 "Gestufte Selektion";
 *     cjcn.com.cn section 二, second-stage selection);
 *   - core attention runs over the selected tokens plus the always-resident
 *     most recent window (cjcn.com.cn section 二, last paragraph, and
 *     section 五: every scheme keeps the recent 8K).
 *
 * Where the pages leave a step open, the reading taken is the plainest one:
 *   score logit  z_c = b + s_c * sum_h w_h (q_h . k_c)       (one KIComp row
 *                per chunk shared by all heads, so this is a dot product with
 *                the fused query qbar = sum_h w_h q_h);
 *   select       sigmoid(z_c) > 0.5  <=>  z_c > 0 (strict);
 *   refine       I_s = s_chunk * sum_h w_h * ReLU(q_h . k_s);
 *   top-k        the min(k, |T|) largest I_s, ties to the lower token index,
 *                emitted in ascending token order;
 *   attention    softmax(sm * q_h K_A^T) V_A over A = top-k U [rs, L).
 *
 * Arithmetic.  Scores that decide a selection are computed in fp32 in the
 * plain sequential order written below (IEEE fmaf, round to nearest even,
 * no flush of subnormals, no other contraction; build with
 * -ffp-contract=off and without fast-math).  Attention is computed in fp64
 * from the decoded inputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { O_F32 = 0, O_BF16 = 1, O_FP8 = 2 };

/* ------------------------------------------------------------------ */
/* O1: decoding of stored values                                       */
/* ------------------------------------------------------------------ */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
static float o_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* OCP FP8 E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; exponent 0 encodes subnormals m/8 * 2^-6. */
static float o_fp8(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    float v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexpf((float)m / 8.0f, -6);
    else
        v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return s ? -v : v;
}

static float o_elem(int dt, const void* base, int64_t i) {
    switch (dt) {
        case O_F32: return ((const float*)base)[i];
        case O_BF16: return o_bf16(((const uint16_t*)base)[i]);
        default: return o_fp8(((const uint8_t*)base)[i]);
    }
}

static int64_t o_esize(int dt) { return dt == O_F32 ? 4 : (dt == O_BF16 ? 2 : 1); }

/* Decode n stored elements; returns the number of NaN results. */
int64_t lsao_decode(int dt, const void* src, int64_t n, float* dst) {
    int64_t bad = 0;
    for (int64_t i = 0; i < n; i++) {
        dst[i] = o_elem(dt, src, i);
        if (isnan(dst[i])) bad++;
    }
    return bad;
}

/* ------------------------------------------------------------------ */
/* O2: geometry of one request                                         */
/* ------------------------------------------------------------------ */

/* The most recent W tokens always stay on the device; history is split
 * into chunks of C tokens.  Partial leftovers next to the recent window
 * count as recent, so the recent region starts at a chunk boundary:
 * rs = C * floor(max(L - W, 0) / C); history chunks are [0, rs/C). */
void lsao_geometry(int32_t L, int32_t C, int32_t W, int64_t out[3]) {
    int64_t h = (int64_t)L - W;
    if (h < 0) h = 0;
    int64_t rs = (int64_t)C * (h / C);
    out[0] = rs;          /* first recent token           */
    out[1] = rs / C;      /* number of history chunks     */
    out[2] = L - rs;      /* number of recent tokens      */
}

/* ------------------------------------------------------------------ */
/* Batch description (raw stored bytes, layout of the C-ABI)           */
/* ------------------------------------------------------------------ */
typedef struct {
    int32_t B, C, W;
    const int32_t* seq_len;          /* [B]                                   */
    int32_t H, d, q_dt, idx_dt;      /* indexer heads, dim, dtypes            */
    int32_t Hq, Dk, Dv, kv_dt, v_off;/* attention heads, dims, dtype, V offset */
    int64_t kv_row_bytes, page_bytes, ikey_off;
    const void* kic;                 /* [sum N, d] compressed index keys      */
    const float* kic_scale;          /* [sum N] (fp8 only, else NULL)         */
    const void* pages;               /* [sum N, page_bytes] cold tier         */
    const float* ikey_scale;         /* [sum N] (fp8 only, else NULL)         */
    const void* recent;              /* [sum R, kv_row_bytes]                 */
} lsao_batch;

static void o_offsets(const lsao_batch* b, int32_t r, int64_t* chunk0, int64_t* rec0,
                      int64_t g[3]) {
    int64_t c0 = 0, q0 = 0, t[3];
    for (int32_t i = 0; i < r; i++) {
        lsao_geometry(b->seq_len[i], b->C, b->W, t);
        c0 += t[1];
        q0 += t[2];
    }
    lsao_geometry(b->seq_len[r], b->C, b->W, g);
    *chunk0 = c0;
    *rec0 = q0;
}

/* ------------------------------------------------------------------ */
/* O3-O5: fused query, chunk logits, threshold selection               */
/* ------------------------------------------------------------------ */

/* For each request: qbar[i] = sum_h w_h q_h[i] (fmaf chain over h from +0);
 * z_c = fmaf(s_c, sum_i qbar[i] k_c[i], b) (fmaf chain over i from +0;
 * s_c = 1 unless fp8); chunk c is selected iff z_c > theta.  theta = 0 is
 * sigmoid(z) > 0.5.  sel holds, per request, the ascending selected ids in
 * the first cnt[r] entries of its segment. */
int lsao_score_select(const lsao_batch* b, const void* q, const float* w, const float* bias,
                      float theta, float* z, int32_t* sel, int32_t* cnt) {
    int64_t chunk0 = 0;
    float* qbar = (float*)malloc(sizeof(float) * (size_t)b->d);
    if (!qbar) return -1;
    for (int32_t r = 0; r < b->B; r++) {
        int64_t g[3];
        lsao_geometry(b->seq_len[r], b->C, b->W, g);
        const int64_t N = g[1];
        for (int32_t i = 0; i < b->d; i++) {
            float acc = 0.0f;
            for (int32_t h = 0; h < b->H; h++)
                acc = fmaf(w[(int64_t)r * b->H + h],
                           o_elem(b->q_dt, q, ((int64_t)r * b->H + h) * b->d + i), acc);
            qbar[i] = acc;
        }
        int32_t n_sel = 0;
        for (int64_t c = 0; c < N; c++) {
            const int64_t row = chunk0 + c;
            float acc = 0.0f;
            for (int32_t i = 0; i < b->d; i++)
                acc = fmaf(qbar[i], o_elem(b->idx_dt, b->kic, row * b->d + i), acc);
            const float s = (b->idx_dt == O_FP8) ? b->kic_scale[row] : 1.0f;
            z[row] = fmaf(s, acc, bias[r]);
            if (z[row] > theta) sel[chunk0 + n_sel++] = (int32_t)c;
        }
        cnt[r] = n_sel;
        chunk0 += N;
    }
    free(qbar);
    return 0;
}

/* OR-mode union over indexer layers.  Independent memory indexers sit at
 * several layers (three: 10, 12 and 20); at inference a chunk is recalled
 * when any of them scores it above 0.5 (cjcn.com.cn explainer, section 四;
 * gist.science summary, section 2.4 "Optimale Konfiguration").  Each layer
 * l has its own query state, head weights, bias and KIComp rows; its logits
 * follow the single-layer definition above in the same fp32 order.  The
 * per-chunk masks (z_l > theta) are OR-ed before one ordered compaction.
 * zmax[c] = max_l z_l[c] (so zmax > theta exactly when the OR mask is set).
 * kic[l], kic_scale[l] replace b->kic, b->kic_scale. */
int lsao_score_select_union(const lsao_batch* b, int32_t n_layers, const void* const* q,
                            const float* const* w, const float* const* bias,
                            const void* const* kic, const float* const* kic_scale, float theta,
                            float* zmax, int32_t* sel, int32_t* cnt) {
    if (n_layers < 1) return -1;
    int64_t chunk0 = 0;
    float* qbar = (float*)malloc(sizeof(float) * (size_t)b->d * (size_t)n_layers);
    if (!qbar) return -1;
    for (int32_t r = 0; r < b->B; r++) {
        int64_t g[3];
        lsao_geometry(b->seq_len[r], b->C, b->W, g);
        const int64_t N = g[1];
        for (int32_t l = 0; l < n_layers; l++)
            for (int32_t i = 0; i < b->d; i++) {
                float acc = 0.0f;
                for (int32_t h = 0; h < b->H; h++)
                    acc = fmaf(w[l][(int64_t)r * b->H + h],
                               o_elem(b->q_dt, q[l], ((int64_t)r * b->H + h) * b->d + i), acc);
                qbar[(int64_t)l * b->d + i] = acc;
            }
        int32_t n_sel = 0;
        for (int64_t c = 0; c < N; c++) {
            const int64_t row = chunk0 + c;
            int any = 0;
            float zm = 0.0f;
            for (int32_t l = 0; l < n_layers; l++) {
                float acc = 0.0f;
                for (int32_t i = 0; i < b->d; i++)
                    acc = fmaf(qbar[(int64_t)l * b->d + i], o_elem(b->idx_dt, kic[l], row * b->d + i),
                               acc);
                const float s = (b->idx_dt == O_FP8) ? kic_scale[l][row] : 1.0f;
                const float z = fmaf(s, acc, bias[l][r]);
                any |= (z > theta);
                zm = (l == 0 || z > zm) ? z : zm;
            }
            zmax[row] = zm;
            if (any) sel[chunk0 + n_sel++] = (int32_t)c;
        }
        cnt[r] = n_sel;
        chunk0 += N;
    }
    free(qbar);
    return 0;
}

/* Per-head sigmoid score.  The memory indexer is the lightning indexer with
 * its ReLU replaced by a sigmoid, so that its score is a probability in
 * (0, 1) and a fixed threshold of 0.5 decides the fetch (cjcn.com.cn
 * explainer, section 二).  Read literally, per chunk c of request r:
 *     S_c = sum_h w_h sigmoid(s_c (q_h . k_c) + b_r),  fetched iff S_c > 0.5.
 * fp32 order: per head the dot product is an fmaf chain over i from +0,
 * x_h = fmaf(s_c, a_h, b_r), and S_c an fmaf chain over h from +0 of
 * w_h * sigmoid(x_h).  The pages fix no precision for the sigmoid, so one
 * fp32 definition is written out (o_sigmoid) and the library follows it:
 *     sigmoid(x) = 1 / (1 + e^(-x)),  e^y = 2^t with t = y * log2(e):
 *     n = rint(t), f = t - n (|f| <= 1/2), 2^f by the degree-7 Taylor
 *     polynomial (ln 2)^k / k! in Horner form with fmaf, times 2^n (ldexp).
 * t is clamped to [-200, 200] first (2^t is 0 or inf beyond, in fp32).
 * The constants are the fp32 values nearest to log2(e) and (ln 2)^k / k!. */
static const float O_LOG2E = 1.44269502162933349609375f;  /* 0x3fb8aa3b */
static const float O_EXP2C[8] = {1.0f, 0.693147182464599609375f, 0.2402265071868896484375f,
                                 0.0555041097104549407958984375f, 0.00961812864989042282104492188f,
                                 0.00133335578721016645431518555f, 0.000154035296873189508914947510f,
                                 1.52527336467755958437919616699e-05f};

float lsao_sigmoid(float x) {
    float t = -x * O_LOG2E;
    t = fminf(fmaxf(t, -200.0f), 200.0f);
    const float n = rintf(t);
    const float f = t - n;
    float p = O_EXP2C[7];
    for (int k = 6; k >= 0; k--) p = fmaf(p, f, O_EXP2C[k]);
    const float e = ldexpf(p, (int)n);
    return 1.0f / (1.0f + e);
}

int lsao_score_select_sigmoid(const lsao_batch* b, const void* q, const float* w, const float* bias,
                              float theta, float* S, int32_t* sel, int32_t* cnt) {
    int64_t chunk0 = 0;
    float* kf = (float*)malloc(sizeof(float) * (size_t)b->d);
    if (!kf) return -1;
    for (int32_t r = 0; r < b->B; r++) {
        int64_t g[3];
        lsao_geometry(b->seq_len[r], b->C, b->W, g);
        const int64_t N = g[1];
        int32_t n_sel = 0;
        for (int64_t c = 0; c < N; c++) {
            const int64_t row = chunk0 + c;
            for (int32_t i = 0; i < b->d; i++) kf[i] = o_elem(b->idx_dt, b->kic, row * b->d + i);
            const float s = (b->idx_dt == O_FP8) ? b->kic_scale[row] : 1.0f;
            float acc_s = 0.0f;
            for (int32_t h = 0; h < b->H; h++) {
                float a = 0.0f;
                for (int32_t i = 0; i < b->d; i++)
                    a = fmaf(o_elem(b->q_dt, q, ((int64_t)r * b->H + h) * b->d + i), kf[i], a);
                const float x = fmaf(s, a, bias[r]);
                acc_s = fmaf(w[(int64_t)r * b->H + h], lsao_sigmoid(x), acc_s);
            }
            S[row] = acc_s;
            if (acc_s > theta) sel[chunk0 + n_sel++] = (int32_t)c;
        }
        cnt[r] = n_sel;
        chunk0 += N;
    }
    free(kf);
    return 0;
}

/* ------------------------------------------------------------------ */
/* O6-O8: candidate tokens, lightning refine score, top-k              */
/* ------------------------------------------------------------------ */
typedef struct {
    float score;
    int32_t tok;
} o_cand;

/* Order: larger score first; equal scores: lower token first. */
static int o_cand_cmp(const void* pa, const void* pb) {
    const o_cand* a = (const o_cand*)pa;
    const o_cand* c = (const o_cand*)pb;
    if (a->score > c->score) return -1;
    if (a->score < c->score) return 1;
    return (a->tok > c->tok) - (a->tok < c->tok);
}

static int o_int_cmp(const void* pa, const void* pb) {
    int32_t a = *(const int32_t*)pa, c = *(const int32_t*)pb;
    return (a > c) - (a < c);
}

/* Candidate tokens T = the tokens of the selected chunks, ascending.  For each
 * s in T (chunk c = s / C):
 *     a_h = fmaf chain over i of q_h[i] * k_s[i] from +0   (per head h)
 *     r_h = a_h > 0 ? a_h : +0
 *     I   = fmaf chain over h of w_h * r_h from +0
 *     I_s = I * s_c   (fp8 index keys only)
 * The result keeps min(k, |T|) tokens: the largest I_s, ties to the lower
 * token, written ascending to topk[].  Returns the count. */
int32_t lsao_refine_topk(const lsao_batch* b, int32_t r, const int32_t* sel_r, int32_t cnt_r,
                         const void* q_r, const float* w_r, int32_t k, int32_t* topk,
                         float* cand_scores) {
    int64_t chunk0, rec0, g[3];
    o_offsets(b, r, &chunk0, &rec0, g);
    const int64_t n_cand = (int64_t)cnt_r * b->C;
    const int64_t ib = o_esize(b->idx_dt);
    o_cand* cand = (o_cand*)malloc(sizeof(o_cand) * (size_t)(n_cand > 0 ? n_cand : 1));
    float* qf = (float*)malloc(sizeof(float) * (size_t)b->H * b->d);
    float* rh = (float*)malloc(sizeof(float) * (size_t)b->H);
    if (!cand || !qf || !rh) return -1;
    for (int64_t i = 0; i < (int64_t)b->H * b->d; i++) qf[i] = o_elem(b->q_dt, q_r, i);
    int64_t pos = 0;
    for (int32_t j = 0; j < cnt_r; j++) {
        const int64_t c = sel_r[j];
        const uint8_t* page = (const uint8_t*)b->pages + (chunk0 + c) * b->page_bytes;
        const float sc = (b->idx_dt == O_FP8) ? b->ikey_scale[chunk0 + c] : 1.0f;
        for (int32_t t = 0; t < b->C; t++) {
            const void* key = page + b->ikey_off + (int64_t)t * b->d * ib;
            for (int32_t h = 0; h < b->H; h++) {
                float a = 0.0f;
                for (int32_t i = 0; i < b->d; i++)
                    a = fmaf(qf[(int64_t)h * b->d + i], o_elem(b->idx_dt, key, i), a);
                rh[h] = (a > 0.0f) ? a : 0.0f;
            }
            float I = 0.0f;
            for (int32_t h = 0; h < b->H; h++) I = fmaf(w_r[h], rh[h], I);
            if (b->idx_dt == O_FP8) I = I * sc;
            if (I == 0.0f) I = 0.0f; /* -0 and +0 compare equal; keep one */
            cand[pos].score = I;
            cand[pos].tok = (int32_t)(c * b->C + t);
            if (cand_scores) cand_scores[pos] = I;
            pos++;
        }
    }
    int32_t kk = (n_cand < k) ? (int32_t)n_cand : k;
    if (n_cand > 0) qsort(cand, (size_t)n_cand, sizeof(o_cand), o_cand_cmp);
    for (int32_t i = 0; i < kk; i++) topk[i] = cand[i].tok;
    if (kk > 0) qsort(topk, (size_t)kk, sizeof(int32_t), o_int_cmp);
    free(cand);
    free(qf);
    free(rh);
    return kk;
}

/* ------------------------------------------------------------------ */
/* O9: sparse decode attention (fp64)                                  */
/* ------------------------------------------------------------------ */

static const void* o_kv_row(const lsao_batch* b, int64_t chunk0, int64_t rec0, int64_t rs,
                            int64_t s) {
    if (s < rs)
        return (const uint8_t*)b->pages + (chunk0 + s / b->C) * b->page_bytes +
               (s % b->C) * b->kv_row_bytes;
    return (const uint8_t*)b->recent + (rec0 + s - rs) * b->kv_row_bytes;
}

/* A = the top-k tokens followed by the recent tokens [rs, L).  For every
 * query head h:  x_i = sm * q_h . K_i,  m = max x,  p_i = exp(x_i - m),
 * l = sum p,  o_h = sum_i p_i V_i / l,  lse_h = m + ln l.  K_i is the first
 * Dk elements of token i's KV row, V_i the Dv elements at v_off.
 * An empty A (no recent token and an empty top-k; the pages never reach it,
 * their recent window is always attended) has no softmax: the reading taken
 * is the value of an empty sum, o_h = 0 and lse_h = ln 0 = -inf. */
int lsao_attend(const lsao_batch* b, int32_t r, const int32_t* topk, int32_t kcnt,
                const void* q_r, double sm, double* out, double* lse) {
    int64_t chunk0, rec0, g[3];
    o_offsets(b, r, &chunk0, &rec0, g);
    const int64_t rs = g[0], L = b->seq_len[r];
    const int64_t nA = kcnt + (L - rs);
    const void** rows = (const void**)malloc(sizeof(void*) * (size_t)(nA > 0 ? nA : 1));
    double* x = (double*)malloc(sizeof(double) * (size_t)(nA > 0 ? nA : 1));
    if (!rows || !x) return -1;
    for (int32_t i = 0; i < kcnt; i++) rows[i] = o_kv_row(b, chunk0, rec0, rs, topk[i]);
    for (int64_t s = rs; s < L; s++) rows[kcnt + (s - rs)] = o_kv_row(b, chunk0, rec0, rs, s);
    for (int32_t h = 0; h < b->Hq && nA == 0; h++) {
        for (int32_t e = 0; e < b->Dv; e++) out[(int64_t)h * b->Dv + e] = 0.0;
        lse[h] = -INFINITY;
    }
    for (int32_t h = 0; h < b->Hq && nA > 0; h++) {
        double m = -INFINITY;
        for (int64_t i = 0; i < nA; i++) {
            double acc = 0.0;
            for (int32_t e = 0; e < b->Dk; e++)
                acc += (double)o_elem(b->kv_dt, q_r, (int64_t)h * b->Dk + e) *
                       (double)o_elem(b->kv_dt, rows[i], e);
            x[i] = sm * acc;
            if (x[i] > m) m = x[i];
        }
        double l = 0.0;
        for (int64_t i = 0; i < nA; i++) {
            x[i] = exp(x[i] - m);
            l += x[i];
        }
        for (int32_t e = 0; e < b->Dv; e++) {
            double acc = 0.0;
            for (int64_t i = 0; i < nA; i++)
                acc += x[i] * (double)o_elem(b->kv_dt, rows[i], b->v_off + e);
            out[(int64_t)h * b->Dv + e] = acc / l;
        }
        lse[h] = m + log(l);
    }
    free(rows);
    free(x);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Decode steps: refine + top-k + attention for a list of              */
/* (request, step) units, independent of each other.                   */
/* ------------------------------------------------------------------ */

/* sel/cnt: the window's selection (layout of lsao_score_select).
 * q_refine [S, B, H, d] (q_dt), w_refine [S, B, H], q_attn [S, B, Hq, Dk]
 * (kv_dt).  Outputs per unit u: topk_out[u*k ...], topk_cnt[u],
 * out[u*Hq*Dv ...], lse[u*Hq ...].  Units run in parallel over threads;
 * each unit's arithmetic is sequential, so results do not depend on the
 * thread count.  Returns 0 or the first failing unit's error. */
int lsao_decode_units(const lsao_batch* b, int32_t n_units, const int32_t* unit_r,
                      const int32_t* unit_step, const int32_t* sel, const int32_t* cnt,
                      const void* q_refine, const float* w_refine, const void* q_attn,
                      int32_t k, double sm, int32_t* topk_out, int32_t* topk_cnt, double* out,
                      double* lse, int32_t n_threads) {
    int err = 0;
    const int64_t qes = o_esize(b->q_dt), kes = o_esize(b->kv_dt);
#ifdef _OPENMP
    if (n_threads <= 0) n_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
#endif
    for (int32_t u = 0; u < n_units; u++) {
        const int32_t r = unit_r[u], j = unit_step[u];
        int64_t chunk0, rec0, g[3];
        o_offsets(b, r, &chunk0, &rec0, g);
        const int64_t qi = ((int64_t)j * b->B + r);
        const uint8_t* qr = (const uint8_t*)q_refine + qi * b->H * b->d * qes;
        const float* wr = w_refine + qi * b->H;
        const uint8_t* qa = (const uint8_t*)q_attn + qi * b->Hq * b->Dk * kes;
        int32_t kc = lsao_refine_topk(b, r, sel + chunk0, cnt[r], qr, wr, k,
                                      topk_out + (int64_t)u * k, NULL);
        int e = 0;
        if (kc < 0)
            e = -1;
        else {
            topk_cnt[u] = kc;
            e = lsao_attend(b, r, topk_out + (int64_t)u * k, kc, qa, sm,
                            out + (int64_t)u * b->Hq * b->Dv, lse + (int64_t)u * b->Hq);
        }
        if (e) {
#ifdef _OPENMP
#pragma omp critical
#endif
            err = e;
        }
    }
    (void)n_threads;
    return err;
}

/* ------------------------------------------------------------------ */
/* O10: attention mass per history chunk                               */
/* ------------------------------------------------------------------ */

/* The pages' oracle experiment ranks history chunks by the attention weight
 * that the full decode actually gives them, and keeps the top 50, 25 or 10
 * percent (cjcn.com.cn explainer, section 六).  Read here: for each given
 * decode step j and query head h, the softmax of x_s = sm * q_{j,h} . K_s
 * over EVERY token s of [0, L) (nothing selected, nothing left out); a
 * history chunk's mass is the sum of those probabilities over its C tokens,
 * over the steps and over the heads:
 *     mass_c = sum_j sum_h sum_{s in chunk c} p_{j,h,s},
 * and rec_mass is the same sum over the recent tokens [rs, L), so that
 * sum_c mass_c + rec_mass = n_steps * Hq.  fp64 from the decoded inputs.
 * q is [n_steps, Hq, Dk] in the KV dtype.  Each (step, head) unit is
 * computed alone and the units are added in order, so the result does not
 * depend on the thread count. */
int lsao_chunk_mass(const lsao_batch* b, int32_t r, int32_t n_steps, const void* q, double sm,
                    double* mass, double* rec_mass, int32_t n_threads) {
    int64_t chunk0, rec0, g[3];
    o_offsets(b, r, &chunk0, &rec0, g);
    const int64_t rs = g[0], N = g[1], L = b->seq_len[r];
    const int32_t nU = n_steps * b->Hq;
    const int64_t kes = o_esize(b->kv_dt);
    double* part = (double*)calloc((size_t)nU * (size_t)(N + 1), sizeof(double));
    if (!part) return -1;
    int err = 0;
#ifdef _OPENMP
    if (n_threads <= 0) n_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
#endif
    for (int32_t u = 0; u < nU; u++) {
        const uint8_t* qh = (const uint8_t*)q + (int64_t)u * b->Dk * kes;
        double* pu = part + (int64_t)u * (N + 1);
        double* x = (double*)malloc(sizeof(double) * (size_t)L);
        if (!x) {
#ifdef _OPENMP
#pragma omp critical
#endif
            err = -1;
            continue;
        }
        double m = -INFINITY;
        for (int64_t t = 0; t < L; t++) {
            const void* row = o_kv_row(b, chunk0, rec0, rs, t);
            double acc = 0.0;
            for (int32_t e = 0; e < b->Dk; e++)
                acc += (double)o_elem(b->kv_dt, qh, e) * (double)o_elem(b->kv_dt, row, e);
            x[t] = sm * acc;
            if (x[t] > m) m = x[t];
        }
        double l = 0.0;
        for (int64_t t = 0; t < L; t++) l += exp(x[t] - m);
        for (int64_t t = 0; t < L; t++) {
            const double p = exp(x[t] - m) / l;
            if (t < rs) pu[t / b->C] += p;
            else pu[N] += p;
        }
        free(x);
    }
    (void)n_threads;
    for (int64_t c = 0; c <= N; c++) {
        double acc = 0.0;
        for (int32_t u = 0; u < nU; u++) acc += part[(int64_t)u * (N + 1) + c];
        if (c < N) mass[c] = acc;
        else *rec_mass = acc;
    }
    free(part);
    return err;
}

int lsao_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
