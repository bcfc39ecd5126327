/*
 * lsa.h -- C-ABI of the Lookahead Sparse Attention (LSA) decode hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * The method is that of "FlashMemory-DeepSeek-V4: Lightning Index
 * Ultra-Long Context via Lookahead Sparse Attention".  Every 64 decode steps a
 * memory indexer scores every history chunk against the current query
 * state.  The chunks whose sigmoid score exceeds 0.5 move from a cold pool
 * into GPU memory.  At each step a lightning-indexer top-k picks tokens
 * inside that set, and sparse attention runs over them plus the recent
 * window.
 *
 * Conventions for every entry point:
 *  - extern "C"; no C++ exception crosses the boundary; every function
 *    returns an lsa_status (or nothing, for destructors).
 *  - Pointers marked (device) are HBM addresses; (host) are CPU addresses.
 *    The caller owns every buffer.  The library keeps no pointer beyond the
 *    call, except for objects created by lsa_pool_create / lsa_ctx_create,
 *    which borrow what they are given until destroyed.
 *  - Streams and events are hipStream_t / hipEvent_t passed as void*.
 *    NULL means the default stream.  Device work is enqueued
 *    asynchronously; outputs are valid once the stream reaches that point.
 *  - Arguments are checked before anything is enqueued.  On an error nothing
 *    has been enqueued and outputs are untouched.  A HIP launch or copy
 *    failure returns LSA_ERR_HIP; a kernel fault surfaces at the next
 *    synchronisation.
 *  - Calls are reentrant when given distinct outputs and workspaces.
 *  - Workspaces (ws) must be 16-byte aligned (hipMalloc and torch device
 *    allocations are); an unaligned one is LSA_ERR_INVALID_ARG.
 *
 * Geometry (per request r, context L_r, chunk C, recent window W).  The most
 * recent W tokens are always attended (cjcn.com.cn explainer, section 二, last
 * paragraph); history is cut into chunks of C tokens ("fixed-size blocks",
 * ai-feeds.com digest, method section), and a partial chunk next to the
 * recent window counts as recent:
 *     rs_r     = C * floor(max(L_r - W, 0) / C)   first recent token
 *     N_r      = rs_r / C                         history chunks
 *     R_r      = L_r - rs_r                       recent tokens (W .. W+C-1, or L_r)
 *     chunk_off[r] = sum_{i<r} N_i,   rec_off[r] = sum_{i<r} R_i
 * Arrays "over chunks" are concatenated over requests: request r owns
 * entries [chunk_off[r], chunk_off[r] + N_r).  Recent KV rows likewise own
 * rows [rec_off[r], rec_off[r] + R_r).  "[sum N]" below means
 * chunk_off[B] entries and "[sum R]" rec_off[B] rows.
 *
 * Growing context.  During decode every step appends one token, and at each
 * trigger the oldest full chunk of the recent region joins the history.
 * For that the
 * geometry can fix rs_r explicitly (hist_tokens, so the recent region stays
 * anchored between triggers while L_r grows), and give each request fixed
 * capacities so that one request's growth moves no other's rows:
 *     chunk_cap > 0:  chunk_off[r] = r * chunk_cap   (N_r <= chunk_cap)
 *     recent_cap > 0: rec_off[r]   = r * recent_cap  (R_r <= recent_cap)
 * Every entry point reads its arrays through chunk_off and rec_off, so the
 * same kernels serve both layouts.
 *
 * Pages.  The cold tier and the HBM slot pool store one chunk per page of
 * page_bytes: C KV rows of row_bytes, then, at byte ikey_off, C index-key
 * rows of d elements.  A page table maps chunk (chunk_off[r] + c) to a page
 * index in a page array; NULL means the identity, i.e. the page array is the
 * cold tier itself.
 */
#ifndef LSA_H_
#define LSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LSA_MAX_BATCH 64
#define LSA_MAX_LAYERS 8   /* indexer layers of lsa_score_chunks_union */
#define LSA_CHUNK 64

typedef enum {
    LSA_OK = 0,
    LSA_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent shapes        */
    LSA_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype or shape)         */
    LSA_ERR_CAPACITY = -3,    /* slot pool too small for the selection              */
    LSA_ERR_WORKSPACE = -4,   /* workspace smaller than the lsa_*_ws_bytes query    */
    LSA_ERR_HIP = -5          /* a HIP runtime call failed                          */
} lsa_status;

typedef enum { LSA_F32 = 0, LSA_BF16 = 1, LSA_FP8_E4M3FN = 2 } lsa_dtype;

/* Batch geometry.  seq_len is a host array of B contexts (each >= 1); the
 * library derives rs, N, R and the offsets above from it.  The last three
 * fields are zero / NULL for the packed layout. */
typedef struct {
    int32_t batch;              /* B, 1..LSA_MAX_BATCH                          */
    int32_t chunk;              /* C, must be LSA_CHUNK (64)                    */
    int32_t window;             /* W >= 0, recent tokens always attended        */
    const int32_t* seq_len;     /* (host) [B]                                   */
    const int32_t* hist_tokens; /* (host) [B] rs_r (a multiple of C, <= L_r), or
                                   NULL for C * floor(max(L_r - W, 0) / C)      */
    int32_t chunk_cap;          /* > 0: chunk_off[r] = r * chunk_cap            */
    int32_t recent_cap;         /* > 0: rec_off[r] = r * recent_cap             */
} lsa_geom;

/* Layout of one KV row and of a page. */
typedef struct {
    lsa_dtype kv_dtype; /* LSA_F32 or LSA_BF16                                    */
    int32_t Dk;         /* key width: K = elements [0, Dk) of the row               */
    int32_t Dv;         /* value width                                              */
    int32_t v_off;      /* V = elements [v_off, v_off+Dv); 0 for a latent row       */
    int64_t row_bytes;  /* bytes per KV row (>= element size * max(Dk, v_off+Dv))   */
    int64_t page_bytes; /* bytes per page                                           */
    int64_t ikey_off;   /* byte offset of the C index-key rows inside a page        */
} lsa_kv_layout;

const char* lsa_status_str(lsa_status s);

/* ------------------------------------------------------------------------
 * a2. Chunk scoring.  "Lookahead index score" between the current query and
 * the compressed index keys (KIComp) of previous chunks: a head-fused
 * matching score through a sigmoid (gist.science summary, section 2.1,
 * "Scoring-Mechanismus"); the match is a plain dot product (cjcn.com.cn,
 * section 六; gist.science, section 5).  Computes the logit of that score:
 *     qbar[i] = sum_h w[r,h] * q[r,h,i]          (fp32 fma chain over h)
 *     z[c]    = fma(s_c, sum_i qbar[i]*k_c[i], bias[r])   (fma chain over i)
 * for every history chunk c of every request; s_c = kic_scale[c] for fp8
 * keys, else 1.  sigmoid(z) > 0.5 exactly when z > 0.
 *   q        (device) [B, H, d] in q_dt (LSA_F32 or LSA_BF16)
 *   w        (device) [B, H] f32;  bias (device) [B] f32
 *   kic      (device) [sum N, d] in kic_dt (f32, bf16 or fp8 e4m3fn)
 *   kic_scale(device) [sum N] f32, required iff kic_dt is fp8, else ignored
 *   z        (device) [sum N] f32 output
 *   ws       (device) >= lsa_score_ws_bytes(g, d) bytes of scratch
 * d must be 64 or 128; 1 <= H <= 256.
 * ---------------------------------------------------------------------- */
size_t lsa_score_ws_bytes(const lsa_geom* g, int32_t d);
lsa_status lsa_score_chunks(const lsa_geom* g, const void* q, lsa_dtype q_dt, const float* w,
                            const float* bias, int32_t H, int32_t d, const void* kic,
                            lsa_dtype kic_dt, const float* kic_scale, float* z, void* ws,
                            size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * a2, OR mode.  Independent memory indexers sit at several layers (the
 * pages place three, at layers 10, 12 and 20); at inference a chunk is
 * fetched when any layer scores it above 0.5 (cjcn.com.cn explainer,
 * section 四; gist.science summary, section 2.4).  Layer l has its own
 * q[l], w[l], bias[l], kic[l] (and kic_scale[l] for fp8 keys), with the
 * shapes, dtypes and meaning of lsa_score_chunks; each layer's logits are
 * computed exactly as there, and z receives their per-chunk maximum
 * (the earliest of equals), so lsa_select_threshold on z selects the OR of
 * the layers' selections.
 *   n_layers  1..LSA_MAX_LAYERS
 *   q, w, bias, kic, kic_scale  (host) arrays of n_layers device pointers
 *             (kic_scale may be NULL unless kic_dt is fp8)
 *   z (device) [sum N] f32 output;  ws as lsa_score_ws_bytes(g, d)
 * ---------------------------------------------------------------------- */
lsa_status lsa_score_chunks_union(const lsa_geom* g, int32_t n_layers, const void* const* q,
                                  lsa_dtype q_dt, const float* const* w, const float* const* bias,
                                  int32_t H, int32_t d, const void* const* kic, lsa_dtype kic_dt,
                                  const float* const* kic_scale, float* z, void* ws, size_t ws_bytes,
                                  void* stream);

/* ------------------------------------------------------------------------
 * a2, per-head sigmoid variant.  The memory indexer is the lightning indexer
 * with its ReLU replaced by a sigmoid, so that its score is a probability
 * and a fixed 0.5 decides the fetch (cjcn.com.cn explainer, section 二).
 * Read per head, for every history chunk c of request r:
 *     x_h = fma(s_c, a_h, b[r]),  a_h = sum_i q[r,h,i] * k_c[i] (fp32 fma chain
 *           over i from +0),  s_c = kic_scale[c] for fp8 keys, else 1
 *     S[c] = sum_h w[r,h] * sigmoid(x_h)  (fp32 fma chain over h from +0)
 * with one written fp32 sigmoid: 1 / (1 + 2^t), t = clamp(-x log2 e, -200,
 * 200), 2^t = ldexp(P(f), n), n = rint(t), f = t - n, P the degree-7 Taylor
 * polynomial of 2^f with coefficients nearest to (ln 2)^k / k! in Horner
 * fma form; IEEE division.
 * With bf16 queries and bf16 or fp8 keys (H <= 64 for d = 128, H <= 128 for
 * d = 64) the dot products run on the matrix cores and S[c] is within a
 * rigorous per-chunk bound E_c (about 1e-4 at unit weights) of the value
 * above; where |S[c] - theta| <= E_c, S[c] is that value bit for bit.  So
 * S[c] > theta holds exactly when it holds in the order above, and
 * lsa_select_threshold(S, theta) with the same theta selects exactly the
 * fetched chunks.  Otherwise (fp32 queries or keys, H * d <= 8192) every
 * S[c] is the value above bit for bit.
 *   q, w, bias, kic, kic_scale as lsa_score_chunks (q 16-byte aligned);
 *   theta   the fetch threshold (0.5 for probabilities)
 *   S (device) [sum N] f32
 * d must be 64 or 128.  No workspace.
 * ---------------------------------------------------------------------- */
lsa_status lsa_score_chunks_sigmoid(const lsa_geom* g, const void* q, lsa_dtype q_dt, const float* w,
                                    const float* bias, float theta, int32_t H, int32_t d,
                                    const void* kic, lsa_dtype kic_dt, const float* kic_scale, float* S,
                                    void* stream);

/* ------------------------------------------------------------------------
 * a3. Threshold selection.  A fixed threshold replaces a fixed top-k, so
 * the number of fetched chunks varies (cjcn.com.cn, section 二; gist.science
 * 2.1 "Dynamisches Fetching").  Chunk c of request r is selected iff
 * z[c] > theta (strict); theta = 0 is sigmoid > 0.5.  Output, per request:
 * the ascending selected chunk ids (0-based within the request) in
 * sel_ids[chunk_off[r] ...], and their count in sel_cnt[r].
 *   z (device) [sum N] f32;  sel_ids (device) [sum N] int32;  sel_cnt (device) [B] int32
 * ---------------------------------------------------------------------- */
lsa_status lsa_select_threshold(const lsa_geom* g, const float* z, float theta, int32_t* sel_ids,
                                int32_t* sel_cnt, void* stream);

/* ------------------------------------------------------------------------
 * a5+a6. Lightning refine and top-k.  Inside the fetched candidate set the
 * native lightning indexer takes a fine-grained top-k for core attention
 * (gist.science 2.1 "Gestufte Selektion"; cjcn.com.cn section 二); its score
 * is a ReLU-weighted sum over heads (cjcn.com.cn section 二 names the ReLU).
 * For every token s of every selected chunk c (candidate set T, ascending):
 *     a_h = sum_i q[r,h,i] * key_s[i]  (fp32 fma chain over i, from +0)
 *     I_s = sum_h w[r,h] * max(a_h, +0) (fp32 fma chain over h, from +0)
 *     I_s = I_s * ikey_scale[chunk]     (fp8 keys only)
 * keeps the min(k, |T|) largest I_s, ties to the lower token, and writes
 * their absolute token positions (c*C + t) ascending.
 *   sel_ids, sel_cnt (device): as produced by lsa_select_threshold
 *   pages      (device) page array; index keys of chunk x live in page
 *              page_table[x] (or x if page_table is NULL) at byte ikey_off
 *   ikey_scale (device) [sum N] f32, required iff idx_dt is fp8
 *   q (device) [B, H, d] q_dt;  w (device) [B, H] f32
 *   topk_idx (device) [B, k] int32 out (first topk_cnt[r] valid); topk_cnt (device) [B] out
 *   ws (device) >= lsa_refine_ws_bytes(g, k) bytes
 * d in {64, 128}; 1 <= H <= 128; 1 <= k.
 * ---------------------------------------------------------------------- */
size_t lsa_refine_ws_bytes(const lsa_geom* g, int32_t k);
lsa_status lsa_topk_refine(const lsa_geom* g, const int32_t* sel_ids, const int32_t* sel_cnt,
                           const void* pages, int64_t page_bytes, int64_t ikey_off,
                           const int32_t* page_table, lsa_dtype idx_dt, const float* ikey_scale,
                           const void* q, lsa_dtype q_dt, const float* w, int32_t H, int32_t d,
                           int32_t k, int32_t* topk_idx, int32_t* topk_cnt, void* ws,
                           size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * a7. Sparse decode attention.  Core attention over the selected tokens plus
 * the always-resident recent window (gist.science 2.1 "Gestufte Selektion";
 * cjcn.com.cn section 二 last paragraph and section 五).  All query heads
 * share one KV (MQA).  With A_r = topk tokens of r followed by [rs_r, L_r):
 *     o[r,h] = softmax(sm_scale * q[r,h] . K_A^T) V_A,   lse[r,h] = log-sum-exp
 * accumulated in fp32, written in the KV dtype (RNE).
 *   q (device) [B, Hq, Dk] kv dtype;  pages/page_table as above (KV rows at
 *   byte 0 of a page);  recent (device) [sum R, row_bytes]
 *   topk_idx/topk_cnt (device): as produced by lsa_topk_refine (stride k)
 *   out (device) [B, Hq, Dv] kv dtype;  lse (device) [B, Hq] f32 or NULL
 *   n_splits: token splits per request (0 = automatic)
 *   ws (device) >= lsa_attn_ws_bytes(g, kv, Hq, k, n_splits) bytes
 * Supported: bf16 latent rows (Dk 576, Dv 512, v_off 0, Hq a multiple of
 * 32); f32 rows with Dk, Dv <= 256 and Hq <= 16.
 * ---------------------------------------------------------------------- */
size_t lsa_attn_ws_bytes(const lsa_geom* g, const lsa_kv_layout* kv, int32_t Hq, int32_t k,
                         int32_t n_splits);
lsa_status lsa_sparse_decode_attn(const lsa_geom* g, const void* q, int32_t Hq,
                                  const lsa_kv_layout* kv, const void* pages,
                                  const int32_t* page_table, const void* recent,
                                  const int32_t* topk_idx, const int32_t* topk_cnt, int32_t k,
                                  float sm_scale, void* out, float* lse, int32_t n_splits,
                                  void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * a7 without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * it).  Same arguments, results and errors as lsa_sparse_decode_attn, bit for
 * bit, but the split partials live in a scratch array of
 * lsa_attn_noalloc_max_bytes() bytes (32 MiB) that the library holds on each
 * GPU from its load until the process ends.  A call whose partials need more
 * (lsa_attn_ws_bytes(...) > that size) returns LSA_ERR_WORKSPACE and
 * enqueues nothing.  The call allocates nothing.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams, or
 * other threads) race and give undefined outputs; serialise them.  Nothing in
 * the array needs to start at zero (each call writes every partial it reads).
 * ---------------------------------------------------------------------- */
size_t lsa_attn_noalloc_max_bytes(void);
lsa_status lsa_sparse_decode_attn_noalloc(const lsa_geom* g, const void* q, int32_t Hq,
                                          const lsa_kv_layout* kv, const void* pages,
                                          const int32_t* page_table, const void* recent,
                                          const int32_t* topk_idx, const int32_t* topk_cnt,
                                          int32_t k, float sm_scale, void* out, float* lse,
                                          int32_t n_splits, void* stream);

/* ------------------------------------------------------------------------
 * Growing context (geometry with recent_cap > 0 and chunk_cap > 0; see the
 * top of this file).  The pages' indexer fires every 64 decode steps to
 * predict the history the next 64 steps need (cjcn.com.cn explainer,
 * section 二); between triggers each step adds one token to the recent
 * region, and at a trigger the region's oldest full chunk becomes history.
 *
 * lsa_append_kv writes each request's newest token: row r of rows goes to
 * recent row rec_off[r] + (L_r - 1 - rs_r).  g must already count the new
 * token (L_r - 1 >= rs_r).
 *   rows (device) [B, kv->row_bytes];  recent (device) [B * recent_cap rows]
 *
 * lsa_commit_chunk moves, for every request with R_r >= W + C (g before the
 * commit), the chunk c = N_r made of recent rows [0, C) into the history:
 * its KV rows into cold page chunk_off[r] + c, new_ikeys[r] (its C
 * index-key rows, d elements in idx_dt) to the same page at kv->ikey_off,
 * new_kic[r] (its KIComp row) to kic row chunk_off[r] + c, and the fp8
 * scales (new_ikey_scale[r], new_kic_scale[r]) to ikey_scale / kic_scale;
 * recent rows [C, R_r) move to recent_dst rows [0, R_r - C).  Other requests
 * copy recent rows [0, R_r) to recent_dst unchanged.  hist_out (host) [B]
 * receives the new rs_r (rs_r + C or rs_r), written before the call returns.
 *   cold (device or pinned host) cold-tier page array, identity-indexed
 *   recent_src, recent_dst (device, not overlapping) [B * recent_cap rows]
 *   new_ikeys (device) [B, C, d];  new_kic (device) [B, d]  (idx_dt)
 *   new_ikey_scale, new_kic_scale (device) [B] f32, fp8 only (else NULL)
 *   kic (device) [B * chunk_cap, d];  kic_scale, ikey_scale (device)
 *   [B * chunk_cap] f32, fp8 only
 * Needs N_r + 1 <= chunk_cap for every committing request.
 * ---------------------------------------------------------------------- */
lsa_status lsa_append_kv(const lsa_geom* g, const lsa_kv_layout* kv, const void* rows,
                         void* recent, void* stream);
lsa_status lsa_commit_chunk(const lsa_geom* g, const lsa_kv_layout* kv, const void* recent_src,
                            void* recent_dst, void* cold, lsa_dtype idx_dt, int32_t d,
                            const void* new_ikeys, const float* new_ikey_scale,
                            float* ikey_scale, const void* new_kic,
                            const float* new_kic_scale, void* kic, float* kic_scale,
                            int32_t* hist_out, void* stream);

/* ------------------------------------------------------------------------
 * Comparison policies.  The pages set LSA against a recency-only scheme
 * (the recent 8K tokens only: lsa_select_threshold with theta = +inf), a
 * scheme that keeps a random 10 % of the history chunks, and an oracle that
 * keeps the top 50 / 25 / 10 % of history chunks by the attention weight
 * the full decode gives them (cjcn.com.cn explainer, sections 五 and 六).
 *
 * lsa_select_ranked keeps, per request r, the min(m[r], N_r) best history
 * chunks by a per-chunk key, ties to the lower chunk, and lists them
 * ascending in sel_ids like lsa_select_threshold:
 *   LSA_RANK_SMALLEST_U32  keys (device) [sum N] uint32, smallest first
 *                          (uniform random keys give a uniform sample);
 *   LSA_RANK_LARGEST_F32   keys (device) [sum N] f32 (no NaN), largest first
 *                          (-0 ranks as +0).
 *   m (host) [B] int32 >= 0;  sel_ids (device) [sum N];  sel_cnt (device) [B]
 * No workspace.
 * ---------------------------------------------------------------------- */
typedef enum { LSA_RANK_SMALLEST_U32 = 0, LSA_RANK_LARGEST_F32 = 1 } lsa_rank_kind;

lsa_status lsa_select_ranked(const lsa_geom* g, const void* keys, lsa_rank_kind kind,
                             const int32_t* m, int32_t* sel_ids, int32_t* sel_cnt, void* stream);

/* lsa_chunk_attn_mass: the attention mass of every history chunk under the
 * full softmax of n_steps decode steps' queries over EVERY token [0, L_r):
 *     mass[c] = sum_j sum_h sum_{s in chunk c} p_{j,h,s},
 *     p_{j,h,s} = softmax over s of sm_scale * q[j,r,h] . K_s,
 * and rec_mass[r] the same sum over the recent tokens [rs_r, L_r), so that
 * sum_c mass[c] + rec_mass[r] = n_steps * Hq up to rounding.  fp32
 * arithmetic (scores on the matrix cores from the bf16 rows, fp32
 * accumulation).  The history rows are read from pages (page_table or the
 * identity, as lsa_sparse_decode_attn), the recent ones from recent.
 *   q (device) [n_steps, B, Hq, Dk] in the KV dtype
 *   mass (device) [sum N] f32 out;  rec_mass (device) [B] f32 out
 *   ws (device) >= lsa_chunk_mass_ws_bytes(g, Hq, n_steps) bytes
 * Supported: bf16 latent rows (Dk 576, v_off 0), Hq a multiple of 64,
 * 1 <= n_steps and n_steps * Hq <= 16384.
 * ---------------------------------------------------------------------- */
size_t lsa_chunk_mass_ws_bytes(const lsa_geom* g, int32_t Hq, int32_t n_steps);
lsa_status lsa_chunk_attn_mass(const lsa_geom* g, const void* q, int32_t Hq, int32_t n_steps,
                               const lsa_kv_layout* kv, const void* pages,
                               const int32_t* page_table, const void* recent, float sm_scale,
                               float* mass, float* rec_mass, void* ws, size_t ws_bytes,
                               void* stream);

/* ------------------------------------------------------------------------
 * a4. Slot pool and candidate fetch.  Selected chunks move from the cold
 * pool (CPU memory) into GPU memory; the rest stay behind (cjcn.com.cn
 * section 二 and Q&A 1; gist.science 2.1 "Dynamisches Fetching").
 * The pool gives request r the slots [r*slots_per_req, (r+1)*slots_per_req)
 * of slot_mem (device, B*slots_per_req*page_bytes bytes, caller-owned).  The
 * cold tier holds page (chunk_off[r] + c) for every history chunk; it is
 * host memory (cold_on_host = 1; pinned memory is fastest for the host's
 * packing copies) or device memory (0).  For the host tier a gather packs
 * the missing chunks on the host into pinned staging (up to 1,024 chunks per
 * batch, several threads) and sends each batch with one DMA copy, then
 * scatters it into the slots on the device; for the device tier it copies
 * with one kernel launch.  Both run on the copy stream.
 * lsa_pool_create allocates only host bookkeeping and one small device copy
 * list; it borrows slot_mem and cold until lsa_pool_destroy.
 * ---------------------------------------------------------------------- */
typedef struct lsa_pool lsa_pool;

typedef struct {
    int64_t fetched;  /* chunks copied by the last gather                 */
    int64_t resident; /* chunks resident after it                         */
    int64_t evicted;  /* chunks released by it                            */
    int64_t copies;   /* packed batches (host tier) or copy launches        */
    int64_t bytes;    /* bytes copied                                     */
} lsa_gather_stats;

lsa_status lsa_pool_create(lsa_pool** pool, const lsa_geom* g, void* slot_mem,
                           int32_t slots_per_req, int64_t page_bytes, const void* cold,
                           int32_t cold_on_host);
void lsa_pool_destroy(lsa_pool* pool);

/* Make the chunks in (sel_ids, sel_cnt) resident while keeping the chunks in
 * (keep_ids, keep_cnt) -- the selection in use by the running window --
 * untouched.  Every other resident chunk is released.  Missing chunks are
 * copied on copy_stream after it waits on wait_event (if not NULL: the event
 * marking that released slots are no longer read).  Then page_table (device,
 * [sum N] int32) is rewritten for the new selection (slot index, or -1 for
 * chunks not selected) and done_event (if not NULL) is recorded on
 * copy_stream.  All id arrays are host arrays in the lsa_select_threshold
 * layout; keep_* may be NULL (nothing to keep).  If the selection and the
 * kept set together exceed a request's slots, LSA_ERR_CAPACITY is returned
 * and the pool is unchanged.  Only one gather per pool may be in flight; the
 * host part runs synchronously. */
lsa_status lsa_gather_kv(lsa_pool* pool, const int32_t* sel_ids, const int32_t* sel_cnt,
                         const int32_t* keep_ids, const int32_t* keep_cnt, int32_t* page_table,
                         void* copy_stream, void* wait_event, void* done_event,
                         lsa_gather_stats* stats);

/* ------------------------------------------------------------------------
 * a1+a8. The window pipeline.  The indexer fires every 64 generation steps
 * and predicts the history the next 64 steps need (cjcn.com.cn section 二;
 * gist.science 2.1 "Periodische Triggerung").  A context binds the static
 * inputs; lsa_ctx_prime scores and fetches the first window; each
 * lsa_step64 call then runs the decode steps of the current window
 * (refine + top-k + attention per step) on main_stream while it scores the
 * next window (if given), fetches its missing chunks on copy_stream, and
 * builds its page table.  One window ahead, so a window's refill overlaps
 * the previous window's steps.  With n_layers > 1 each trigger scores every
 * layer's KIComp against that layer's query (one lsa_trigger_in per layer)
 * and selects the OR union of their selections, as lsa_score_chunks_union
 * followed by lsa_select_threshold does (cjcn.com.cn explainer, section 四;
 * gist.science summary, section 2.4).
 *
 * Growing context (growing != 0).  Decode adds one token per step and, as
 * the context grows, the recent region's oldest full chunk joins the history
 * at each trigger (cjcn.com.cn explainer, section 二).  The geometry then
 * needs chunk_cap > 0 and recent_cap >= 2 * Rmax, where
 *     Rmax = max(W + 63, max_r R_r) + 64
 * bounds the recent rows of a request during any window (R_r as given).
 * For window m (steps s, L_r and rs_r as lsa_ctx_state reports at the call):
 *   - request r commits chunk N_r = rs_r / C iff R_r + s >= W + C; its
 *     KV rows are recent tokens [rs_r, rs_r + C), already present;
 *   - the next trigger (in->next) scores the history with the chunks
 *     committed in this window included, so the pages of those chunks are
 *     written at the start of the call: KV rows from the recent region,
 *     in->commit_ikeys[r] at kv.ikey_off, in->commit_ikey_scale[r] into
 *     desc->ikey_scale (fp8) -- the library writes the pool's cold tier
 *     and desc->ikey_scale, which the caller keeps writable;
 *   - the caller writes each committing chunk's KIComp row (and fp8 scale)
 *     into the next trigger's kic arrays, row chunk_off[r] + N_r of every
 *     layer, before the call (on main_stream or earlier);
 *   - step j appends in->new_rows[j][r] as token L_r + j of request r and
 *     attends over the grown recent region (desc->recent is written too);
 *   - at the window's end a committing request's history boundary moves to
 *     rs_r + C: those rows leave the recent region and are attended from
 *     then on only when a later trigger selects their chunk.
 * The recent rows of request r slide inside its recent_cap rows (the row
 * of token t is r * recent_cap + recent_first_r + t - rs_r); when a window
 * would run past the end they move back to the start, in one copy.
 * ---------------------------------------------------------------------- */
typedef struct lsa_ctx lsa_ctx;

typedef struct {
    lsa_geom geom;
    int32_t H, d;             /* indexer heads and dim                       */
    lsa_dtype q_dt, idx_dt;   /* indexer query dtype, index key dtype         */
    int32_t Hq, k;            /* attention heads, top-k                       */
    lsa_kv_layout kv;         /* KV row and page layout                       */
    float sm_scale, theta;    /* softmax scale, logit threshold (0 = sig 0.5) */
    const void* recent;       /* (device) [sum R, row_bytes]                  */
    const float* ikey_scale;  /* (device) [sum N] (fp8 index keys), else NULL */
    lsa_pool* pool;           /* slot pool (its cold tier holds the pages)    */
    void* ws;                 /* (device) >= lsa_ctx_ws_bytes(desc) bytes     */
    size_t ws_bytes;
    int32_t n_layers;         /* indexer layers whose OR union each trigger
                                 selects (the pages' inference configuration
                                 runs three), 1..LSA_MAX_LAYERS; 0 means 1    */
    int32_t growing;          /* nonzero: growing context (see above)          */
} lsa_ctx_desc;

typedef struct {
    const void* kic;          /* (device) [sum N, d] KIComp for this scoring  */
    const float* kic_scale;   /* (device) [sum N] or NULL                      */
    const void* q;            /* (device) [B, H, d] coarse query               */
    const float* w;           /* (device) [B, H]                               */
    const float* bias;        /* (device) [B]                                  */
} lsa_trigger_in;

typedef struct {
    int32_t steps;            /* decode steps in this window, 1..64           */
    const void* q_refine;     /* (device) [steps, B, H, d] q_dt               */
    const float* w_refine;    /* (device) [steps, B, H]                        */
    const void* q_attn;       /* (device) [steps, B, Hq, Dk] kv dtype          */
    const lsa_trigger_in* next; /* (host) next window's trigger, one per indexer
                                   layer (n_layers of them), or NULL (last window) */
    /* growing context only (else ignored):                                    */
    const void* new_rows;     /* (device) [steps, B, row_bytes] appended tokens */
    const void* commit_ikeys; /* (device) [B, C, d] idx_dt: index keys of the
                                 chunk each committing request moves to its
                                 history (rows of other requests unread)     */
    const float* commit_ikey_scale; /* (device) [B] fp8 index keys, else NULL */
} lsa_window_in;

typedef struct {
    void* out;                /* (device) [steps, B, Hq, Dv] kv dtype          */
    float* lse;               /* (device) [steps, B, Hq] or NULL               */
    int32_t* topk_idx;        /* (device) [steps, B, k] or NULL                */
    int32_t* topk_cnt;        /* (device) [steps, B] or NULL                   */
    int32_t* sel_cnt;         /* (host) [B] or NULL: the next window's counts  */
    lsa_gather_stats stats;   /* the next window's fetch                       */
} lsa_window_out;

size_t lsa_ctx_ws_bytes(const lsa_ctx_desc* desc);
lsa_status lsa_ctx_create(lsa_ctx** ctx, const lsa_ctx_desc* desc);
void lsa_ctx_destroy(lsa_ctx* ctx);
/* Score, select and fetch the first window (synchronous on the host);
 * first points to one lsa_trigger_in per indexer layer. */
lsa_status lsa_ctx_prime(lsa_ctx* ctx, const lsa_trigger_in* first, void* main_stream,
                         void* copy_stream, lsa_window_out* out);
lsa_status lsa_step64(lsa_ctx* ctx, const lsa_window_in* in, lsa_window_out* out,
                      void* main_stream, void* copy_stream);
/* The context's lengths as of now (host arrays [B], each may be NULL):
 * seq_len L_r, hist_tokens rs_r and recent_first_r (the recent region's
 * first row within request r's recent_cap rows; 0 without growing).  A
 * growing window that would take a history past chunk_cap returns
 * LSA_ERR_CAPACITY from lsa_step64 before it launches anything. */
lsa_status lsa_ctx_state(const lsa_ctx* ctx, int32_t* seq_len, int32_t* hist_tokens,
                         int32_t* recent_first);

/* ------------------------------------------------------------------------
 * Diagnostics: per-kernel timing.  While enabled, every kernel the library
 * launches is bracketed by two hipEvents recorded on the stream it is
 * launched on (adds a little launch overhead).  lsa_timing_read waits for
 * the recorded events and returns, for one kernel name (k_score,
 * k_select, k_select_tiles, k_refine, k_topk, k_refine_mfma, k_band_fine,
 * k_band_list, k_topk_band, k_attn_mla, k_attn_f32, k_attn_merge,
 * k_gather, k_stream_read, k_score_sig, k_select_ranked, k_chunk_ml, k_append_kv,
 * k_commit_chunk, k_commit_page, k_compact_recent, k_resolve_sel, k_key_norm2), the
 * number of timed launches and
 * their summed duration in
 * milliseconds since the last reset.  lsa_timing_only(name) restricts the
 * timing to that one kernel (NULL: all; a name of 64 or more characters is
 * LSA_ERR_INVALID_ARG), so that one kernel can be timed inside a run with
 * little disturbance.  lsa_timing_every(n) brackets only every n-th launch
 * of each timed kernel (n >= 1; 1 is the default), which spreads the events'
 * own cost (a few microseconds per record on this GPU) over n launches.
 * The events skip the system-scope fence.  Process-wide; the hooks are
 * thread-safe.
 * ---------------------------------------------------------------------- */
lsa_status lsa_timing_enable(int32_t on);
lsa_status lsa_timing_only(const char* kernel);
lsa_status lsa_timing_every(int32_t n);
void lsa_timing_reset(void);
lsa_status lsa_timing_read(const char* kernel, int64_t* launches, double* total_ms);

/* ------------------------------------------------------------------------
 * Diagnostics: launch-shape overrides.  Each knob replaces one launch-shape
 * choice of the library, process-wide, until set again; a value < 0 restores
 * the library's own choice.  They exist so that tests reach rarely taken
 * kernel paths at small sizes, and for measurement sweeps; the results of
 * every entry point stay as documented under any setting.
 *   LSA_TUNE_REFINE_BLOCKS    blocks per request of the matrix-core refine
 *                             pass (>= 1; fewer blocks make each of its waves
 *                             walk more chunks)
 *   LSA_TUNE_ATTN_PAIR_POLLS  polls of the bf16 attention kernel's bounded
 *                             wait for its partner wave (>= 0).  A wait that
 *                             runs out is reported through lsa_device_status
 *                             and lsa_step64 (LSA_ERR_HIP) and leaves that
 *                             launch's output undefined; 0 makes every wait
 *                             run out at once, which tests that report.
 * Returns LSA_ERR_INVALID_ARG for an unknown knob or an invalid value.
 * ---------------------------------------------------------------------- */
typedef enum {
    LSA_TUNE_REFINE_BLOCKS = 0,
    LSA_TUNE_ATTN_PAIR_POLLS = 1,
    LSA_TUNE_COUNT_ = 2
} lsa_tune_knob;
lsa_status lsa_tune_set(lsa_tune_knob knob, int32_t value);

/* ------------------------------------------------------------------------
 * Device-side error report.  A kernel whose bounded wait runs out (the bf16
 * attention kernel's wait for its partner wave; see LSA_TUNE_ATTN_PAIR_POLLS)
 * records that in a word that each GPU holds for the library, instead of
 * returning a wrong result silently.  lsa_device_status waits for `stream`
 * (NULL: the default stream), then returns LSA_OK if the current device's
 * word is clear, or LSA_ERR_HIP if any kernel of the library set it since the
 * last call, and clears it.  flags (host, nullable) receives the word:
 *   bit 0  an attention pair wait ran out (that launch's output is undefined)
 * lsa_step64 takes the word over at the end of each window (reads and clears
 * it on the main stream) and returns LSA_ERR_HIP from the next call when that
 * window set it; the window's own outputs are then undefined.  Library calls
 * running on other streams of the same device meanwhile share the word.
 * ---------------------------------------------------------------------- */
lsa_status lsa_device_status(void* stream, uint32_t* flags);

/* ------------------------------------------------------------------------
 * Diagnostics: achievable read bandwidth.  Reads `bytes` of device memory at
 * src (16-byte aligned, a multiple of 16) with a plain streaming kernel
 * (k_stream_read) and writes nothing but, practically never, one word to
 * sink (device, 4 bytes).  Time it with lsa_timing_* or events: bytes over
 * its duration is the read bandwidth a simple kernel reaches on this GPU,
 * the reference line for the HBM figures of the kernels above.
 * ---------------------------------------------------------------------- */
lsa_status lsa_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LSA_H_ */
