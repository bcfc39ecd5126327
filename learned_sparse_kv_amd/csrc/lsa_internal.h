// Internal declarations of the LSA HIP library (gfx950).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lsa.h"

// Batch geometry derived on the host and passed by value to every kernel
// (B <= LSA_MAX_BATCH keeps it well under the kernel-argument limit).
struct GeomDev {
    int32_t B;
    int32_t W;
    int32_t L[LSA_MAX_BATCH];
    int32_t rs[LSA_MAX_BATCH];       // first recent token
    int32_t nhist[LSA_MAX_BATCH];    // history chunks
    int32_t nrec[LSA_MAX_BATCH];     // recent tokens
    int32_t tile_off[LSA_MAX_BATCH + 1];   // prefix of ceil(nhist/64) (score tiles)
    int64_t chunk_off[LSA_MAX_BATCH + 1];  // prefix of nhist
    int64_t rec_off[LSA_MAX_BATCH + 1];    // prefix of nrec
};

// Fills d from the caller's geometry; returns LSA_OK or LSA_ERR_INVALID_ARG.
lsa_status geom_derive(const lsa_geom* g, GeomDev* d);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- launchers (each returns the launch error) ----
hipError_t launch_fuse_query(const GeomDev& g, const void* q, lsa_dtype q_dt, const float* w,
                             int H, int d, float* qbar, hipStream_t s);
// Chunk logits; with tmask the kernel also records, per tile of 64 chunks
// (tile_off order), the mask of z > theta and its count, for
// launch_select_tiles.
hipError_t launch_score(const GeomDev& g, const void* kic, lsa_dtype kdt, const float* kscale,
                        const float* qbar, const float* bias, int d, float* z, hipStream_t s,
                        bool combine = false, float theta = 0.0f, uint64_t* tmask = nullptr,
                        int32_t* tcount = nullptr);
hipError_t launch_select_tiles(const GeomDev& g, const uint64_t* tmask, const int32_t* tcount,
                               int32_t* sel, int32_t* cnt, hipStream_t s);
hipError_t launch_score_sig(const GeomDev& g, const void* kic, lsa_dtype kdt, const float* kscale,
                            const void* q, lsa_dtype q_dt, const float* w, int H, const float* bias,
                            float theta, int d, float* S, hipStream_t s);
hipError_t launch_select(const GeomDev& g, const float* z, float theta, int32_t* sel,
                         int32_t* cnt, hipStream_t s);

hipError_t launch_refine(const GeomDev& g, const int32_t* sel, const int32_t* cnt,
                         const void* pages, int64_t page_bytes, int64_t ikey_off,
                         const int32_t* page_table, lsa_dtype idx_dt, const float* ikey_scale,
                         const void* q, lsa_dtype q_dt, const float* w, int H, int d,
                         float* scores, int grid_hint, hipStream_t s);
hipError_t launch_topk(const GeomDev& g, const int32_t* sel, const int32_t* cnt,
                       const float* scores, int k, int32_t* topk, int32_t* tcnt, hipStream_t s);

hipError_t launch_append_kv(const GeomDev& g, const void* rows, int64_t row_bytes, void* recent,
                            hipStream_t s);
hipError_t launch_commit_chunk(const GeomDev& g, int64_t row_bytes, int64_t page_bytes, int64_t ikey_off,
                               const void* rsrc, void* rdst, void* cold, int64_t key_row_bytes,
                               const void* new_ikeys, const float* new_iks, float* ikey_scale,
                               const void* new_kic, const float* new_kcs, void* kic, float* kic_scale,
                               bool fp8, hipStream_t s);
// The window pipeline's growing context: which requests commit a chunk in
// the window, and the recent rows moved back to the start of their area.
struct CommitSet {
    int32_t on[LSA_MAX_BATCH];
};
struct RecentMoves {
    int64_t src[LSA_MAX_BATCH], dst[LSA_MAX_BATCH];  // first rows
    int32_t n[LSA_MAX_BATCH];                        // rows (0: none)
};
hipError_t launch_commit_page(const GeomDev& g, const CommitSet& f, int64_t row_bytes,
                              int64_t page_bytes, int64_t ikey_off, const void* recent, void* cold,
                              int64_t key_row_bytes, const void* ikeys, const float* iks,
                              float* ikey_scale, hipStream_t s);
hipError_t launch_compact_recent(int B, const RecentMoves& m, int64_t row_bytes, void* recent,
                                 hipStream_t s);

// Per-request keep counts of lsa_select_ranked (by value).
struct RankCounts {
    int32_t m[LSA_MAX_BATCH];
};
// Pseudo-chunks of the attention-mass pass: the history chunks, then the
// recent window cut into 64-token pieces; offsets of each request's
// (m, l) partials and recent-window pieces.
struct MassGeom {
    int32_t nc[LSA_MAX_BATCH];
    int32_t rc_off[LSA_MAX_BATCH];
    int64_t ml_off[LSA_MAX_BATCH];
    int64_t ml_total;
    int64_t rc_total;
};
void mass_geom(const GeomDev& g, int Hq, int n_steps, MassGeom* mg);
hipError_t launch_select_ranked(const GeomDev& g, const void* keys, int kind, const RankCounts& m,
                                int32_t* sel, int32_t* cnt, hipStream_t s);
hipError_t launch_chunk_mass(const GeomDev& g, const MassGeom& mg, const void* q, int Hq, int n_steps,
                             const void* pages, int64_t page_bytes, const int32_t* page_table,
                             const void* recent, int64_t row_bytes, float sm_scale, float* mass,
                             float* rec, float2* ml, float* lse2, float* recbuf, hipStream_t s);

struct AttnPlan {
    int mode;        // 0: f32 VALU, 1: bf16 MFMA latent 576/512
    int n_splits;    // splits per request
    int per_split;   // positions per split (multiple of the tile)
    int head_groups; // WGs per (request, split) along heads
    int waves;       // waves per WG (mode 1)
    int P_max;       // k + max recent
    size_t part_o_bytes, part_ml_bytes;
};
lsa_status attn_plan(const GeomDev& g, const lsa_kv_layout* kv, int Hq, int k, int n_splits,
                     AttnPlan* plan);
hipError_t launch_attn(const GeomDev& g, const AttnPlan& plan, const void* q, int Hq,
                       const lsa_kv_layout& kv, const void* pages, const int32_t* page_table,
                       const void* recent, const int32_t* topk, const int32_t* tcnt, int k,
                       float sm_scale, void* out, float* lse, void* ws, hipStream_t s);

hipError_t launch_gather(const int32_t* pairs, int n_pairs, const void* src, void* dst,
                         int64_t page_bytes, hipStream_t s);

// Device address of the attention scratch array of the current device
// (nullptr if it cannot be had) and its size.
void* attn_scratch();
size_t attn_scratch_bytes();

// Device slot memory of a pool (pages of the resident chunks).
void* lsa_pool_slots(const lsa_pool* p);
int64_t lsa_pool_page_bytes(const lsa_pool* p);
int32_t lsa_pool_batch(const lsa_pool* p);
void* lsa_pool_cold(const lsa_pool* p);
// A grown history: the pool takes the new chunk counts (nhist) of g; chunks
// beyond the old counts start not resident.  Host only.
lsa_status pool_grow(lsa_pool* p, const GeomDev& g);
// tile_off of g from its nhist (after the history counts change)
void geom_retile(GeomDev* g);

// Launch-shape override of lsa_tune_set (-1: the library's own choice).
int tune_get(lsa_tune_knob knob);
// The current device's error word (kernels OR flags into it), or nullptr if
// its address cannot be had.
uint32_t* dev_err_word();

// Per-kernel event timing hooks (no-ops unless lsa_timing_enable(1)).
void timing_begin(const char* name, hipStream_t s);
void timing_end(const char* name, hipStream_t s);

// Matrix-core refine with an exact re-score band (refine_band.hip).
bool band_supported(lsa_dtype idx_dt, lsa_dtype q_dt, int H, int d);
size_t band_ws_bytes(const GeomDev& g);
// A growing context's new KV rows, one per request (rows: B * n16 16-byte
// units), for the band's fine-histogram pass to write at the end of each
// request's recent rows (row rec_off[r] + nrec[r] - 1); rows null: none.
struct AppendRow {
    const uint8_t* rows = nullptr;
    uint8_t* recent = nullptr;
    int32_t n16 = 0;  // 16-byte units per row, at most 256
};
hipError_t launch_refine_band(const GeomDev& g, const int32_t* sel, const int32_t* cnt,
                              const void* pages, int64_t page_bytes, int64_t ikey_off,
                              const int32_t* page_table, lsa_dtype idx_dt,
                              const float* ikey_scale, const int32_t* sel_slot,
                              const float* sel_scale, const float* kn2, const void* q,
                              const float* w, int H, int d, int k, int32_t* topk, int32_t* tcnt,
                              void* ws, bool ws_clean, hipStream_t s,
                              const AppendRow& app = AppendRow());
// |key|^2 of every token of the selected chunks (selection order, 64 per
// chunk) for launch_refine_band's kn2 (nullptr: formed there per step).
hipError_t launch_key_norm2(const GeomDev& g, const int32_t* cnt, const int32_t* sel_slot,
                            const void* pages, int64_t page_bytes, int64_t ikey_off,
                            lsa_dtype idx_dt, int d, float* kn2, hipStream_t s);
// sel_slot / sel_scale: pages and scales of the selected chunks in selection
// order (-1 past the count), for launch_refine_band (nullptr: looked up there).
hipError_t launch_resolve_sel(const GeomDev& g, const int32_t* sel, const int32_t* cnt,
                              const int32_t* page_table, const float* ikey_scale,
                              int32_t* sel_slot, float* sel_scale, hipStream_t s);
// Zeroes the part of a band workspace that must start at zero (every band
// launch leaves it zero again).
hipError_t launch_band_clear(const GeomDev& g, void* ws, hipStream_t s);
