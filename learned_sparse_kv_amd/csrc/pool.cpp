// HBM slot pool and candidate fetch.
//
// Selected chunks move from the cold pool into GPU memory and the rest stay
// in the cold pool (cjcn.com.cn explainer, section 二 and Q&A 1;
// gist.science summary, section 2.1 "Dynamisches Fetching").  The pool keeps
// a chunk -> slot table per request on the host.  A gather releases every
// resident chunk outside (new selection U kept selection), gives each
// missing chunk the lowest free slot of its request, and copies them on the
// copy stream.  Device cold tier: one k_gather launch (one block per chunk).
// Host cold tier: the host packs the missing chunks into a pinned staging
// buffer (several threads), one DMA copy takes the whole batch across the
// host link, and k_gather scatters it from device staging into the slots.
// One DMA command per scattered chunk would cost about 11 us of command
// overhead each (a few hundred per window), and a kernel reading host memory
// would hold compute units for the whole transfer; the packed copy runs at
// the link's rate on the copy engine.  The page table for the new selection
// then goes up from pinned staging on the same stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <thread>
#include <vector>

#include "lsa_internal.h"

struct lsa_pool {
    GeomDev g;
    int32_t spr = 0;
    int64_t page_bytes = 0;
    uint8_t* slots = nullptr;
    const uint8_t* cold = nullptr;
    int32_t on_host = 0;
    std::vector<std::vector<int32_t>> chunk_slot;  // [r][c] slot within r, or -1
    std::vector<std::vector<int32_t>> slot_chunk;  // [r][s] chunk, or -1
    std::vector<std::vector<uint8_t>> mark;        // scratch marks [r][c]
    int32_t* h_pairs = nullptr;                    // pinned [B*spr*2]
    int32_t* d_pairs = nullptr;                    // device [B*spr*2]
    int32_t* h_pt = nullptr;                       // pinned [sum N]
    hipEvent_t staging_done = nullptr;
    bool staging_pending = false;
    // host tier: packed batches of missing chunks
    uint8_t* h_stage = nullptr;    // pinned [kStageChunks * page_bytes]
    uint8_t* d_stage = nullptr;    // device [kStageChunks * page_bytes]
    int32_t* h_spairs = nullptr;   // pinned [kStageChunks * 2]: (staging index, slot)
    int32_t* d_spairs = nullptr;   // device copy
    hipEvent_t stage_done = nullptr;  // the last batch's uploads have read h_stage
    bool stage_pending = false;
};

namespace {

constexpr int kStageChunks = 1024;  // chunks per packed batch (84 MB at 82 KB pages)
constexpr int kPackThreads = 8;

// dst[i] = src + idx[i] * pb for i in [0, n): contiguous ranges per thread
void pack_chunks(uint8_t* dst, const uint8_t* src, const int32_t* pairs, int n, int64_t pb) {
    auto work = [&](int a, int b) {
        for (int i = a; i < b; ++i) std::memcpy(dst + (int64_t)i * pb, src + (int64_t)pairs[2 * i] * pb, pb);
    };
    const int nt = std::max(1, std::min(kPackThreads, n / 16));
    if (nt == 1) {
        work(0, n);
        return;
    }
    std::vector<std::thread> th;
    th.reserve(nt - 1);
    const int per = (n + nt - 1) / nt;
    for (int t = 1; t < nt; ++t) th.emplace_back(work, std::min(n, t * per), std::min(n, (t + 1) * per));
    work(0, std::min(n, per));
    for (auto& x : th) x.join();
}

}  // namespace

void* lsa_pool_slots(const lsa_pool* p) { return p ? p->slots : nullptr; }
int64_t lsa_pool_page_bytes(const lsa_pool* p) { return p ? p->page_bytes : 0; }
int32_t lsa_pool_batch(const lsa_pool* p) { return p ? p->g.B : 0; }
void* lsa_pool_cold(const lsa_pool* p) { return p ? (void*)p->cold : nullptr; }

lsa_status pool_grow(lsa_pool* p, const GeomDev& g) {
    if (!p || g.B != p->g.B) return LSA_ERR_INVALID_ARG;
    for (int r = 0; r < g.B; ++r) {
        if (g.chunk_off[r] != p->g.chunk_off[r] || g.nhist[r] < p->g.nhist[r]) return LSA_ERR_INVALID_ARG;
        if (g.nhist[r] > p->g.chunk_off[r + 1] - p->g.chunk_off[r]) return LSA_ERR_INVALID_ARG;
    }
    for (int r = 0; r < g.B; ++r) {
        p->chunk_slot[r].resize(g.nhist[r], -1);
        p->mark[r].resize(g.nhist[r], 0);
        p->g.nhist[r] = g.nhist[r];
        p->g.L[r] = g.L[r];
        p->g.rs[r] = g.rs[r];
    }
    return LSA_OK;
}

extern "C" {

lsa_status lsa_pool_create(lsa_pool** pool, const lsa_geom* g, void* slot_mem,
                           int32_t slots_per_req, int64_t page_bytes, const void* cold,
                           int32_t cold_on_host) {
    if (!pool) return LSA_ERR_INVALID_ARG;
    *pool = nullptr;
    GeomDev gd;
    lsa_status st = geom_derive(g, &gd);
    if (st != LSA_OK) return st;
    if (slots_per_req < 1 || page_bytes < 16 || page_bytes % 16) return LSA_ERR_INVALID_ARG;
    if (!slot_mem || (!cold && gd.chunk_off[gd.B] > 0)) return LSA_ERR_INVALID_ARG;
    if (((uintptr_t)slot_mem & 15u) || ((uintptr_t)cold & 15u)) return LSA_ERR_INVALID_ARG;
    if ((int64_t)gd.B * slots_per_req > INT32_MAX / 2) return LSA_ERR_INVALID_ARG;
    lsa_pool* p = new (std::nothrow) lsa_pool();
    if (!p) return LSA_ERR_INVALID_ARG;
    p->g = gd;
    p->spr = slots_per_req;
    p->page_bytes = page_bytes;
    p->slots = (uint8_t*)slot_mem;
    p->cold = (const uint8_t*)cold;
    p->on_host = cold_on_host ? 1 : 0;
    p->chunk_slot.resize(gd.B);
    p->slot_chunk.resize(gd.B);
    p->mark.resize(gd.B);
    for (int r = 0; r < gd.B; ++r) {
        p->chunk_slot[r].assign(gd.nhist[r], -1);
        p->slot_chunk[r].assign(slots_per_req, -1);
        p->mark[r].assign(gd.nhist[r], 0);
    }
    const size_t npairs = (size_t)gd.B * slots_per_req;
    const size_t nh = (size_t)(gd.chunk_off[gd.B] > 0 ? gd.chunk_off[gd.B] : 1);
    if (hipHostMalloc((void**)&p->h_pairs, npairs * 2 * sizeof(int32_t), hipHostMallocDefault) != hipSuccess ||
        hipHostMalloc((void**)&p->h_pt, nh * sizeof(int32_t), hipHostMallocDefault) != hipSuccess ||
        hipMalloc((void**)&p->d_pairs, npairs * 2 * sizeof(int32_t)) != hipSuccess ||
        hipEventCreateWithFlags(&p->staging_done, hipEventDisableTiming) != hipSuccess) {
        lsa_pool_destroy(p);
        return LSA_ERR_HIP;
    }
    if (p->on_host &&
        (hipHostMalloc((void**)&p->h_stage, (size_t)kStageChunks * page_bytes, hipHostMallocDefault) != hipSuccess ||
         hipMalloc((void**)&p->d_stage, (size_t)kStageChunks * page_bytes) != hipSuccess ||
         hipHostMalloc((void**)&p->h_spairs, (size_t)kStageChunks * 2 * sizeof(int32_t), hipHostMallocDefault) != hipSuccess ||
         hipMalloc((void**)&p->d_spairs, (size_t)kStageChunks * 2 * sizeof(int32_t)) != hipSuccess ||
         hipEventCreateWithFlags(&p->stage_done, hipEventDisableTiming) != hipSuccess)) {
        lsa_pool_destroy(p);
        return LSA_ERR_HIP;
    }
    *pool = p;
    return LSA_OK;
}

void lsa_pool_destroy(lsa_pool* p) {
    if (!p) return;
    if (p->staging_done) {
        if (p->staging_pending) (void)hipEventSynchronize(p->staging_done);
        (void)hipEventDestroy(p->staging_done);
    }
    if (p->stage_done) {
        if (p->stage_pending) (void)hipEventSynchronize(p->stage_done);
        (void)hipEventDestroy(p->stage_done);
    }
    if (p->h_pairs) (void)hipHostFree(p->h_pairs);
    if (p->h_pt) (void)hipHostFree(p->h_pt);
    if (p->d_pairs) (void)hipFree(p->d_pairs);
    if (p->h_stage) (void)hipHostFree(p->h_stage);
    if (p->d_stage) (void)hipFree(p->d_stage);
    if (p->h_spairs) (void)hipHostFree(p->h_spairs);
    if (p->d_spairs) (void)hipFree(p->d_spairs);
    delete p;
}

lsa_status lsa_gather_kv(lsa_pool* p, const int32_t* sel_ids, const int32_t* sel_cnt,
                         const int32_t* keep_ids, const int32_t* keep_cnt, int32_t* page_table,
                         void* copy_stream, void* wait_event, void* done_event,
                         lsa_gather_stats* stats) {
    if (!p || !sel_cnt || !page_table) return LSA_ERR_INVALID_ARG;
    const GeomDev& g = p->g;
    const int64_t nh = g.chunk_off[g.B];
    if (nh > 0 && !sel_ids) return LSA_ERR_INVALID_ARG;
    if ((keep_ids == nullptr) != (keep_cnt == nullptr)) return LSA_ERR_INVALID_ARG;
    // ---- validate everything and check capacity before touching the pool ----
    for (int r = 0; r < g.B; ++r) {
        const int n = g.nhist[r];
        const int32_t* s = sel_ids + g.chunk_off[r];
        if (sel_cnt[r] < 0 || sel_cnt[r] > n) return LSA_ERR_INVALID_ARG;
        for (int i = 0; i < sel_cnt[r]; ++i)
            if (s[i] < 0 || s[i] >= n || (i > 0 && s[i] <= s[i - 1])) return LSA_ERR_INVALID_ARG;
        int need = sel_cnt[r];
        std::vector<uint8_t>& mk = p->mark[r];
        for (int i = 0; i < sel_cnt[r]; ++i) mk[s[i]] = 1;
        if (keep_ids) {
            const int32_t* kp = keep_ids + g.chunk_off[r];
            if (keep_cnt[r] < 0 || keep_cnt[r] > n) {
                for (int i = 0; i < sel_cnt[r]; ++i) mk[s[i]] = 0;
                return LSA_ERR_INVALID_ARG;
            }
            for (int i = 0; i < keep_cnt[r]; ++i) {
                const int32_t c = kp[i];
                if (c >= 0 && c < n && !mk[c] && p->chunk_slot[r][c] >= 0) {
                    mk[c] = 2;
                    ++need;
                }
            }
            for (int i = 0; i < keep_cnt[r]; ++i) {
                const int32_t c = kp[i];
                if (c >= 0 && c < n && mk[c] == 2) mk[c] = 0;
            }
        }
        for (int i = 0; i < sel_cnt[r]; ++i) mk[s[i]] = 0;
        if (need > p->spr) return LSA_ERR_CAPACITY;
    }
    if (p->staging_pending) {
        if (hipEventSynchronize(p->staging_done) != hipSuccess) return LSA_ERR_HIP;
        p->staging_pending = false;
    }
    // ---- update residency ----
    lsa_gather_stats st{};
    int npairs = 0;
    for (int r = 0; r < g.B; ++r) {
        const int n = g.nhist[r];
        const int32_t* s = sel_ids + g.chunk_off[r];
        std::vector<uint8_t>& mk = p->mark[r];
        std::vector<int32_t>& cs = p->chunk_slot[r];
        std::vector<int32_t>& sc = p->slot_chunk[r];
        for (int i = 0; i < sel_cnt[r]; ++i) mk[s[i]] = 1;
        if (keep_ids) {
            const int32_t* kp = keep_ids + g.chunk_off[r];
            for (int i = 0; i < keep_cnt[r]; ++i)
                if (kp[i] >= 0 && kp[i] < n) mk[kp[i]] |= 2;
        }
        for (int sl = 0; sl < p->spr; ++sl) {
            const int32_t c = sc[sl];
            if (c >= 0 && !mk[c]) {
                sc[sl] = -1;
                cs[c] = -1;
                ++st.evicted;
            }
        }
        int cursor = 0;
        for (int i = 0; i < sel_cnt[r]; ++i) {
            const int32_t c = s[i];
            if (cs[c] >= 0) continue;
            while (sc[cursor] >= 0) ++cursor;  // capacity was checked above
            sc[cursor] = c;
            cs[c] = cursor;
            p->h_pairs[2 * npairs] = (int32_t)(g.chunk_off[r] + c);
            p->h_pairs[2 * npairs + 1] = r * p->spr + cursor;
            ++npairs;
        }
        for (int i = 0; i < sel_cnt[r]; ++i) mk[s[i]] = 0;
        if (keep_ids) {
            const int32_t* kp = keep_ids + g.chunk_off[r];
            for (int i = 0; i < keep_cnt[r]; ++i)
                if (kp[i] >= 0 && kp[i] < n) mk[kp[i]] = 0;
        }
        for (int sl = 0; sl < p->spr; ++sl) st.resident += sc[sl] >= 0;
    }
    st.fetched = npairs;
    st.bytes = (int64_t)npairs * p->page_bytes;
    // ---- copies on the copy stream ----
    hipStream_t cs = (hipStream_t)copy_stream;
    if (wait_event && hipStreamWaitEvent(cs, (hipEvent_t)wait_event, 0) != hipSuccess)
        return LSA_ERR_HIP;
    if (npairs > 0 && !p->on_host) {
        if (hipMemcpyAsync(p->d_pairs, p->h_pairs, (size_t)npairs * 2 * sizeof(int32_t),
                           hipMemcpyHostToDevice, cs) != hipSuccess)
            return LSA_ERR_HIP;
        if (launch_gather(p->d_pairs, npairs, p->cold, p->slots, p->page_bytes, cs) != hipSuccess)
            return LSA_ERR_HIP;
        st.copies = 1;
    }
    for (int b0 = 0; p->on_host && b0 < npairs; b0 += kStageChunks) {
        const int n = std::min(kStageChunks, npairs - b0);
        if (p->stage_pending) {  // the previous batch's uploads still read h_stage
            if (hipEventSynchronize(p->stage_done) != hipSuccess) return LSA_ERR_HIP;
            p->stage_pending = false;
        }
        pack_chunks(p->h_stage, p->cold, p->h_pairs + 2 * b0, n, p->page_bytes);
        for (int i = 0; i < n; ++i) {
            p->h_spairs[2 * i] = i;
            p->h_spairs[2 * i + 1] = p->h_pairs[2 * (b0 + i) + 1];
        }
        if (hipMemcpyAsync(p->d_stage, p->h_stage, (size_t)n * p->page_bytes, hipMemcpyHostToDevice,
                           cs) != hipSuccess ||
            hipMemcpyAsync(p->d_spairs, p->h_spairs, (size_t)n * 2 * sizeof(int32_t),
                           hipMemcpyHostToDevice, cs) != hipSuccess ||
            hipEventRecord(p->stage_done, cs) != hipSuccess)
            return LSA_ERR_HIP;
        p->stage_pending = true;
        if (launch_gather(p->d_spairs, n, p->d_stage, p->slots, p->page_bytes, cs) != hipSuccess)
            return LSA_ERR_HIP;
        ++st.copies;
    }
    // ---- page table of the new selection ----
    if (nh > 0) {
        for (int64_t i = 0; i < nh; ++i) p->h_pt[i] = -1;
        for (int r = 0; r < g.B; ++r) {
            const int32_t* s = sel_ids + g.chunk_off[r];
            for (int i = 0; i < sel_cnt[r]; ++i)
                p->h_pt[g.chunk_off[r] + s[i]] = r * p->spr + p->chunk_slot[r][s[i]];
        }
        if (hipMemcpyAsync(page_table, p->h_pt, (size_t)nh * sizeof(int32_t),
                           hipMemcpyHostToDevice, cs) != hipSuccess)
            return LSA_ERR_HIP;
    }
    if (hipEventRecord(p->staging_done, cs) != hipSuccess) return LSA_ERR_HIP;
    p->staging_pending = true;
    if (done_event && hipEventRecord((hipEvent_t)done_event, cs) != hipSuccess) return LSA_ERR_HIP;
    if (stats) *stats = st;
    return LSA_OK;
}

}  // extern "C"
