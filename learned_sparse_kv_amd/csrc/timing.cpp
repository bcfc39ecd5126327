// Diagnostics: per-kernel timing with HIP events, and launch-shape overrides.
//
// When enabled, every kernel the library launches is bracketed by two
// events recorded on the stream it is launched on; lsa_timing_read
// synchronises them and returns the launch count and summed duration per
// kernel name.  Disabled (the default), the hooks cost one relaxed load.
//
// The overrides (lsa_tune_set) replace a launch-shape choice of the library
// process-wide, so that tests reach rarely taken kernel paths at small sizes
// and sweeps can try other shapes; -1 means the library's own choice.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "lsa_internal.h"

namespace {

struct Pair {
    hipEvent_t a, b;
};

std::atomic<int> g_on{0};
std::atomic<int> g_every{1};     // bracket every n-th launch of a timed kernel
std::map<std::string, int64_t> g_seen;  // launches of each timed kernel (under g_mu)
std::atomic<int> g_filtered{0};  // time only the kernel named in g_only
char g_only[64] = {0};
std::mutex g_mu;
std::map<std::string, std::vector<Pair>> g_pending;
std::map<std::string, std::pair<int64_t, double>> g_done;
std::vector<hipEvent_t> g_free;  // recycled events (created once, reused)
thread_local hipEvent_t t_start = nullptr;
std::atomic<int> g_tune[LSA_TUNE_COUNT_] = {-1, -1};

hipEvent_t take_event() {
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (!g_free.empty()) {
            hipEvent_t e = g_free.back();
            g_free.pop_back();
            return e;
        }
    }
    // timing only: no system-scope fence (no cache writeback and invalidate
    // between the bracketed kernel and its neighbours)
    hipEvent_t e = nullptr;
    return hipEventCreateWithFlags(&e, hipEventDisableSystemFence) == hipSuccess ? e : nullptr;
}

}  // namespace

static bool wanted(const char* name) {
    return !g_filtered.load(std::memory_order_acquire) || std::strcmp(name, g_only) == 0;
}

void timing_begin(const char* name, hipStream_t s) {
    if (!g_on.load(std::memory_order_relaxed) || !wanted(name)) return;
    const int every = g_every.load(std::memory_order_relaxed);
    if (every > 1) {
        std::lock_guard<std::mutex> lk(g_mu);
        if (g_seen[name]++ % every != 0) return;
    }
    t_start = take_event();
    if (t_start) (void)hipEventRecord(t_start, s);
}

void timing_end(const char* name, hipStream_t s) {
    if (!g_on.load(std::memory_order_relaxed) || !t_start) return;
    hipEvent_t e = take_event();
    if (!e) return;
    (void)hipEventRecord(e, s);
    std::lock_guard<std::mutex> lk(g_mu);
    g_pending[name].push_back({t_start, e});
    t_start = nullptr;
}

static void drain() {
    for (auto& kv : g_pending) {
        auto& acc = g_done[kv.first];
        for (auto& p : kv.second) {
            float ms = 0.f;
            if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
                acc.first += 1;
                acc.second += ms;
            }
            g_free.push_back(p.a);
            g_free.push_back(p.b);
        }
    }
    g_pending.clear();
}

int tune_get(lsa_tune_knob knob) {
    return (int)knob >= 0 && (int)knob < LSA_TUNE_COUNT_ ? g_tune[knob].load(std::memory_order_relaxed) : -1;
}

extern "C" {

lsa_status lsa_tune_set(lsa_tune_knob knob, int32_t value) {
    if ((int)knob < 0 || (int)knob >= LSA_TUNE_COUNT_) return LSA_ERR_INVALID_ARG;
    if (knob == LSA_TUNE_REFINE_BLOCKS && value == 0) return LSA_ERR_INVALID_ARG;
    g_tune[knob].store(value < 0 ? -1 : value, std::memory_order_relaxed);
    return LSA_OK;
}

lsa_status lsa_timing_enable(int32_t on) {
    g_on.store(on ? 1 : 0);
    return LSA_OK;
}

lsa_status lsa_timing_every(int32_t n) {
    if (n < 1) return LSA_ERR_INVALID_ARG;
    g_every.store(n);
    return LSA_OK;
}

lsa_status lsa_timing_only(const char* kernel) {
    if (kernel && std::strlen(kernel) >= sizeof(g_only)) return LSA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_mu);
    g_filtered.store(0, std::memory_order_release);
    if (kernel) {
        std::strcpy(g_only, kernel);
        g_filtered.store(1, std::memory_order_release);
    }
    return LSA_OK;
}

void lsa_timing_reset(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    drain();
    g_done.clear();
    g_seen.clear();
}

lsa_status lsa_timing_read(const char* kernel, int64_t* launches, double* total_ms) {
    if (!kernel || !launches || !total_ms) return LSA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_mu);
    drain();
    auto it = g_done.find(kernel);
    *launches = it == g_done.end() ? 0 : it->second.first;
    *total_ms = it == g_done.end() ? 0.0 : it->second.second;
    return LSA_OK;
}

}  // extern "C"
