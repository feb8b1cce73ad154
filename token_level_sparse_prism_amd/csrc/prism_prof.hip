// prism_prof.hip -- per-kernel HIP-event timing behind prism_profile_* (diagnostics only).
#include <atomic>
#include <mutex>
#include <string.h>
#include <vector>

#include "../../include/prism.h"
#include "prism_prof.hpp"

namespace prism {
namespace {

struct ProfRec {
    const char* name;
    hipEvent_t b;
    hipEvent_t e;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_free;

hipEvent_t take_event() {
    if (!g_free.empty()) {
        hipEvent_t ev = g_free.back();
        g_free.pop_back();
        return ev;
    }
    hipEvent_t ev = nullptr;
    if (hipEventCreate(&ev) != hipSuccess) return nullptr;
    return ev;
}

}  // namespace

bool prof_enabled() { return g_on.load(std::memory_order_relaxed); }

bool prof_pair(const char* name, hipEvent_t* begin, hipEvent_t* end) {
    std::lock_guard<std::mutex> lk(g_mu);
    hipEvent_t b = take_event();
    if (!b) return false;
    hipEvent_t e = take_event();
    if (!e) {
        g_free.push_back(b);
        return false;
    }
    g_recs.push_back({name, b, e});
    *begin = b;
    *end = e;
    return true;
}

}  // namespace prism

extern "C" {

prism_status prism_profile_enable(int on) {
    prism::g_on.store(on != 0);
    return PRISM_OK;
}

prism_status prism_profile_query(const char* name, int* launches, double* total_ms) {
    if (!name || !launches || !total_ms) return PRISM_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(prism::g_mu);
    int n = 0;
    double tot = 0.0;
    for (const auto& r : prism::g_recs) {
        if (!r.e || strcmp(r.name, name) != 0) continue;
        if (hipEventSynchronize(r.e) != hipSuccess) return PRISM_ERR_HIP;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, r.b, r.e) != hipSuccess) return PRISM_ERR_HIP;
        tot += ms;
        ++n;
    }
    *launches = n;
    *total_ms = tot;
    return PRISM_OK;
}

void prism_profile_reset(void) {
    std::lock_guard<std::mutex> lk(prism::g_mu);
    for (auto& r : prism::g_recs) {
        if (r.b) {
            hipEventSynchronize(r.b);
            prism::g_free.push_back(r.b);
        }
        if (r.e) {
            hipEventSynchronize(r.e);
            prism::g_free.push_back(r.e);
        }
    }
    prism::g_recs.clear();
}

}  // extern "C"
