// Per-kernel timing with HIP events (diagnostics).  When enabled, every
// kernel launch of the library is bracketed by two events recorded on the
// launch stream; ia_profile_report waits for them and sums the elapsed time
// per kernel name.  Disabled (the default), a launch pays one branch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "ia_internal.h"

namespace ia {
namespace {

struct Record {
    const char* name;
    hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Record> g_pending;
std::map<std::string, std::pair<long, double>> g_done;  // name -> (calls, total ms)

void drain_locked() {
    for (Record& r : g_pending) {
        float ms = 0.0f;
        if (hipEventSynchronize(r.stop) == hipSuccess && hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
            auto& d = g_done[r.name];
            d.first += 1;
            d.second += ms;
        }
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    g_pending.clear();
}

}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t s) : name_(name), s_(s) {
    if (!g_on.load(std::memory_order_relaxed)) return;
    if (hipEventCreate(&start_) != hipSuccess) return;
    if (hipEventCreate(&stop_) != hipSuccess) {
        (void)hipEventDestroy(start_);
        return;
    }
    (void)hipEventRecord(start_, s_);
    active_ = true;
}

ProfScope::~ProfScope() {
    if (!active_) return;
    (void)hipEventRecord(stop_, s_);
    std::lock_guard<std::mutex> lk(g_mu);
    g_pending.push_back({name_, start_, stop_});
}

}  // namespace ia

extern "C" {

ia_status ia_profile_enable(int32_t on) {
    ia::g_on.store(on != 0);
    return IA_OK;
}

void ia_profile_reset(void) {
    std::lock_guard<std::mutex> lk(ia::g_mu);
    ia::drain_locked();
    ia::g_done.clear();
}

ia_status ia_profile_report(char* buf, size_t len, size_t* needed) {
    std::lock_guard<std::mutex> lk(ia::g_mu);
    ia::drain_locked();
    std::string s = "{";
    bool first = true;
    for (auto& kv : ia::g_done) {
        char item[256];
        std::snprintf(item, sizeof(item), "%s\"%s\": [%ld, %.6f]", first ? "" : ", ", kv.first.c_str(),
                      kv.second.first, kv.second.second);
        s += item;
        first = false;
    }
    s += "}";
    if (needed) *needed = s.size() + 1;
    if (!buf || len < s.size() + 1) return IA_ERR_INVALID_ARG;
    std::snprintf(buf, len, "%s", s.c_str());
    return IA_OK;
}

}  // extern "C"
