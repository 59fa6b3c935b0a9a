// Opt-in kernel timing with pooled HIP events (muon_profile_begin / _end).
#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "muon_internal.h"

namespace muon {

namespace {

struct Record {
    const char* name;
    hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
    // caller holds g_mu
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

LaunchTimer::LaunchTimer(const char* name, hipStream_t s) : name_(name), stream_(s) {
    if (!g_on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lock(g_mu);
    hipEvent_t e = take_event();
    if (e == nullptr) return;
    if (hipEventRecord(e, stream_) != hipSuccess) {
        g_pool.push_back(e);
        return;
    }
    start_ = e;
}

LaunchTimer::~LaunchTimer() {
    if (start_ == nullptr) return;
    std::lock_guard<std::mutex> lock(g_mu);
    hipEvent_t stop = take_event();
    hipEvent_t start = static_cast<hipEvent_t>(start_);
    if (stop == nullptr || hipEventRecord(stop, stream_) != hipSuccess) {
        g_pool.push_back(start);
        if (stop) g_pool.push_back(stop);
        return;
    }
    g_records.push_back({name_, start, stop});
}

}  // namespace muon

extern "C" {

int muon_profile_begin(void) {
    std::lock_guard<std::mutex> lock(muon::g_mu);
    for (auto& r : muon::g_records) {
        muon::g_pool.push_back(r.start);
        muon::g_pool.push_back(r.stop);
    }
    muon::g_records.clear();
    muon::g_on.store(true);
    return MUON_OK;
}

int muon_profile_end(muon_kernel_time_t* out, int max_entries, int* n_entries) {
    muon::g_on.store(false);
    std::lock_guard<std::mutex> lock(muon::g_mu);
    std::map<std::string, std::pair<double, int64_t>> agg;
    int rc = MUON_OK;
    for (auto& r : muon::g_records) {
        float ms = 0.f;
        if (hipEventSynchronize(r.stop) != hipSuccess ||
            hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
            rc = MUON_ERR_HIP;
            continue;
        }
        auto& a = agg[r.name];
        a.first += ms;
        a.second += 1;
    }
    for (auto& r : muon::g_records) {
        muon::g_pool.push_back(r.start);
        muon::g_pool.push_back(r.stop);
    }
    muon::g_records.clear();
    int k = 0;
    for (auto& kv : agg) {
        if (out != nullptr && k < max_entries) {
            std::memset(out[k].name, 0, sizeof(out[k].name));
            std::strncpy(out[k].name, kv.first.c_str(), sizeof(out[k].name) - 1);
            out[k].total_ms = kv.second.first;
            out[k].launches = kv.second.second;
        }
        ++k;
    }
    if (n_entries != nullptr) *n_entries = k;
    return rc;
}

}  // extern "C"
