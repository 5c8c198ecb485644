// Per-kernel device timing behind ls_profile_begin / ls_profile_end: each launch made while
// profiling is on is bracketed by two HIP events on its own stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/longstraw.h"
#include "launch.hpp"

namespace {

struct Record {
    const char* name;
    hipEvent_t start;
    hipEvent_t end;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
    hipEvent_t e = nullptr;
    if (!g_pool.empty()) {
        e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

namespace ls {

KernelTimer::KernelTimer(const char* name, hipStream_t s) : name_(name), stream_(s) {
    if (!g_on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lk(g_mu);
    start_ = take_event();
    if (start_ && hipEventRecord(start_, stream_) != hipSuccess) {
        g_pool.push_back(start_);
        start_ = nullptr;
    }
}

KernelTimer::~KernelTimer() {
    if (!start_) return;
    std::lock_guard<std::mutex> lk(g_mu);
    hipEvent_t end = take_event();
    if (!end || hipEventRecord(end, stream_) != hipSuccess) {
        g_pool.push_back(start_);
        if (end) g_pool.push_back(end);
        return;
    }
    g_records.push_back({name_, start_, end});
}

}  // namespace ls

extern "C" {

int ls_profile_begin(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    for (auto& r : g_records) {
        g_pool.push_back(r.start);
        g_pool.push_back(r.end);
    }
    g_records.clear();
    g_on.store(true);
    return LS_OK;
}

int ls_profile_end(ls_kernel_stat_t* out, int max_entries, int* n_entries) {
    if (!n_entries || (max_entries > 0 && !out)) return LS_ERR_INVALID;
    std::vector<Record> recs;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (!g_on.load()) return LS_ERR_INVALID;
        g_on.store(false);
        recs.swap(g_records);
    }
    std::map<std::string, std::pair<int64_t, double>> agg;
    int rc = LS_OK;
    for (auto& r : recs) {
        float ms = 0.f;
        if (hipEventSynchronize(r.end) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.end) != hipSuccess)
            rc = LS_ERR_HIP;
        auto& a = agg[r.name];
        a.first += 1;
        a.second += ms;
    }
    {
        std::lock_guard<std::mutex> lk(g_mu);
        for (auto& r : recs) {
            g_pool.push_back(r.start);
            g_pool.push_back(r.end);
        }
    }
    int i = 0;
    for (auto& kv : agg) {
        if (i < max_entries) {
            std::memset(out[i].name, 0, sizeof out[i].name);
            std::strncpy(out[i].name, kv.first.c_str(), sizeof out[i].name - 1);
            out[i].launches = kv.second.first;
            out[i].total_ms = kv.second.second;
        }
        i++;
    }
    *n_entries = i;
    return rc;
}

}  // extern "C"
