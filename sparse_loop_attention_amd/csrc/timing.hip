// Per-kernel hipEvent timing registry (see flashloop_timing_enable).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "flashloop.h"
#include "fl_timing.hpp"

namespace {

struct Pending {
  const char* name;
  hipEvent_t start, stop;
};
struct Total {
  double ms = 0.0;
  int64_t launches = 0;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;
std::map<std::string, Total> g_totals;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void drain_locked() {
  for (const Pending& p : g_pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(p.stop) == hipSuccess && hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
      Total& t = g_totals[p.name];
      t.ms += ms;
      t.launches += 1;
    }
    g_pool.push_back(p.start);
    g_pool.push_back(p.stop);
  }
  g_pending.clear();
}

}  // namespace

namespace fl {

TimedLaunch::TimedLaunch(hipStream_t st, const char* name) : st_(st), name_(name) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  start_ = take_event();
  if (start_ && hipEventRecord(start_, st_) != hipSuccess) {
    g_pool.push_back(start_);
    start_ = nullptr;
  }
}

TimedLaunch::~TimedLaunch() {
  if (!start_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t stop = take_event();
  if (!stop || hipEventRecord(stop, st_) != hipSuccess) {
    g_pool.push_back(start_);
    if (stop) g_pool.push_back(stop);
    return;
  }
  g_pending.push_back({name_, start_, stop});
}

}  // namespace fl

extern "C" {

fl_status flashloop_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_mu);
  drain_locked();
  if (on) g_totals.clear();
  g_on.store(on != 0);
  return FL_OK;
}

int32_t flashloop_timing_read(char* names_out, double* ms_out, int64_t* launches_out, int32_t max_entries) {
  std::lock_guard<std::mutex> lk(g_mu);
  drain_locked();
  int32_t i = 0;
  for (const auto& kv : g_totals) {
    if (i < max_entries) {
      if (names_out) {
        std::memset(names_out + 64 * i, 0, 64);
        std::strncpy(names_out + 64 * i, kv.first.c_str(), 63);
      }
      if (ms_out) ms_out[i] = kv.second.ms;
      if (launches_out) launches_out[i] = kv.second.launches;
    }
    ++i;
  }
  return i;
}

}  // extern "C"
