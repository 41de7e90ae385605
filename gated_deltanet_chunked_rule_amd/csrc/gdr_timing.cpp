// gdr_timing.cpp -- optional per-kernel timing with HIP events.
//
// When enabled, each launch is bracketed by two events recorded on the launch
// stream.  gdr_timing_collect() waits for the pending pairs and folds their
// elapsed times into per-kernel totals.  Event objects are pooled and reused.
// With timing off (the default) a launch reads one atomic flag and takes no
// lock: the registry below is touched only while timing is on.
#include <hip/hip_runtime.h>

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gdr.h"
#include "gdr_kernels.h"

namespace {

struct Pending {
  std::string name;
  hipEvent_t a, b;
};

struct Totals {
  double ms = 0.0;
  int32_t launches = 0;
};

std::mutex g_mu;
std::atomic<bool> g_enabled{false};
std::vector<hipEvent_t> g_pool;
std::vector<Pending> g_pending;
std::vector<std::pair<std::string, Totals>> g_totals;
thread_local std::string t_name;
thread_local hipEvent_t t_start = nullptr;

hipEvent_t get_event() {
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

namespace gdr {

void timing_before(const char* name, hipStream_t st) {
  t_start = nullptr;
  if (!g_enabled.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  t_start = get_event();
  t_name = name;
  if (t_start) (void)hipEventRecord(t_start, st);
}

void timing_after(hipStream_t st) {
  if (!t_start) return;   // timing was off when this launch began
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t end = get_event();
  if (!end) return;
  (void)hipEventRecord(end, st);
  g_pending.push_back({t_name, t_start, end});
  t_start = nullptr;
}

}  // namespace gdr

extern "C" {

void gdr_timing_enable(int enable) { g_enabled.store(enable != 0, std::memory_order_relaxed); }

int gdr_timing_collect(void) {
  std::vector<Pending> todo;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    todo.swap(g_pending);
  }
  std::vector<std::pair<std::string, float>> done;
  for (auto& p : todo) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess)
      done.push_back({p.name, ms});
  }
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& d : done) {
    bool found = false;
    for (auto& t : g_totals)
      if (t.first == d.first) {
        t.second.ms += d.second;
        t.second.launches += 1;
        found = true;
        break;
      }
    if (!found) g_totals.push_back({d.first, Totals{d.second, 1}});
  }
  for (auto& p : todo) {
    g_pool.push_back(p.a);
    g_pool.push_back(p.b);
  }
  return (int)g_totals.size();
}

int gdr_timing_entry(int i, const char** name, double* total_ms, int32_t* launches) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (i < 0 || i >= (int)g_totals.size()) return -1;
  if (name) *name = g_totals[i].first.c_str();
  if (total_ms) *total_ms = g_totals[i].second.ms;
  if (launches) *launches = g_totals[i].second.launches;
  return 0;
}

void gdr_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_totals.clear();
}

}  // extern "C"
