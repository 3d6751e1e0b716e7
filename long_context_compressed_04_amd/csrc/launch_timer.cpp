// Per-launch timing: a HIP event pair per kernel dispatch (stamped by the runtime with
// the dispatch's start and end), aggregated per kernel name on collection.  Events
// are pooled and reused; nothing is recorded while timing is off or while the launch
// stream is being captured into a graph.
#include "launch_timer.hpp"

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/csa.h"

namespace csa {
namespace {

struct Record {
  hipEvent_t start = nullptr, stop = nullptr;
  const char* kernel = nullptr;
  bool done = false;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Record> g_recs;
std::vector<hipEvent_t> g_pool;

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

}  // namespace

bool timing_enabled() { return g_on.load(std::memory_order_relaxed); }

int timing_begin(hipStream_t s, hipEvent_t* start, hipEvent_t* stop) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return -1;
  std::lock_guard<std::mutex> lk(g_mu);
  Record r;
  r.start = take_event();
  r.stop = take_event();
  if (!r.start || !r.stop) {
    if (r.start) g_pool.push_back(r.start);
    if (r.stop) g_pool.push_back(r.stop);
    return -1;
  }
  *start = r.start;
  *stop = r.stop;
  g_recs.push_back(r);
  return (int)g_recs.size() - 1;
}

void timing_end(int slot, const char* kernel, bool launched) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (slot < 0 || slot >= (int)g_recs.size()) return;
  Record& r = g_recs[slot];
  r.kernel = kernel;
  r.done = launched;
}

}  // namespace csa

extern "C" {

csa_status csa_timing_enable(int32_t on) {
  csa::g_on.store(on != 0);
  return CSA_OK;
}

int32_t csa_timing_collect(csa_kernel_time* out, int32_t cap) {
  using namespace csa;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!out) {   // count the distinct kernels launched so far; records are kept
    std::vector<std::string> names;
    for (const Record& r : g_recs) {
      if (!r.done || !r.kernel) continue;
      bool seen = false;
      for (const std::string& n : names) seen = seen || n == r.kernel;
      if (!seen) names.push_back(r.kernel);
    }
    return (int32_t)names.size();
  }
  struct Agg { int32_t n = 0; double total = 0, mn = 1e30, mx = 0; };
  std::map<std::string, Agg> agg;
  std::vector<std::string> order;
  for (Record& r : g_recs) {
    if (r.done && r.kernel && hipEventSynchronize(r.stop) == hipSuccess) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
        auto it = agg.find(r.kernel);
        if (it == agg.end()) {
          order.push_back(r.kernel);
          it = agg.emplace(r.kernel, Agg{}).first;
        }
        Agg& a = it->second;
        const double us = ms * 1e3;
        a.n += 1;
        a.total += us;
        a.mn = us < a.mn ? us : a.mn;
        a.mx = us > a.mx ? us : a.mx;
      }
    }
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_recs.clear();
  int32_t n = 0;
  for (const std::string& name : order) {
    if (n >= cap) break;
    const Agg& a = agg[name];
    csa_kernel_time& t = out[n++];
    size_t i = 0;
    for (; i + 1 < sizeof(t.name) && i < name.size(); ++i) t.name[i] = name[i];
    t.name[i] = '\0';
    t.launches = a.n;
    t.total_us = a.total;
    t.min_us = a.mn;
    t.max_us = a.mx;
  }
  return n;
}

}  // extern "C"
