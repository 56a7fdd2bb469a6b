// Optional per-kernel timing: while enabled, every library launch records a
// pair of HIP events at the kernel's own start and end (hipExtLaunchKernelGGL);
// reading the profile synchronises those events and aggregates per kernel
// name. This is a diagnostic and must not be enabled inside graph capture.
#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "dsa.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

struct Rec {
  const char* name;
  hipEvent_t start, stop;
};

std::mutex g_mu;
std::atomic<bool> g_on{false};
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_free;

hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  // timing-only events: no system-scope fence (a fence would write back the
  // L2 of every XCD and inflate the measured kernel)
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

ProfSlot prof_slot(const char* name) {
  ProfSlot ps;
  if (!g_on.load(std::memory_order_relaxed)) return ps;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return ps;
  Rec r{name, take_event(), take_event()};
  if (!r.start || !r.stop) return ps;
  g_recs.push_back(r);
  ps.start = r.start;
  ps.stop = r.stop;
  return ps;
}

}  // namespace dsa

extern "C" {

dsa_status dsa_profile_begin(void) {
  std::lock_guard<std::mutex> lk(dsa::g_mu);
  for (auto& r : dsa::g_recs) {
    dsa::g_free.push_back(r.start);
    dsa::g_free.push_back(r.stop);
  }
  dsa::g_recs.clear();
  dsa::g_on = true;
  return DSA_OK;
}

dsa_status dsa_profile_end(dsa_kernel_time* out, int32_t capacity, int32_t* n_out) {
  std::lock_guard<std::mutex> lk(dsa::g_mu);
  dsa::g_on = false;
  std::vector<dsa_kernel_time> agg;
  dsa_status st = DSA_OK;
  for (auto& r : dsa::g_recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) {
      st = DSA_ERR_HIP;
      continue;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      st = DSA_ERR_HIP;
      continue;
    }
    size_t j = 0;
    for (; j < agg.size(); ++j)
      if (std::strncmp(agg[j].name, r.name, sizeof(agg[j].name)) == 0) break;
    if (j == agg.size()) {
      dsa_kernel_time t{};
      std::strncpy(t.name, r.name, sizeof(t.name) - 1);
      agg.push_back(t);
    }
    agg[j].launches += 1;
    agg[j].total_ms += ms;
  }
  for (auto& r : dsa::g_recs) {
    dsa::g_free.push_back(r.start);
    dsa::g_free.push_back(r.stop);
  }
  dsa::g_recs.clear();
  const int32_t n = static_cast<int32_t>(agg.size());
  if (n_out) *n_out = n;
  if (out) {
    for (int32_t i = 0; i < n && i < capacity; ++i) out[i] = agg[i];
  }
  return st;
}

}  // extern "C"
