// Optional HIP-event timing of the library's own kernel launches.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "tq_internal.h"

namespace tq {
namespace {

struct Rec {
  std::string name;
  hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::string g_select;  // record only launches whose name contains this (empty: all)
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t get_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  // timing events without a system-scope release: the bracketed kernel is not slowed by cache writebacks
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

bool profiling() { return g_on.load(std::memory_order_relaxed); }

void *prof_begin(const char *name, hipStream_t st) {
  if (!profiling()) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_select.empty() && std::strstr(name, g_select.c_str()) == nullptr) return nullptr;
  hipEvent_t a = get_event(), b = get_event();
  if (!a || !b) return nullptr;
  hipEventRecord(a, st);
  g_recs.push_back(Rec{name, a, b});
  return reinterpret_cast<void *>(g_recs.size());
}

void prof_kernel_events(const char *name, hipEvent_t *start, hipEvent_t *stop) {
  *start = *stop = nullptr;
  if (!profiling()) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_select.empty() && std::strstr(name, g_select.c_str()) == nullptr) return;
  hipEvent_t a = get_event(), b = get_event();
  if (!a || !b) return;
  g_recs.push_back(Rec{name, a, b});
  *start = a;
  *stop = b;
}

void prof_end(void *tok, hipStream_t st) {
  if (!tok) return;
  std::lock_guard<std::mutex> lk(g_mu);
  size_t i = reinterpret_cast<size_t>(tok) - 1;
  if (i < g_recs.size()) hipEventRecord(g_recs[i].stop, st);
}

}  // namespace tq

extern "C" {

int tq_profile_enable(int on) {
  tq::g_on.store(on != 0);
  return TQ_OK;
}

int tq_profile_select(const char *name) {
  std::lock_guard<std::mutex> lk(tq::g_mu);
  tq::g_select = name ? name : "";
  return TQ_OK;
}

int tq_profile_query(const char *name, double *total_ms, int64_t *count) {
  std::lock_guard<std::mutex> lk(tq::g_mu);
  double tot = 0.0;
  int64_t n = 0;
  for (auto &r : tq::g_recs) {
    if (name && *name && r.name.find(name) == std::string::npos) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return tq::hip_fail(e);
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return tq::hip_fail(e);
    tot += ms;
    ++n;
  }
  if (total_ms) *total_ms = tot;
  if (count) *count = n;
  return TQ_OK;
}

int tq_profile_reset(void) {
  std::lock_guard<std::mutex> lk(tq::g_mu);
  for (auto &r : tq::g_recs) {
    hipEventSynchronize(r.stop);
    tq::g_pool.push_back(r.start);
    tq::g_pool.push_back(r.stop);
  }
  tq::g_recs.clear();
  return TQ_OK;
}

}  // extern "C"
