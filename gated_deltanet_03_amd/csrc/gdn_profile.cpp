// Opt-in per-kernel timing with HIP events.  When enabled, every kernel the
// entry points launch is bracketed by a start/stop event recorded on its launch
// stream; gdn_profile_collect() waits for them and reports per-kernel totals.
// Disabled (the default) it costs one relaxed atomic load per launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

const char* const kNames[kNumKernels] = {"chunk_plan_kernel", "chunk_prep_kernel", "chunk_state_kernel",
                                          "recurrent_step_kernel", "replay_kernel", "copy_kernel"};

struct Rec {
  int id;
  hipEvent_t a, b;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_pending;
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

thread_local int t_open_id = -1;
thread_local hipEvent_t t_open_ev = nullptr;

}  // namespace

void prof_begin(KernelId id, hipStream_t s) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t e = take_event();
  if (e == nullptr) return;
  if (hipEventRecord(e, s) != hipSuccess) {
    g_pool.push_back(e);
    return;
  }
  t_open_id = (int)id;
  t_open_ev = e;
}

void prof_end(KernelId id, hipStream_t s) {
  if (!g_on.load(std::memory_order_relaxed) || t_open_ev == nullptr || t_open_id != (int)id) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t e = take_event();
  if (e == nullptr || hipEventRecord(e, s) != hipSuccess) {
    if (e) g_pool.push_back(e);
    g_pool.push_back(t_open_ev);
  } else {
    g_pending.push_back(Rec{(int)id, t_open_ev, e});
  }
  t_open_ev = nullptr;
  t_open_id = -1;
}

}  // namespace gdn

extern "C" {

gdn_status gdn_profile_enable(int32_t on) {
  gdn::g_on.store(on != 0);
  return GDN_OK;
}

int32_t gdn_profile_collect(const char** names, double* total_ms, int32_t* launches, int32_t max_kernels) {
  using namespace gdn;
  std::vector<Rec> recs;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    recs.swap(g_pending);
  }
  double tot[kNumKernels] = {0};
  int cnt[kNumKernels] = {0};
  for (const Rec& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      tot[r.id] += ms;
      cnt[r.id] += 1;
    }
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (const Rec& r : recs) {
      g_pool.push_back(r.a);
      g_pool.push_back(r.b);
    }
  }
  int n = 0;
  for (int k = 0; k < kNumKernels; ++k) {
    if (cnt[k] == 0) continue;
    if (n < max_kernels) {
      if (names) names[n] = kNames[k];
      if (total_ms) total_ms[n] = tot[k];
      if (launches) launches[n] = cnt[k];
    }
    ++n;
  }
  return n;
}

}  // extern "C"
