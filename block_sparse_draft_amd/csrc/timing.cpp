// Per-kernel event timing of libsplitkv launches.  Events come from a pool
// that grows on demand; pending (start, stop) pairs are resolved and returned
// to the pool by skv_timing_collect.
#include "timing.h"

#include <atomic>
#include <mutex>
#include <vector>

#include "internal.h"

namespace skv {
namespace {

const char* const kNames[kNumKernels] = {"fill_partials", "partial_fwd_bf16", "partial_fwd_f32", "lse_merge",
                                         "bwd_pack", "bwd_kv", "bwd_dq", "bwd_finalize",
                                         "own_fwd", "own_bwd"};

struct Pending {
  KernelId k;
  hipEvent_t start, stop;
};

std::atomic<bool> g_enabled{false};
std::mutex g_mu;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_pool.empty()) {
      hipEvent_t e = g_pool.back();
      g_pool.pop_back();
      return e;
    }
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void give_event(hipEvent_t e) {
  if (!e) return;
  std::lock_guard<std::mutex> lk(g_mu);
  g_pool.push_back(e);
}

}  // namespace

TimedLaunch::TimedLaunch(KernelId k, hipStream_t stream) : k_(k), stream_(stream), start_(nullptr), stop_(nullptr) {
  if (!g_enabled.load(std::memory_order_relaxed)) return;
  start_ = take_event();
  stop_ = take_event();
  if (!start_ || !stop_ || hipEventRecord(start_, stream_) != hipSuccess) {
    give_event(start_);
    give_event(stop_);
    start_ = stop_ = nullptr;
  }
}

TimedLaunch::~TimedLaunch() {
  if (!start_) return;
  if (hipEventRecord(stop_, stream_) != hipSuccess) {
    give_event(start_);
    give_event(stop_);
    return;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  g_pending.push_back({k_, start_, stop_});
}

}  // namespace skv

using namespace skv;

extern "C" int skv_timing_enable(int32_t on) {
  g_enabled.store(on != 0);
  clear_error();
  return SKV_OK;
}

extern "C" int skv_timing_collect(skv_kernel_time* out, int32_t max_entries, int32_t* n_entries) {
  if (max_entries < 0 || (max_entries > 0 && !out)) return fail(SKV_EINVAL, "bad output array");
  std::vector<Pending> pend;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    pend.swap(g_pending);
  }
  int64_t launches[kNumKernels] = {};
  double ms[kNumKernels] = {};
  int rc = SKV_OK;
  for (const Pending& p : pend) {
    float t = 0.f;
    if (rc == SKV_OK) {
      hipError_t e = hipEventSynchronize(p.stop);
      if (e == hipSuccess) e = hipEventElapsedTime(&t, p.start, p.stop);
      if (e != hipSuccess) rc = fail(SKV_EHIP, "skv_timing_collect: %s", hipGetErrorString(e));
    }
    launches[p.k] += 1;
    ms[p.k] += t;
    give_event(p.start);
    give_event(p.stop);
  }
  if (rc != SKV_OK) return rc;
  int n = 0;
  for (int k = 0; k < kNumKernels; ++k) {
    if (!launches[k]) continue;
    if (n < max_entries) out[n] = skv_kernel_time{kNames[k], launches[k], ms[k]};
    ++n;
  }
  if (n_entries) *n_entries = n;
  clear_error();
  return SKV_OK;
}
