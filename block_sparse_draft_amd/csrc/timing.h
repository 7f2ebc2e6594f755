// Optional per-kernel event timing of libsplitkv launches (see skv_timing_*).
#pragma once
#include <hip/hip_runtime.h>

namespace skv {

enum KernelId {
  kFillPartials, kFwdBf16, kFwdF32, kMerge, kBwdPack, kBwdKv, kBwdDq, kBwdFinalize,
  kOwnFwd, kOwnBwd, kNumKernels
};

// Brackets the launches made during its lifetime with two events on `stream`
// when timing is enabled; does nothing otherwise.
class TimedLaunch {
 public:
  TimedLaunch(KernelId k, hipStream_t stream);
  ~TimedLaunch();
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;

 private:
  KernelId k_;
  hipStream_t stream_;
  hipEvent_t start_, stop_;
};

}  // namespace skv
