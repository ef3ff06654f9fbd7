// Optional per-kernel timing with hipEvents (diagnostics for the benchmark).
#pragma once
#include <hip/hip_runtime.h>

namespace fl {

// Brackets the launches made during its lifetime with two events on `st`
// when timing is enabled (flashloop_timing_enable); otherwise does nothing.
class TimedLaunch {
 public:
  TimedLaunch(hipStream_t st, const char* name);
  ~TimedLaunch();
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;

 private:
  hipStream_t st_;
  const char* name_;
  hipEvent_t start_ = nullptr;
};

}  // namespace fl
