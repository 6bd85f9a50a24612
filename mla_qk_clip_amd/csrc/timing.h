// Optional per-kernel timing: when enabled, every launch is bracketed by a
// pair of HIP events recorded on the caller's stream. Off by default; the
// cost when off is one relaxed atomic load per launch.
#pragma once

#include <hip/hip_runtime.h>

namespace mla {

bool timing_enabled();
// Records the start event; returns the stop event to record after the
// launch (nullptr when timing is off).
hipEvent_t timing_begin(const char* kernel, hipStream_t st);

struct TimedScope {
  hipEvent_t stop;
  hipStream_t st;
  TimedScope(const char* kernel, hipStream_t s) : stop(timing_begin(kernel, s)), st(s) {}
  ~TimedScope() {
    if (stop) (void)hipEventRecord(stop, st);
  }
};

}  // namespace mla
