// Optional per-launch timing (diagnostics).  When switched on through the C ABI,
// every kernel the library launches on a stream that is not being captured into a
// graph is bracketed by a HIP event pair recorded on that same stream.
#pragma once
#include <hip/hip_runtime.h>

namespace csa {

bool timing_enabled();
// Returns a slot handle (or -1 when timing is off / the stream is capturing).
int timing_begin(hipStream_t s);
void timing_end(int slot, const char* kernel, hipStream_t s);

// Scope guard: begin on construction, end on destruction.
struct LaunchTimer {
  LaunchTimer(const char* kernel, hipStream_t s) : kernel_(kernel), s_(s), slot_(timing_enabled() ? timing_begin(s) : -1) {}
  ~LaunchTimer() {
    if (slot_ >= 0) timing_end(slot_, kernel_, s_);
  }
  LaunchTimer(const LaunchTimer&) = delete;
  LaunchTimer& operator=(const LaunchTimer&) = delete;

 private:
  const char* kernel_;
  hipStream_t s_;
  int slot_;
};

}  // namespace csa
