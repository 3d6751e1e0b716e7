// Kernel launches, with optional per-launch timing (diagnostics).  When timing is
// switched on through the C ABI, every kernel the library launches on a stream that
// is not being captured into a graph is launched with hipExtLaunchKernel and a pair
// of HIP events that the runtime stamps with that dispatch's own start and end (the
// kernel's execution, not the launch call around it).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <utility>

namespace csa {

bool timing_enabled();
// Returns a slot handle and its two events (or -1 when the stream is capturing or no
// event is available).
int timing_begin(hipStream_t s, hipEvent_t* start, hipEvent_t* stop);
void timing_end(int slot, const char* kernel, bool launched);

// Launches kernel<<<grid, block, lds, s>>>(args...) and returns hipGetLastError();
// timed under `name` when timing is on.
template <typename... KArgs, typename... Args>
hipError_t launch(const char* name, void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                  Args&&... args) {
  if (timing_enabled()) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    const int slot = timing_begin(s, &e0, &e1);
    if (slot >= 0) {
      hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)lds, s, e0, e1, 0u,
                            static_cast<KArgs>(std::forward<Args>(args))...);
      const hipError_t e = hipGetLastError();
      timing_end(slot, name, e == hipSuccess);
      return e;
    }
  }
  kernel<<<grid, block, lds, s>>>(static_cast<KArgs>(std::forward<Args>(args))...);
  return hipGetLastError();
}

}  // namespace csa
