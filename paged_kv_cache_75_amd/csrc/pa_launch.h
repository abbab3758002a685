// Kernel launch with the measurement hook (pa_profile_start / pa_profile_stop):
// while timing is on, a launch gets a start and a stop event attached to its
// own dispatch, so the pair brackets that kernel alone.  Shared by the HIP
// sources; the timer itself lives in pa_kernels.hip.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <utility>
#include <vector>

namespace pa {

struct KernelTimer {
  std::atomic<bool> on{false};
  std::mutex mu;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> events;
};
KernelTimer& kernel_timer();

template <typename Kernel, typename... Args>
void launch_timed(Kernel kernel, dim3 grid, dim3 block, hipStream_t stream, Args... args) {
  KernelTimer& t = kernel_timer();
  if (t.on.load(std::memory_order_relaxed)) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
      {
        std::lock_guard<std::mutex> lock(t.mu);
        t.events.emplace_back(e0, e1);
      }
      hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, e0, e1, 0, args...);
      return;
    }
    if (e0) (void)hipEventDestroy(e0);
  }
  hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
}

}  // namespace pa
