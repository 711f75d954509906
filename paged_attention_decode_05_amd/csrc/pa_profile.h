// pa_profile.h -- the measurement hook behind pa_profile_next(): events armed
// by the caller time the next call's dominant kernel, then are disarmed.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <utility>

namespace pa {

struct ProfileHook {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
extern thread_local ProfileHook g_profile;

// Launches kernel k on stream s.  With the hook armed, the launch goes through
// hipExtLaunchKernelGGL with the hook's events, which the command processor
// stamps as the kernel's own dispatch starts and ends (the clock a kernel
// trace reports; a pair of stream events around an ordinary launch would
// also count the dispatch of the kernel), and the hook is disarmed.
template <typename... KArgs, typename... Args>
inline void launch_profiled(void (*k)(KArgs...), dim3 grid, dim3 block, unsigned shmem,
                            hipStream_t s, Args&&... args) {
  if (g_profile.start && g_profile.stop) {
    const ProfileHook h = g_profile;
    g_profile = ProfileHook{};
    hipExtLaunchKernelGGL(k, grid, block, shmem, s, h.start, h.stop, 0u, std::forward<Args>(args)...);
  } else {
    hipLaunchKernelGGL(k, grid, block, shmem, s, std::forward<Args>(args)...);
  }
}

}  // namespace pa
