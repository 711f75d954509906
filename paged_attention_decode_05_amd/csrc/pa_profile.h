// pa_profile.h -- the measurement hook behind pa_profile_next(): events armed
// by the caller are recorded on the launch stream around the next call's
// dominant kernel, then disarmed.
#pragma once

#include <hip/hip_runtime.h>

namespace pa {

struct ProfileHook {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
extern thread_local ProfileHook g_profile;

inline void profile_begin(hipStream_t s) {
  if (g_profile.start) (void)hipEventRecord(g_profile.start, s);
}
inline void profile_end(hipStream_t s) {
  if (g_profile.stop) (void)hipEventRecord(g_profile.stop, s);
  g_profile = ProfileHook{};
}

}  // namespace pa
