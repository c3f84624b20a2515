// Optional per-kernel timing hook (mx_profile_kernel in include/mxattn.h): when a caller has
// registered HIP events for a kernel kind, the launcher records launch i between
// start[i % n] and stop[i % n] on the launch stream. Host-side only, process-wide, and meant
// for measurement; it is off unless a caller registers events.
#pragma once
#include <hip/hip_runtime.h>

namespace mx {

enum ProfileKind {
  kProfNone = 0, kProfFwd = 1, kProfBwdKV = 2, kProfQuantize = 3, kProfBwdPrep = 4, kProfBwdQ = 5, kProfRmsNorm = 6, kProfGemm = 7
};

struct ProfileHook {
  int kind = kProfNone;
  hipEvent_t* start = nullptr;
  hipEvent_t* stop = nullptr;
  int n = 0;
  long long count = 0;
};

ProfileHook& profile_hook();

inline int profile_begin(int kind, hipStream_t stream) {
  ProfileHook& h = profile_hook();
  if (h.kind != kind || h.n <= 0) return -1;
  const int slot = (int)(h.count++ % h.n);
  (void)hipEventRecord(h.start[slot], stream);
  return slot;
}

inline void profile_end(int slot, hipStream_t stream) {
  if (slot < 0) return;
  (void)hipEventRecord(profile_hook().stop[slot], stream);
}

}  // namespace mx
