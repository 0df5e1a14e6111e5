// Event-timing hook (usaf_timer_arm / usaf_timer_read in usaf.h).
#pragma once

#include <hip/hip_runtime.h>

#include "usaf.h"

namespace usaf {

struct KernelTimer {
  int armed = -1;
  int cap = 0;
  int n = 0;
  hipEvent_t* start = nullptr;
  hipEvent_t* stop = nullptr;
};
KernelTimer& timer();

inline void timer_begin(int kclass, hipStream_t s) {
  KernelTimer& t = timer();
  if (kclass >= 0 && t.armed == kclass && t.n < t.cap) (void)hipEventRecord(t.start[t.n], s);
}
inline void timer_end(int kclass, hipStream_t s) {
  KernelTimer& t = timer();
  if (kclass >= 0 && t.armed == kclass && t.n < t.cap) {
    (void)hipEventRecord(t.stop[t.n], s);
    ++t.n;
  }
}

}  // namespace usaf
