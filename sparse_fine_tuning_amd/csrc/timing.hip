// Event-timing hook used by the benchmark to time one kernel class on the
// stream it is launched on.
#include <stdlib.h>

#include "timing.hpp"

namespace usaf {
KernelTimer& timer() {
  static KernelTimer t;
  return t;
}
}  // namespace usaf

using namespace usaf;

static void release_events(KernelTimer& t) {
  for (int i = 0; i < t.cap; ++i) {
    (void)hipEventDestroy(t.start[i]);
    (void)hipEventDestroy(t.stop[i]);
  }
  free(t.start);
  free(t.stop);
  t.start = t.stop = nullptr;
  t.cap = 0;
}

extern "C" usaf_status usaf_timer_arm(int32_t kernel_class, int32_t capacity) {
  KernelTimer& t = timer();
  if (kernel_class == -1) {
    t.armed = -1;
    return USAF_OK;
  }
  if (kernel_class < 0 || kernel_class >= USAF_K_COUNT || capacity < 1 || capacity > 65536)
    return USAF_ERR_INVALID_ARG;
  if (capacity > t.cap) {
    release_events(t);
    t.start = static_cast<hipEvent_t*>(calloc(size_t(capacity), sizeof(hipEvent_t)));
    t.stop = static_cast<hipEvent_t*>(calloc(size_t(capacity), sizeof(hipEvent_t)));
    if (!t.start || !t.stop) return USAF_ERR_HIP;
    for (int i = 0; i < capacity; ++i) {
      if (hipEventCreate(&t.start[i]) != hipSuccess || hipEventCreate(&t.stop[i]) != hipSuccess) {
        t.cap = i;
        release_events(t);
        return USAF_ERR_HIP;
      }
    }
    t.cap = capacity;
  }
  t.armed = kernel_class;
  t.n = 0;
  return USAF_OK;
}

extern "C" usaf_status usaf_timer_read(float* ms, int32_t capacity, int32_t* count) {
  KernelTimer& t = timer();
  if (!ms || !count || capacity < 0) return USAF_ERR_INVALID_ARG;
  const int n = t.n < capacity ? t.n : capacity;
  for (int i = 0; i < n; ++i) {
    if (hipEventSynchronize(t.stop[i]) != hipSuccess) return USAF_ERR_HIP;
    if (hipEventElapsedTime(&ms[i], t.start[i], t.stop[i]) != hipSuccess) return USAF_ERR_HIP;
  }
  *count = n;
  return USAF_OK;
}
