// The regression loss of a layer output without a caller workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops, harnesses that forbid allocation).  The partial sums that
// usaf_mse_grad keeps in the caller's workspace live here in a fixed
// file-scope device array instead.
#include <mutex>

#include "common.hpp"
#include "moe_internal.hpp"

namespace usaf {

// Partial sums of the loss, one per 4096 elements of Y.
constexpr int64_t kNoAllocParts = 65536;
constexpr int64_t kNoAllocMaxElems = kNoAllocParts * 4096;  // T*H at most 2^28

// Every device the library runs on holds its own copy until the process ends.
static __device__ __align__(256) float scratch[kNoAllocParts];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device.  In host code the array's name is only a stand-in for the symbol,
// never an address a kernel may use.
usaf_status scratch_of_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return USAF_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return USAF_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return USAF_ERR_HIP;
    g_scratch[dev] = static_cast<float*>(p);
  }
  *out = g_scratch[dev];
  return USAF_OK;
}
}  // namespace

}  // namespace usaf

using namespace usaf;

extern "C" USAF_API usaf_status usaf_mse_grad_noalloc(const usaf_moe_shape* shape, const void* Y,
                                                      const void* tgt, void* dY, float* loss,
                                                      int32_t* nonfinite, hipStream_t stream) {
  USAF_TRY(check_shape(shape));
  if (!Y || !tgt || !dY || !loss) return USAF_ERR_INVALID_ARG;
  if (int64_t(shape->T) * shape->H > kNoAllocMaxElems) return USAF_ERR_UNSUPPORTED;
  float* part = nullptr;
  USAF_TRY(scratch_of_current_device(&part));
  // every partial is written by its block before the final kernel reads it,
  // so nothing needs clearing between calls
  return mse_launch(*shape, Y, tgt, dY, loss, nonfinite, part, stream);
}
