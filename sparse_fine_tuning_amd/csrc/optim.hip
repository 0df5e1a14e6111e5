// SparseAdam, resident int4 dequantisation, and the library's small helpers.
//
// Method: the usaf README ("tsuyu122/usaf"): SparseAdam over the trainable
// entries (A100 per-operation table); 4-bit experts dequantised once into a
// resident working copy ("how it works": caching bullet; quantisation recipe).
#include <math.h>

#include "common.hpp"
#include "moe_internal.hpp"
#include "timing.hpp"

namespace usaf {

// Adam (Kingma & Ba 2015, Algorithm 1) on a list of entries; W updated in
// place at idx[i] (or at i when idx is null).  A non-zero *skip makes the
// whole launch a no-op (NaN step skipped).
template <class W>
__global__ __launch_bounds__(256) void adam_kernel(W* __restrict__ w, const uint32_t* __restrict__ idx,
                                                   int64_t n, const float* __restrict__ g,
                                                   float* __restrict__ m, float* __restrict__ v,
                                                   float lr, float b1, float b2, float omb1,
                                                   float omb2, float bc1, float bc2, float eps,
                                                   const int32_t* __restrict__ skip) {
  if (skip && *skip != 0) return;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float gi = g[i];
    const float mi = fmaf(b1, m[i], omb1 * gi);
    const float vi = fmaf(b2, v[i], omb2 * gi * gi);
    m[i] = mi;
    v[i] = vi;
    const float mhat = mi / bc1;
    const float vhat = vi / bc2;
    const int64_t f = idx ? int64_t(idx[i]) : i;
    const float wv = Act<W>::ld(w, f) - lr * mhat / (sqrtf(vhat) + eps);
    Act<W>::st(w, f, wv);
  }
}

// Adam over a list with a compact weight copy: one entry per lane, so the
// lanes of a wave hold 64 consecutive entries of the ascending list and each
// of its scattered W stores covers the shortest span of W (list loads and
// stores are coalesced 4- and 2-byte accesses).  The weight is read from the
// list and written to the list and to W at idx.
template <class W>
__global__ __launch_bounds__(256) void adam_list_kernel(W* __restrict__ w, const uint32_t* __restrict__ idx,
                                                        int64_t n, W* __restrict__ wl,
                                                        const float* __restrict__ g,
                                                        float* __restrict__ m, float* __restrict__ v,
                                                        float lr, float b1, float b2, float omb1,
                                                        float omb2, float bc1, float bc2, float eps,
                                                        const int32_t* __restrict__ skip) {
  if (skip && *skip != 0) return;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float gi = g[i];
    const uint32_t f = idx[i];
    const float mi = fmaf(b1, m[i], omb1 * gi);
    const float vi = fmaf(b2, v[i], omb2 * gi * gi);
    const float wv = Act<W>::ld(wl, i) - lr * (mi / bc1) / (sqrtf(vi / bc2) + eps);
    m[i] = mi;
    v[i] = vi;
    Act<W>::st(wl, i, wv);
    Act<W>::st(w, int64_t(f), wv);
  }
}

template <class W>
__global__ __launch_bounds__(256) void gather_kernel(const W* __restrict__ w, const uint32_t* __restrict__ idx,
                                                     int64_t n, W* __restrict__ out) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = w[idx[i]];
}

// W[idx[i]] = vals[i]: one entry per lane, the lanes of a wave writing
// consecutive list entries.
template <class W>
__global__ __launch_bounds__(256) void scatter_kernel(W* __restrict__ w, const uint32_t* __restrict__ idx,
                                                      int64_t n, const W* __restrict__ vals) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    w[idx[i]] = vals[i];
}

// int4 -> bf16: one thread per 8 outputs (one 32-bit word of codes).
__global__ __launch_bounds__(256) void dequant_int4_kernel(const uint32_t* __restrict__ q,
                                                           const uint16_t* __restrict__ scale,
                                                           int64_t rows, int64_t cols,
                                                           uint4* __restrict__ out) {
  const int64_t wpr = cols / 8, gpr = cols / 64;
  const int64_t total = rows * wpr;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t row = i / wpr, wc = i - row * wpr;
    const uint32_t word = q[i];
    const float s = float(__builtin_bit_cast(_Float16, scale[row * gpr + (wc >> 3)]));
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n0 = int((word >> (8 * j)) & 0xfu), n1 = int((word >> (8 * j + 4)) & 0xfu);
      const float v0 = float(n0 - ((n0 & 8) << 1)) * s;
      const float v1 = float(n1 - ((n1 & 8) << 1)) * s;
      o[j] = f2bf2(v0, v1);
    }
    out[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

static unsigned grid_for(int64_t n, int64_t per_block = 256, int64_t cap = 256 * 1024) {
  int64_t b = ceil_div(n > 0 ? n : 1, per_block);
  return unsigned(b < cap ? b : cap);
}

}  // namespace usaf

using namespace usaf;

extern "C" usaf_status usaf_sparse_adam(int32_t w_dtype, void* W, const uint32_t* idx, int64_t n,
                                        void* w_list, const float* g, float* m, float* v,
                                        int64_t step, double lr, double beta1, double beta2,
                                        double eps, const int32_t* skip_if_nonzero,
                                        hipStream_t stream) {
  if (n < 0 || step < 1) return USAF_ERR_INVALID_ARG;
  if (w_dtype != USAF_F32 && w_dtype != USAF_BF16) return USAF_ERR_INVALID_ARG;
  if (w_list && !idx) return USAF_ERR_INVALID_ARG;
  if (n == 0) return USAF_OK;
  if (!W || !g || !m || !v) return USAF_ERR_INVALID_ARG;
  const double bc1 = 1.0 - pow(beta1, double(step));
  const double bc2 = 1.0 - pow(beta2, double(step));
  const float omb1 = float(1.0 - beta1), omb2 = float(1.0 - beta2);
  timer_begin(USAF_K_ADAM, stream);
  if (w_list) {
    const unsigned grid = grid_for(n);
    if (w_dtype == USAF_BF16)
      hipLaunchKernelGGL(adam_list_kernel<bf16_t>, dim3(grid), dim3(256), 0, stream,
                         static_cast<bf16_t*>(W), idx, n, static_cast<bf16_t*>(w_list), g, m, v,
                         float(lr), float(beta1), float(beta2), omb1, omb2, float(bc1),
                         float(bc2), float(eps), skip_if_nonzero);
    else
      hipLaunchKernelGGL(adam_list_kernel<float>, dim3(grid), dim3(256), 0, stream,
                         static_cast<float*>(W), idx, n, static_cast<float*>(w_list), g, m, v,
                         float(lr), float(beta1), float(beta2), omb1, omb2, float(bc1),
                         float(bc2), float(eps), skip_if_nonzero);
  } else if (w_dtype == USAF_BF16)
    hipLaunchKernelGGL(adam_kernel<bf16_t>, dim3(grid_for(n)), dim3(256), 0, stream,
                       static_cast<bf16_t*>(W), idx, n, g, m, v, float(lr), float(beta1),
                       float(beta2), omb1, omb2, float(bc1), float(bc2), float(eps),
                       skip_if_nonzero);
  else
    hipLaunchKernelGGL(adam_kernel<float>, dim3(grid_for(n)), dim3(256), 0, stream,
                       static_cast<float*>(W), idx, n, g, m, v, float(lr), float(beta1),
                       float(beta2), omb1, omb2, float(bc1), float(bc2), float(eps),
                       skip_if_nonzero);
  timer_end(USAF_K_ADAM, stream);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

extern "C" usaf_status usaf_gather(int32_t w_dtype, const void* W, const uint32_t* idx, int64_t n,
                                   void* out, hipStream_t stream) {
  if (n < 0 || (w_dtype != USAF_F32 && w_dtype != USAF_BF16)) return USAF_ERR_INVALID_ARG;
  if (n == 0) return USAF_OK;
  if (!W || !idx || !out) return USAF_ERR_INVALID_ARG;
  if (w_dtype == USAF_BF16)
    hipLaunchKernelGGL(gather_kernel<bf16_t>, dim3(grid_for(n)), dim3(256), 0, stream,
                       static_cast<const bf16_t*>(W), idx, n, static_cast<bf16_t*>(out));
  else
    hipLaunchKernelGGL(gather_kernel<float>, dim3(grid_for(n)), dim3(256), 0, stream,
                       static_cast<const float*>(W), idx, n, static_cast<float*>(out));
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

extern "C" usaf_status usaf_scatter(int32_t w_dtype, void* W, const uint32_t* idx, int64_t n,
                                    const void* vals, hipStream_t stream) {
  if (n < 0 || (w_dtype != USAF_F32 && w_dtype != USAF_BF16)) return USAF_ERR_INVALID_ARG;
  if (n == 0) return USAF_OK;
  if (!W || !idx || !vals) return USAF_ERR_INVALID_ARG;
  if (w_dtype == USAF_BF16)
    hipLaunchKernelGGL(scatter_kernel<bf16_t>, dim3(grid_for(n)), dim3(256), 0, stream,
                       static_cast<bf16_t*>(W), idx, n, static_cast<const bf16_t*>(vals));
  else
    hipLaunchKernelGGL(scatter_kernel<float>, dim3(grid_for(n)), dim3(256), 0, stream,
                       static_cast<float*>(W), idx, n, static_cast<const float*>(vals));
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

// Affine int4 -> bf16 (the HQQ-style storage): w = bf16((q - z) * s) with
// q - z and the product each rounded once in fp32; q an unsigned nibble.
// One thread per 8 outputs (one 32-bit word of codes); group % 8 == 0.
__global__ __launch_bounds__(256) void dequant_affine_kernel(const uint32_t* __restrict__ q,
                                                             const uint16_t* __restrict__ scale,
                                                             const uint16_t* __restrict__ zero,
                                                             int64_t rows, int64_t cols, int group,
                                                             uint4* __restrict__ out) {
  const int64_t wpr = cols / 8, gpr = cols / group;
  const int wpg = group / 8;
  const int64_t total = rows * wpr;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t row = i / wpr, wc = i - row * wpr;
    const int64_t gi = row * gpr + wc / wpg;
    const uint32_t word = q[i];
    const float s = float(__builtin_bit_cast(_Float16, scale[gi]));
    const float z = float(__builtin_bit_cast(_Float16, zero[gi]));
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float d0 = float((word >> (8 * j)) & 0xfu) - z;
      const float d1 = float((word >> (8 * j + 4)) & 0xfu) - z;
      o[j] = f2bf2(d0 * s, d1 * s);
    }
    out[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

extern "C" usaf_status usaf_dequant_affine(const uint8_t* q, const uint16_t* scale_f16,
                                           const uint16_t* zero_f16, int64_t rows, int64_t cols,
                                           int32_t group, void* out_bf16, hipStream_t stream) {
  if (rows < 0 || cols < 0) return USAF_ERR_INVALID_ARG;
  if ((group != 64 && group != 128) || cols % group != 0) return USAF_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return USAF_OK;
  if (!q || !scale_f16 || !zero_f16 || !out_bf16) return USAF_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q) & 3) || (reinterpret_cast<uintptr_t>(out_bf16) & 15))
    return USAF_ERR_UNSUPPORTED;
  const int64_t words = rows * (cols / 8);
  timer_begin(USAF_K_DEQUANT, stream);
  hipLaunchKernelGGL(dequant_affine_kernel, dim3(grid_for(words)), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t*>(q), scale_f16, zero_f16, rows, cols, group,
                     static_cast<uint4*>(out_bf16));
  timer_end(USAF_K_DEQUANT, stream);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

extern "C" usaf_status usaf_dequant_resident(const uint8_t* q, const uint16_t* scale_f16,
                                             int64_t rows, int64_t cols, int32_t group,
                                             void* out_bf16, hipStream_t stream) {
  if (rows < 0 || cols < 0) return USAF_ERR_INVALID_ARG;
  if (group != 64 || cols % 64 != 0) return USAF_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return USAF_OK;
  if (!q || !scale_f16 || !out_bf16) return USAF_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q) & 3) || (reinterpret_cast<uintptr_t>(out_bf16) & 15))
    return USAF_ERR_UNSUPPORTED;
  const int64_t words = rows * (cols / 8);
  timer_begin(USAF_K_DEQUANT, stream);
  hipLaunchKernelGGL(dequant_int4_kernel, dim3(grid_for(words)), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t*>(q), scale_f16, rows, cols,
                     static_cast<uint4*>(out_bf16));
  timer_end(USAF_K_DEQUANT, stream);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

extern "C" usaf_status usaf_workspace_size(int32_t kind, const usaf_moe_shape* shape, int64_t n,
                                           int64_t k, size_t* bytes) {
  if (!bytes) return USAF_ERR_INVALID_ARG;
  switch (kind) {
    case USAF_WS_FORWARD:
      USAF_TRY(check_shape(shape));
      *bytes = ws_forward(*shape).total;
      return USAF_OK;
    case USAF_WS_BACKWARD:
      USAF_TRY(check_shape(shape));
      *bytes = ws_backward(*shape).total;
      return USAF_OK;
    case USAF_WS_TOPK:
      if (n < 0 || n >= (int64_t(1) << 32)) return USAF_ERR_INVALID_ARG;
      *bytes = topk_ws_bytes(n);
      return USAF_OK;
    case USAF_WS_RIGL:
      if (n < 0 || k < 0 || k > n || n >= (int64_t(1) << 32)) return USAF_ERR_INVALID_ARG;
      *bytes = rigl_ws_bytes(n, k);
      return USAF_OK;
    case USAF_WS_MASKED_PLAN:
      USAF_TRY(check_shape(shape));
      *bytes = shape->act == USAF_BF16 ? size_t(masked_plan_bytes(*shape)) : 256;
      return USAF_OK;
    case USAF_WS_UNION:
      if (n < 0 || n >= (int64_t(1) << 32)) return USAF_ERR_INVALID_ARG;
      *bytes = union_ws_bytes(n);
      return USAF_OK;
    default:
      return USAF_ERR_INVALID_ARG;
  }
}

__global__ __launch_bounds__(256) void adjacent_diff_kernel(const int32_t* __restrict__ in, int64_t n,
                                                             int32_t* __restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] = in[i + 1] - in[i];
}

extern "C" usaf_status usaf_adjacent_diff(const int32_t* in, int64_t n, int32_t* out,
                                          hipStream_t stream) {
  if (n < 0 || (n > 0 && (!in || !out))) return USAF_ERR_INVALID_ARG;
  if (n == 0) return USAF_OK;
  hipLaunchKernelGGL(adjacent_diff_kernel, dim3(unsigned(ceil_div(n, 256))), dim3(256), 0, stream,
                     in, n, out);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

extern "C" const char* usaf_status_string(usaf_status s) {
  switch (s) {
    case USAF_OK: return "ok";
    case USAF_ERR_INVALID_ARG: return "invalid argument";
    case USAF_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case USAF_ERR_WORKSPACE: return "workspace missing or too small";
    case USAF_ERR_HIP: return "HIP launch failed";
    case USAF_ERR_NOT_IMPLEMENTED: return "not implemented";
  }
  return "unknown status";
}

extern "C" int32_t usaf_version(void) { return 100; }
