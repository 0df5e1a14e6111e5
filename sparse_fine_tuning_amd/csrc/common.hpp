// Device helpers shared by the USAF HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "usaf.h"

namespace usaf {

using bf16_t = uint16_t;  // bf16 storage (upper half of an fp32 word)

constexpr int kWave = 64;

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// f(std::integral_constant<int, 0>{}), ..., f(...<N-1>): a loop whose index is
// a compile-time constant in each copy (accumulator registers are indexed
// statically even where the body is too large for the unroller).
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// bf16 -> fp32 is exact: the bf16 bits are the fp32 word's upper half.
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays a NaN.  gfx950's
// v_cvt_pk_bf16_f32 converts two values per instruction; on every finite
// fp32 input (subnormals and infinities included) it gives the same bits as
// adding 0x7fff plus the kept lsb to the word and truncating.
typedef __bf16 hw_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float hw_f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  const hw_f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, hw_bf16x2_t));
}
__device__ __forceinline__ bf16_t f2bf(float f) { return bf16_t(f2bf2(f, 0.f) & 0xffffu); }

// Activation element access, fp32 or bf16 storage.
template <class T> struct Act;
template <> struct Act<float> {
  static constexpr int32_t code = USAF_F32;
  __device__ __forceinline__ static float ld(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void st(float* p, int64_t i, float v) { p[i] = v; }
  // value as stored (rounded to the storage type)
  __device__ __forceinline__ static float round(float v) { return v; }
};
template <> struct Act<bf16_t> {
  static constexpr int32_t code = USAF_BF16;
  __device__ __forceinline__ static float ld(const bf16_t* p, int64_t i) { return bf2f(p[i]); }
  __device__ __forceinline__ static void st(bf16_t* p, int64_t i, float v) { p[i] = f2bf(v); }
  __device__ __forceinline__ static float round(float v) { return bf2f(f2bf(v)); }
};

// Hardware exp2 and reciprocal (about 1 ulp each): the results are rounded to
// the activation type right after, and the fp32 path's error stays near 1e-7.
__device__ __forceinline__ float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
__device__ __forceinline__ float silu_f(float g) { return g * sigmoid_f(g); }

__device__ __forceinline__ bool finite_f(float v) { return (__float_as_uint(v) & 0x7f800000u) != 0x7f800000u; }

// Blocks are dealt round-robin to the 8 XCDs (each with its own L2); remap
// so that each XCD owns a contiguous range of logical block ids.  nb must be
// a multiple of 8.
__device__ __forceinline__ int xcd_remap_blocks(int b, int nb) { return (b & 7) * (nb >> 3) + (b >> 3); }

// Wave-wide helpers (64 lanes).
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Router weight as the forward GEMM multiplies it: bf16-rounded for bf16 layers.
template <class T> __device__ __forceinline__ float router_w(const float* Wr, int64_t i) {
  float w = Wr[i];
  return Act<T>::code == USAF_BF16 ? bf2f(f2bf(w)) : w;
}

}  // namespace usaf

// Host-side launch checking: every launcher returns a usaf_status.
#define USAF_LAUNCH_CHECK()                                         \
  do {                                                              \
    if (hipGetLastError() != hipSuccess) return USAF_ERR_HIP;       \
  } while (0)

#define USAF_TRY(expr)                                              \
  do {                                                              \
    usaf_status _s = (expr);                                        \
    if (_s != USAF_OK) return _s;                                   \
  } while (0)
