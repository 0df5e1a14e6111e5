// Host-side shape validation and workspace layouts shared by the entry points.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "usaf.h"

namespace usaf {

// Bytes of a masked-gradient plan (segment starts and tile lists).
int64_t masked_plan_bytes(const usaf_moe_shape& s);
bool masked_dw_fits(const usaf_moe_shape& s);  // sizes the masked gradient kernels address
// Compute units of the current device (cached per device).
int device_cus();
// The loss kernels of usaf_mse_grad with their partial sums in `part`
// (ceil(T*H / 4096) floats, each written before it is read).
usaf_status mse_launch(const usaf_moe_shape& s, const void* Y, const void* tgt, void* dY,
                       float* loss, int32_t* nonfinite, float* part, hipStream_t stream);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline int64_t n_weights(const usaf_moe_shape& s) {
  return int64_t(3) * s.E * int64_t(s.H) * s.I;
}

// Shapes the kernels handle (see usaf_moe_shape in usaf.h).
inline usaf_status check_shape(const usaf_moe_shape* s) {
  if (!s) return USAF_ERR_INVALID_ARG;
  if (s->T < 1 || s->H < 1 || s->E < 1 || s->K < 1 || s->I < 1) return USAF_ERR_INVALID_ARG;
  if (s->K > s->E) return USAF_ERR_INVALID_ARG;
  if (s->act != USAF_F32 && s->act != USAF_BF16) return USAF_ERR_INVALID_ARG;
  if (s->E > 1024 || s->K > 64) return USAF_ERR_UNSUPPORTED;
  if (s->H % 64 != 0 || s->I % 32 != 0) return USAF_ERR_UNSUPPORTED;
  if (n_weights(*s) >= (int64_t(1) << 32)) return USAF_ERR_UNSUPPORTED;
  if (int64_t(s->T) * s->K >= (int64_t(1) << 31)) return USAF_ERR_UNSUPPORTED;
  return USAF_OK;
}

// Forward workspace: expert outputs before the combine, [S, H] in the
// activation dtype (sized for fp32; also holds the router split-K partials).
// bf16 layers keep the down GEMM's split partials in the second half.
struct WsForward {
  size_t ybuf, total;
};
// The half of an [S, H] fp32-sized region that bf16 rows leave free.
inline size_t bf16_spare_offset(const usaf_moe_shape& s) { return size_t(s.T) * s.K * s.H * 2; }
inline WsForward ws_forward(const usaf_moe_shape& s) {
  WsForward L;
  const size_t S = size_t(s.T) * s.K;
  L.ybuf = 0;
  size_t mse = ((size_t(s.T) * s.H + 4095) / 4096) * 4 + 64;
  size_t y = S * s.H * 4;
  size_t parts = size_t(8) * s.T * s.E * 4;  // router split-K partials (consumed before y)
  size_t m = y > mse ? y : mse;
  L.total = align256(m > parts ? m : parts);
  return L;
}

// Backward workspace: dX contributions [S, H] (activation dtype, sized for
// fp32), partial dw sums
// [S, NT] (NT = dA column tiles), dlogits of the chosen experts [S], and
// a masked-gradient plan built per call when the caller keeps none.
struct WsBackward {
  size_t vbuf, dwpart, dl, seg, wrb, total;
  int nt;
};
inline WsBackward ws_backward(const usaf_moe_shape& s) {
  WsBackward L;
  const size_t S = size_t(s.T) * s.K;
  L.nt = 4 * ((s.I + 127) / 128);  // >= ceil(I/64) and >= WN * ceil(I/BN) for WN <= 4, BN >= 128
  L.vbuf = 0;
  L.dwpart = align256(S * s.H * 4);
  L.dl = L.dwpart + align256(S * L.nt * 4);
  L.seg = L.dl + align256(S * 4);
  L.wrb = L.seg + align256(size_t(masked_plan_bytes(s)));  // bf16(Wr) [E, H] (bf16 layers)
  L.total = L.wrb + align256(size_t(s.E) * s.H * 2);
  return L;
}

}  // namespace usaf

namespace usaf {
// bf16 MFMA GEMMs of the layer (moe_mfma.hip).
usaf_status mfma_router(const usaf_moe_shape& s, const uint16_t* X, const float* Wr, float* parts,
                        int nparts, hipStream_t st);
// Split-K factor of the router GEMM (partial sums [nparts][T][E]).
constexpr int kMaxRouterParts = 8;
inline int mfma_router_splits(const usaf_moe_shape& s) {
  const int tiles = ((s.T + 127) / 128) * ((s.E + 127) / 128);
  int ks = 1;
  while (ks < kMaxRouterParts && tiles * ks < 256 && s.H / (64 * ks * 2) >= 1) ks *= 2;
  return ks;
}
// split_ws / split_bytes of the grouped GEMMs: scratch for the tail split's
// fp32 partials (see launch_persistent_split; none: no split), free while
// the GEMM runs and apart from its outputs.
usaf_status mfma_gate_up(const usaf_moe_shape& s, const uint16_t* X, const uint16_t* Wgu,
                         const int32_t* offsets, const int32_t* perm, uint16_t* gu, uint16_t* a,
                         float* split_ws, size_t split_bytes, hipStream_t st);
// split_ws: split_bytes of scratch for the tail split's fp32 partials
// (none: no split); not ybuf.
usaf_status mfma_down(const usaf_moe_shape& s, const uint16_t* a, const uint16_t* Wd,
                      const int32_t* offsets, uint16_t* ybuf, float* split_ws, size_t split_bytes,
                      hipStream_t st);
int mfma_dw_partials(const usaf_moe_shape& s);
usaf_status mfma_da(const usaf_moe_shape& s, const uint16_t* dY, const uint16_t* Wd,
                    const int32_t* offsets, const int32_t* perm, const float* topk_w,
                    const uint16_t* gu, const uint16_t* a, uint16_t* dgu, float* dwpart,
                    float* split_ws, size_t split_bytes, hipStream_t st);
usaf_status mfma_dx(const usaf_moe_shape& s, const uint16_t* dgu, const uint16_t* Wgu,
                    const int32_t* offsets, uint16_t* vbuf, float* split_ws, size_t split_bytes,
                    hipStream_t st);
// stage: S*H*2 bf16 scratch (the backward workspace's vbuf) for the
// expert-major gathered X and w*dY operands.
usaf_status mfma_dense_dw(const usaf_moe_shape& s, const uint16_t* X, const uint16_t* dY,
                          const uint16_t* dgu, const uint16_t* a, const int32_t* offsets,
                          const int32_t* perm, const float* topk_w, uint16_t* stage, float* dW,
                          hipStream_t st);

// Masked gradient of a bf16 layer at idx: with plan == NULL a plan is built
// in ws_plan (masked_plan_bytes) first.
usaf_status masked_dw_bf16(const usaf_moe_shape& s, const uint32_t* idx, int64_t nnz,
                           const uint16_t* X, const uint16_t* dY, const uint16_t* dgu,
                           const uint16_t* a, const float* topk_w, const int32_t* offsets,
                           const int32_t* perm, float* dW, int32_t* nonfinite, const void* plan,
                           void* ws_plan, hipStream_t st);
usaf_status masked_plan_bf16(const usaf_moe_shape& s, const uint32_t* idx, int64_t nnz, void* plan,
                             hipStream_t st);

// Workspace of one top-k selection over n keys / one RigL reselection.
size_t topk_ws_bytes(int64_t n);
size_t rigl_ws_bytes(int64_t N, int64_t k);
size_t union_ws_bytes(int64_t n);  // usaf_sorted_union of lists totalling n entries
// Forward expert GEMMs on 4-bit affine codes, dequantised as they load.
usaf_status q4_gate_up(const usaf_moe_shape& s, const uint16_t* X, const usaf_q4_experts& w,
                       const int32_t* offsets, const int32_t* perm, uint16_t* gu, uint16_t* a,
                       float* split_ws, size_t split_bytes, hipStream_t st);
usaf_status q4_down(const usaf_moe_shape& s, const uint16_t* a, const usaf_q4_experts& w,
                    const int32_t* offsets, uint16_t* ybuf, float* split_ws, size_t split_bytes,
                    hipStream_t st);
}  // namespace usaf
