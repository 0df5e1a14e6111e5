// bf16 MFMA GEMM skeleton for gfx950 (CDNA4, wave64), used by the router
// logits GEMM (split over the contraction, fp32 master weights rounded to
// bf16 while staging).  The expert GEMMs use the direct-to-LDS kernel in
// gemm_v2.hpp, which includes this header for its tile and vector types.
//
// Block tile 128 x 128 x 64, 256 threads = 4 waves in a 2 x 2 grid, each wave
// computing 64 x 64 with v_mfma_f32_32x32x16_bf16 (fp32 accumulate).  Both
// operand tiles are staged in LDS as [row][k] (k contiguous, rows padded to
// 144 B so the 16 rows a quarter-wave reads land in distinct banks), double
// buffered: the next k-tile is fetched into registers while the current one
// feeds the matrix cores.  Both operands are k-contiguous and are copied
// with 16-byte loads and stores.
//
// MFMA 32x32 output layout (per lane l, accumulator element r = 0..15):
//   row = 8*(r/4) + 4*(l/32) + (r%4),  col = l%32.
// The A/B input layouts only need to agree with each other on which k each
// lane supplies, so both use k = 8*(l/32) + 0..7 within a 16-wide k chunk.
#pragma once

#include "common.hpp"

namespace usaf {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kMB = 128, kNB = 128, kKB = 64;
constexpr int kLdsRow = kKB + 8;  // bf16 elements per LDS row

struct MTile {
  int e;       // group (expert)
  int m0, mc;  // first row / valid rows of the tile
  int n0, nc;  // first column / valid columns
  int kb, ke;  // contraction range [kb, ke)
  int off;     // expert-major row offset of the group
  int nt;      // column-tile index
  int part = 0, nparts = 1;  // a contraction part of a split tail tile: part of nparts
  int tidx = 0;              // the tail tile's index among the split ones
};

// Logical tile ids are XCD-remapped (xcd_remap_blocks) so tiles that share
// weights or rows run on one XCD and share its L2.

// ---------------------------------------------------------------------------
// Operand loaders.  Src supplies:
//   k-contiguous:   int rows;  const E* row(int r) (row r's element 0), or
//                   nullptr for rows past the end; int kend.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) { return f2bf2(lo, hi); }

template <class E>
struct KcLoader;

// Loads are branch-free: rows past the tile and k past the end read a
// clamped, valid address and are zeroed by a select, so the compiler can
// count outstanding loads exactly (no exec-masked load blocks).
template <>
struct KcLoader<bf16_t> {
  const bf16_t* rp[4];
  uint32_t ok;  // bit i: row i of this thread is inside the tile
  int c, kend;
  uint4 v[4];
  template <class Src>
  __device__ __forceinline__ void init(const Src& s, int tid) {
    c = tid & 7;
    kend = s.kend;
    ok = 0;
    const bf16_t* safe = s.row(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      const bf16_t* p = r < s.rows ? s.row(r) : nullptr;
      ok |= p ? (1u << i) : 0u;
      rp[i] = p ? p : safe;
    }
  }
  int klive;
  __device__ __forceinline__ void load(int k0) {
    const int k = k0 + 8 * c;
    const int kk = min(k, kend - 8);
    klive = k < kend;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const uint4*>(rp[i] + kk);
  }
  __device__ __forceinline__ void store(bf16_t* S, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool live = ((ok >> i) & 1u) && klive;
      const uint4 x = v[i];
      const uint4 y = make_uint4(live ? x.x : 0u, live ? x.y : 0u, live ? x.z : 0u, live ? x.w : 0u);
      *reinterpret_cast<uint4*>(&S[((tid >> 3) + 32 * i) * kLdsRow + 8 * c]) = y;
    }
  }
};

// fp32 source rounded to bf16 while staging (the router weight).
template <>
struct KcLoader<float> {
  const float* rp[4];
  uint32_t ok;
  int c, kend;
  float4 x[4], y[4];
  template <class Src>
  __device__ __forceinline__ void init(const Src& s, int tid) {
    c = tid & 7;
    kend = s.kend;
    ok = 0;
    const float* safe = s.row(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      const float* p = r < s.rows ? s.row(r) : nullptr;
      ok |= p ? (1u << i) : 0u;
      rp[i] = p ? p : safe;
    }
  }
  int klive;
  __device__ __forceinline__ void load(int k0) {
    const int k = k0 + 8 * c;
    const int kk = min(k, kend - 8);
    klive = k < kend;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = *reinterpret_cast<const float4*>(rp[i] + kk);
      y[i] = *reinterpret_cast<const float4*>(rp[i] + kk + 4);
    }
  }
  __device__ __forceinline__ void store(bf16_t* S, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool live = ((ok >> i) & 1u) && klive;
      const uint4 v = make_uint4(live ? pack_bf16x2(x[i].x, x[i].y) : 0u,
                                 live ? pack_bf16x2(x[i].z, x[i].w) : 0u,
                                 live ? pack_bf16x2(y[i].x, y[i].y) : 0u,
                                 live ? pack_bf16x2(y[i].z, y[i].w) : 0u);
      *reinterpret_cast<uint4*>(&S[((tid >> 3) + 32 * i) * kLdsRow + 8 * c]) = v;
    }
  }
};

// ---------------------------------------------------------------------------
// The kernel.  P supplies:
//   bool tile(int L, MTile&)                       (uniform per block)
//   ASrc a_src(const MTile&), BSrc b_src(const MTile&)
//   typedef ALoader / BLoader
//   void epilogue(const MTile&, f32x16_t acc[2][2], int wm, int wn, int lane)
// ---------------------------------------------------------------------------
template <class P>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(P p) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][kMB * kLdsRow];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][kNB * kLdsRow];
  MTile t;
  if (!p.tile(xcd_remap_blocks(blockIdx.x, gridDim.x), t)) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  // two register stages: k-tile kt+2 is in flight while kt is multiplied
  typename P::ALoader la0, la1;
  typename P::BLoader lb0, lb1;
  la0.init(p.a_src(t), tid);
  lb0.init(p.b_src(t), tid);
  la1 = la0;
  lb1 = lb0;
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = (t.ke - t.kb + kKB - 1) / kKB;
  if (nk > 0) {
    la0.load(t.kb);
    lb0.load(t.kb);
    if (nk > 1) {
      la1.load(t.kb + kKB);
      lb1.load(t.kb + kKB);
    }
    la0.store(As[0], tid);
    lb0.store(Bs[0], tid);
    if (nk > 2) {
      la0.load(t.kb + 2 * kKB);
      lb0.load(t.kb + 2 * kKB);
    }
  }
  __syncthreads();
  const int lrow = lane & 31, lk = (lane >> 5) * 8;
  auto mma = [&](const bf16_t* Ab, const bf16_t* Bb) {
#pragma unroll
    for (int kc = 0; kc < kKB / 16; ++kc) {
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&Ab[(wm * 64 + i * 32 + lrow) * kLdsRow + kc * 16 + lk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&Bb[(wn * 64 + j * 32 + lrow) * kLdsRow + kc * 16 + lk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };
  // iterations in pairs so each register stage has a fixed name
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    mma(As[0], Bs[0]);
    la1.store(As[1], tid);  // stage kt+1
    lb1.store(Bs[1], tid);
    if (kt + 3 < nk) {
      la1.load(t.kb + (kt + 3) * kKB);
      lb1.load(t.kb + (kt + 3) * kKB);
    }
    __syncthreads();
    mma(As[1], Bs[1]);
    if (kt + 2 < nk) {
      la0.store(As[0], tid);  // stage kt+2
      lb0.store(Bs[0], tid);
      if (kt + 4 < nk) {
        la0.load(t.kb + (kt + 4) * kKB);
        lb0.load(t.kb + (kt + 4) * kKB);
      }
    }
    __syncthreads();
  }
  if (kt < nk) mma(As[0], Bs[0]);  // odd count: last tile sits in buffer 0
  p.epilogue(t, acc, wm, wn, lane);
}

// Row (within the 128-row tile) held by accumulator element r of lane `lane`
// in MFMA block i of wave row wm.
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return wn * 64 + j * 32 + (lane & 31); }

}  // namespace usaf
