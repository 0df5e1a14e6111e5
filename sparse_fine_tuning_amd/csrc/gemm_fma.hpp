// LDS-tiled fp32-FMA grouped GEMM skeleton (64x64 tile, k-step 16, 256
// threads, 4x4 outputs per thread).  Used for fp32 layers, where the MFMA
// path does not apply.  A problem type P supplies:
//   struct Tile;                                   per-block tile description
//   bool get_tile(bx, by, bz, Tile&)               false -> the block has no work
//   int  kbeg(const Tile&), kend(const Tile&)      contraction range
//   void load_a(const Tile&, k0, float As[16][68], tid)   As[kk][m], zero-filled
//   void load_b(const Tile&, k0, float Bs[16][68], tid)   Bs[kk][n], zero-filled
//   void epilogue(const Tile&, float acc[4][4], tm, tn)   rows tm+16i, cols tn+16j
#pragma once

#include "common.hpp"

namespace usaf {

constexpr int kFmaBM = 64, kFmaBN = 64, kFmaBK = 16, kFmaLd = 68;

// Linear M-tile index -> (group, first row, rows) for groups whose row counts
// come from device offsets[G+1].  Uniform across the block.
__device__ __forceinline__ bool find_mtile(const int32_t* __restrict__ offsets, int G, int tile,
                                           int BM, int& g, int& m0, int& mcount) {
  int rem = tile;
  for (int e = 0; e < G; ++e) {
    int cnt = offsets[e + 1] - offsets[e];
    int nt = (cnt + BM - 1) / BM;
    if (rem < nt) {
      g = e;
      m0 = rem * BM;
      mcount = min(BM, cnt - m0);
      return true;
    }
    rem -= nt;
  }
  return false;
}

template <class P>
__global__ __launch_bounds__(256) void gemm_fma_kernel(P p) {
  __shared__ float As[kFmaBK][kFmaLd];
  __shared__ float Bs[kFmaBK][kFmaLd];
  typename P::Tile t;
  if (!p.get_tile(blockIdx.x, blockIdx.y, blockIdx.z, t)) return;
  const int tid = threadIdx.x, tm = tid >> 4, tn = tid & 15;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  const int kb = p.kbeg(t), ke = p.kend(t);
  for (int k0 = kb; k0 < ke; k0 += kFmaBK) {
    p.load_a(t, k0, As, tid);
    p.load_b(t, k0, Bs, tid);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFmaBK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][tm + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tn + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  p.epilogue(t, acc, tm, tn);
}

// Cooperative tile loaders.  "k-contiguous": element (r, k) at row_ptr(r)[k].
// "r-contiguous": element (r, k) at col_ptr(k)[r].  Out-of-range -> 0.
template <class RowFn>
__device__ __forceinline__ void load_kcontig(float (*S)[kFmaLd], int tid, int rcount, int k0,
                                             int kend, RowFn row_val) {
  const int kk = tid & 15;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = (tid >> 4) + 16 * rr;
    float v = 0.f;
    if (r < rcount && k0 + kk < kend) v = row_val(r, k0 + kk);
    S[kk][r] = v;
  }
}

template <class ColFn>
__device__ __forceinline__ void load_rcontig(float (*S)[kFmaLd], int tid, int rcount, int k0,
                                             int kend, ColFn val) {
  const int r = tid & 63;
#pragma unroll
  for (int kr = 0; kr < 4; ++kr) {
    const int kk = (tid >> 6) + 4 * kr;
    float v = 0.f;
    if (r < rcount && k0 + kk < kend) v = val(r, k0 + kk);
    S[kk][r] = v;
  }
}

}  // namespace usaf
