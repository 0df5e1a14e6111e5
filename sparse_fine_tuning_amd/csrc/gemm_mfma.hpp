// bf16 MFMA grouped GEMM skeleton for gfx950 (CDNA4, wave64).
//
// Block tile 128 x 128 x 64, 256 threads = 4 waves in a 2 x 2 grid, each wave
// computing 64 x 64 with v_mfma_f32_32x32x16_bf16 (fp32 accumulate).  Both
// operand tiles are staged in LDS as [row][k] (k contiguous, rows padded to
// 144 B so the 16 rows a quarter-wave reads land in distinct banks), double
// buffered: the next k-tile is fetched into registers while the current one
// feeds the matrix cores.
//
// An operand whose contraction index is contiguous in memory ("k-contiguous")
// is copied with 16-byte loads and stores.  An operand whose row index is
// contiguous ("row-contiguous", e.g. a weight used as [K][N], or token-major
// activations contracted over tokens) is loaded as 8 k-rows x 4 elements per
// thread and transposed in registers before the 16-byte LDS store.
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
};

// Logical tile ids are XCD-remapped (xcd_remap_blocks) so tiles that share
// weights or rows run on one XCD and share its L2.

// Logical tile L -> (expert, column tile, row tile) for groups whose row
// counts come from device offsets[E+1]; tiles ordered expert-major, then
// column tile, then row tile.  Wave 0 scans the experts 64 at a time and
// broadcasts through LDS; returns false (for the whole block) past the end.
__device__ __forceinline__ bool grouped_m_tile(const int32_t* __restrict__ offsets, int E, int NT,
                                               int L, MTile& t) {
  __shared__ int sh[4];
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    int base = 0;
    bool found = false;
    for (int e0 = 0; e0 < E && !found; e0 += 64) {
      const int e = e0 + lane;
      const int o0 = e < E ? offsets[e] : 0;
      const int cnt = e < E ? offsets[e + 1] - o0 : 0;
      const int tiles = ((cnt + kMB - 1) / kMB) * NT;
      int incl = tiles;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
      }
      const int excl = incl - tiles;
      const bool hit = tiles > 0 && L >= base + excl && L < base + incl;
      const uint64_t bal = __ballot(hit);
      if (bal) {
        if (lane == __ffsll((long long)bal) - 1) {
          sh[0] = e;
          sh[1] = L - base - excl;
          sh[2] = cnt;
          sh[3] = o0;
        }
        found = true;
      }
      base += __shfl(incl, 63, 64);
    }
    if (!found && lane == 0) sh[0] = -1;
  }
  __syncthreads();
  t.e = sh[0];
  if (t.e < 0) return false;
  const int rem = sh[1], cnt = sh[2];
  const int mts = (cnt + kMB - 1) / kMB;
  t.nt = rem / mts;
  t.m0 = (rem - t.nt * mts) * kMB;
  t.mc = min(kMB, cnt - t.m0);
  t.off = sh[3];
  return true;
}

// ---------------------------------------------------------------------------
// Operand loaders.  Src supplies:
//   k-contiguous:   int rows;  const E* row(int r) (row r's element 0), or
//                   nullptr for rows past the end; int kend.
//   row-contiguous: int rows (multiple of 4); int kend;
//                   const bf16_t* kptr(int k) (element (row 0, k));
//                   float scale(int k) when Src::kScaled.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f2bf(lo)) | (uint32_t(f2bf(hi)) << 16);
}

template <class E>
struct KcLoader;

template <>
struct KcLoader<bf16_t> {
  const bf16_t* rp[4];
  int c, kend;
  uint4 v[4];
  template <class Src>
  __device__ __forceinline__ void init(const Src& s, int tid) {
    c = tid & 7;
    kend = s.kend;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      rp[i] = r < s.rows ? s.row(r) : nullptr;
    }
  }
  __device__ __forceinline__ void load(int k0) {
    const int k = k0 + 8 * c;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = (rp[i] && k < kend) ? *reinterpret_cast<const uint4*>(rp[i] + k) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void store(bf16_t* S, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(&S[((tid >> 3) + 32 * i) * kLdsRow + 8 * c]) = v[i];
  }
};

// fp32 source rounded to bf16 while staging (the router weight).
template <>
struct KcLoader<float> {
  const float* rp[4];
  int c, kend;
  uint4 v[4];
  template <class Src>
  __device__ __forceinline__ void init(const Src& s, int tid) {
    c = tid & 7;
    kend = s.kend;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      rp[i] = r < s.rows ? s.row(r) : nullptr;
    }
  }
  __device__ __forceinline__ void load(int k0) {
    const int k = k0 + 8 * c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (rp[i] && k < kend) {
        const float4 x = *reinterpret_cast<const float4*>(rp[i] + k);
        const float4 y = *reinterpret_cast<const float4*>(rp[i] + k + 4);
        v[i] = make_uint4(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w), pack_bf16x2(y.x, y.y),
                          pack_bf16x2(y.z, y.w));
      } else {
        v[i] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(bf16_t* S, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(&S[((tid >> 3) + 32 * i) * kLdsRow + 8 * c]) = v[i];
  }
};

// Row-contiguous source: thread (mq = tid%32, kq = tid/32) loads k-rows
// kq*8 .. kq*8+7 of rows 4*mq .. 4*mq+3, then writes those 4 rows' 8 k-values
// as one 16-byte LDS store each.
template <class Src>
struct RcLoader {
  Src s;
  int mq, kq;
  bool live;
  uint2 v[8];
  __device__ __forceinline__ void init(const Src& src, int tid) {
    s = src;
    mq = tid & 31;
    kq = tid >> 5;
    live = 4 * mq < s.rows;
  }
  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + 8 * kq + i;
      if (live && k < s.kend) {
        uint2 x = *reinterpret_cast<const uint2*>(s.kptr(k) + 4 * mq);
        if constexpr (Src::kScaled) {
          const float sc = s.scale(k);
          x.x = pack_bf16x2(bf2f(bf16_t(x.x & 0xffffu)) * sc, bf2f(bf16_t(x.x >> 16)) * sc);
          x.y = pack_bf16x2(bf2f(bf16_t(x.y & 0xffffu)) * sc, bf2f(bf16_t(x.y >> 16)) * sc);
        }
        v[i] = x;
      } else {
        v[i] = make_uint2(0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(bf16_t* S, int) const {
    // element j of k-row i: 16-bit half (j&1) of word (j>>1) of v[i]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t a = (j < 2) ? v[2 * d].x : v[2 * d].y;
        const uint32_t b = (j < 2) ? v[2 * d + 1].x : v[2 * d + 1].y;
        w[d] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      *reinterpret_cast<uint4*>(&S[(4 * mq + j) * kLdsRow + 8 * kq]) = make_uint4(w[0], w[1], w[2], w[3]);
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
  typename P::ALoader la;
  typename P::BLoader lb;
  la.init(p.a_src(t), tid);
  lb.init(p.b_src(t), tid);
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = (t.ke - t.kb + kKB - 1) / kKB;
  if (nk > 0) {
    la.load(t.kb);
    lb.load(t.kb);
    la.store(As[0], tid);
    lb.store(Bs[0], tid);
  }
  __syncthreads();
  const int lrow = lane & 31, lk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(t.kb + (kt + 1) * kKB);
      lb.load(t.kb + (kt + 1) * kKB);
    }
    const bf16_t* Ab = As[cur];
    const bf16_t* Bb = Bs[cur];
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
    if (kt + 1 < nk) {
      la.store(As[cur ^ 1], tid);
      lb.store(Bs[cur ^ 1], tid);
    }
    __syncthreads();
  }
  p.epilogue(t, acc, wm, wn, lane);
}

// Row (within the 128-row tile) held by accumulator element r of lane `lane`
// in MFMA block i of wave row wm.
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return wn * 64 + j * 32 + (lane & 31); }

}  // namespace usaf
