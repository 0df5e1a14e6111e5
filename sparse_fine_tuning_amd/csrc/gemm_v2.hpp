// bf16 MFMA grouped GEMM for gfx950 with direct global->LDS staging.
//
// Block tile 128 x BN x 64 (BN = 128 or 256), 256 threads = 4 waves in a
// 2 x 2 grid; each wave computes 64 x BN/2 with v_mfma_f32_32x32x16_bf16
// (fp32 accumulate).  Operand tiles are copied straight from global memory
// into an NS-deep ring of LDS stages with 16-byte global_load_lds_dwordx4
// (no register staging), so the loads of stages kt+1 .. kt+NS-1 are in flight
// while stage kt feeds the matrix cores.
//
// Two operand forms:
//   k-major  (contraction index contiguous in memory, e.g. X rows, a weight
//            used as [N][K]): LDS [row][64 k] in 128-byte rows; 16-byte chunk
//            q of row r sits at slot q ^ (r & 7), so the 8 rows a 32-bank LDS
//            serves together hit distinct banks.  Fragments are read with
//            ds_read_b128.
//   mn-major (row index contiguous, e.g. a weight used as [K][N], or
//            activations contracted over slots): LDS [64 k][R rows]; chunk c
//            of k-row k sits at slot c ^ (2 (k & 3)).  Fragments are read with
//            two ds_read_b64_tr_b16 (gfx950's transposing LDS read), which
//            hand each lane 4 consecutive k of one row.
// Rows past the tile and k past the end read clamped, valid addresses; the
// k tail of the last stage is zeroed in LDS before it is used, and rows or
// columns past the tile are never stored.
//
// The MFMA is issued with the operands swapped (the B fragment as the
// instruction's first operand), so each lane's accumulator holds one row of
// the tile and runs of 4 consecutive columns: for block (i, j), lane l and
// element r = 4 g + e:
//   row = wm*64 + 32 i + (l % 32),  col = wn*BN/2 + 32 j + 8 g + 4 (l / 32) + e.
// Epilogues therefore read and write 4-column vectors per lane.
#pragma once

#include "common.hpp"
#include "gemm_mfma.hpp"

namespace usaf {
namespace g2 {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kBM = 128, kBK = 64;

// s_waitcnt with vmcnt <= n (expcnt and lgkmcnt left unconstrained).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One wave-wide 16-byte-per-lane copy: lane l's 16 bytes land at
// lds_base + 16 l.  lds_base must be the same for the whole wave.  Issued as
// inline assembly: completion is tracked only by the explicit vmcnt waits of
// the pipeline (the compiler's own tracking would wait for every copy in
// flight before each LDS read).  M0 holds the LDS address; one wait state
// separates its write from the copy.
__device__ __forceinline__ void dma16(const void* g, unsigned char* lds_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(uint32_t(size_t((lds_void_t*)lds_base)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(l)
               : "memory", "m0");
}

__device__ __forceinline__ int out_row(int wm, int i, int lane) { return wm * 64 + 32 * i + (lane & 31); }
// first of the 4 consecutive columns of group g of block j
__device__ __forceinline__ int out_col(int BN, int wn, int j, int g, int lane) {
  return wn * (BN / 2) + 32 * j + 8 * g + 4 * (lane >> 5);
}

// ---------------------------------------------------------------------------
// Operand staging.  A k-major operand of R rows supplies row(r) (element
// (r, 0); r < R, always a valid row).  An mn-major operand of R rows supplies
// kptr(k) (element (row 0, k); k < kend, always valid) and ncols (valid rows,
// a multiple of 8).
// ---------------------------------------------------------------------------
template <int R>
struct KMajor {
  static constexpr int kInst = R / 32;  // dma instructions per wave per stage
  static constexpr int kBytes = R * 128;
  const bf16_t* p[kInst];
  int kend;
  template <class Src>
  __device__ __forceinline__ void init(const Src& s, int kend_, int w, int lane) {
    kend = kend_;
    const int chunk = (lane & 7) ^ (lane >> 3);
#pragma unroll
    for (int i = 0; i < kInst; ++i) p[i] = s.row(w * (R / 4) + 8 * i + (lane >> 3)) + 8 * chunk;
  }
  // stage kt into lds (operand tile base)
  template <class Src>
  __device__ __forceinline__ void issue(const Src&, int kt, unsigned char* lds, int w, int lane) const {
    const int chunk = (lane & 7) ^ (lane >> 3);
    // a chunk past kend (kend % 64 != 0, last stage) reads the row's last
    // chunk instead; it is zeroed before use
    const int k0 = kt * kBK;
    const int over = k0 + 8 * chunk + 8 - kend;
    const int koff = over > 0 ? k0 - over : k0;
#pragma unroll
    for (int i = 0; i < kInst; ++i) dma16(p[i] + koff, lds + (w * (R / 4) + 8 * i) * 128);
  }
  // zero k >= kvalid (kvalid a multiple of 8) in a stage
  __device__ __forceinline__ static void zero_tail(unsigned char* lds, int kvalid, int tid) {
    for (int x = tid; x < R * 8; x += 256) {
      const int r = x >> 3, q = x & 7;
      if (8 * q >= kvalid)
        *reinterpret_cast<uint4*>(lds + r * 128 + 16 * (q ^ (r & 7))) = make_uint4(0, 0, 0, 0);
    }
  }
  // fragment rows base..base+31, k-substep kc
  __device__ __forceinline__ static bf16x8_t frag(const unsigned char* lds, int base, int kc, int lane) {
    const int r = base + (lane & 31);
    const int q = (2 * kc + (lane >> 5)) ^ (lane & 7);
    return *reinterpret_cast<const bf16x8_t*>(lds + r * 128 + 16 * q);
  }
};

template <int R>
struct MNMajor {
  static constexpr int kCPR = R / 8;         // 16-byte chunks per k-row
  static constexpr int kKPI = 64 / kCPR;     // k-rows per dma instruction
  static constexpr int kInst = kCPR / 4;     // dma instructions per wave per stage
  static constexpr int kBytes = kBK * R * 2;
  int kend, slot, last, krow0;
  template <class Src>
  __device__ __forceinline__ void init(const Src& s, int kend_, int w, int lane) {
    kend = kend_;
    krow0 = w * kInst * kKPI + lane / kCPR;  // k-row of this lane in its first instruction
    slot = lane % kCPR;
    last = s.ncols / 8 - 1;                  // chunks past the valid columns read the last one
  }
  template <class Src>
  __device__ __forceinline__ void issue(const Src& s, int kt, unsigned char* lds, int w, int) const {
#pragma unroll
    for (int i = 0; i < kInst; ++i) {
      const int kr = krow0 + i * kKPI;
      const int chunk = min(slot ^ (2 * (kr & 3)), last);
      const int k = min(kt * kBK + kr, kend - 1);
      dma16(s.kptr(k) + 8 * chunk, lds + (w * kInst + i) * kKPI * R * 2);
    }
  }
  __device__ __forceinline__ static void zero_tail(unsigned char* lds, int kvalid, int tid) {
    for (int x = tid + kvalid * kCPR; x < kBK * kCPR; x += 256)
      *reinterpret_cast<uint4*>(lds + x * 16) = make_uint4(0, 0, 0, 0);
  }
  // fragment rows base..base+31 (the contiguous dimension), k-substep kc
  __device__ __forceinline__ static bf16x8_t frag(const unsigned char* lds, int base, int kc, int lane) {
    const int g = lane >> 4, pq = lane & 15, jj = pq >> 2, q = pq & 3;
    const int n = base + 16 * (g & 1) + 4 * q;
    const int k = 16 * kc + 8 * (g >> 1) + jj;
    const int off = k * (R * 2) + 16 * ((n >> 3) ^ (2 * jj)) + 8 * (q & 1);
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds + off));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds + off + 4 * R * 2));
    typedef short s16x8_t __attribute__((ext_vector_type(8)));
    const s16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
  }
};

// ---------------------------------------------------------------------------
// The kernel.  P supplies
//   static constexpr int BN, NS; types AOp, BOp (KMajor<128> / MNMajor<128>,
//   KMajor<BN> / MNMajor<BN>)
//   bool tile(int L, MTile&)      (uniform per block; contraction [0, t.ke))
//   a_src(t), b_src(t): row(r) for a k-major operand, kptr(k) + ncols for an
//   mn-major one
//   void epilogue(const MTile&, f32x16_t (&acc)[2][BN/64], int wm, int wn, int lane)
// ---------------------------------------------------------------------------
template <class P>
__global__ __launch_bounds__(256) void gemm2_kernel(P p) {
  constexpr int BN = P::BN, NS = P::NS, NJ = BN / 64;
  using AOp = typename P::AOp;
  using BOp = typename P::BOp;
  constexpr int A_BYTES = AOp::kBytes, B_BYTES = BOp::kBytes;
  constexpr int NLOAD = AOp::kInst + BOp::kInst;
  static_assert((NS - 2) * NLOAD < 64, "vmcnt");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[NS][A_BYTES + B_BYTES];
  MTile t;
  if (!p.tile(xcd_remap_blocks(blockIdx.x, gridDim.x), t)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int K = t.ke;  // contraction range [0, ke)
  const auto as = p.a_src(t);
  const auto bs = p.b_src(t);
  AOp ao;
  BOp bo;
  ao.init(as, K, w, lane);
  bo.init(bs, K, w, lane);
  const int nk = (K + kBK - 1) / kBK;
  f32x16_t acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) {
      ao.issue(as, s, lds[s], w, lane);
      bo.issue(bs, s, lds[s] + A_BYTES, w, lane);
    }
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + NS - 2 < nk) wait_vmcnt<(NS - 2) * NLOAD>(); else wait_vmcnt<0>();
    __syncthreads();
    unsigned char* cur = lds[kt % NS];
    const int kvalid = K - kt * kBK;
    if (kvalid < kBK) {  // uniform: only the last stage
      AOp::zero_tail(cur, kvalid, tid);
      BOp::zero_tail(cur + A_BYTES, kvalid, tid);
      __syncthreads();
    }
    if (kt + NS - 1 < nk) {
      unsigned char* nxt = lds[(kt + NS - 1) % NS];
      ao.issue(as, kt + NS - 1, nxt, w, lane);
      bo.issue(bs, kt + NS - 1, nxt + A_BYTES, w, lane);
    }
    const unsigned char* As = cur;
    const unsigned char* Bs = cur + A_BYTES;
    // fragments of substep kc+1 are read while the MFMAs of kc run
    bf16x8_t af[2][2], bfr[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i) af[0][i] = AOp::frag(As, wm * 64 + 32 * i, 0, lane);
#pragma unroll
    for (int j = 0; j < NJ; ++j) bfr[0][j] = BOp::frag(Bs, wn * (BN / 2) + 32 * j, 0, lane);
#pragma unroll
    for (int kc = 0; kc < kBK / 16; ++kc) {
      const int c = kc & 1, n = c ^ 1;
      if (kc + 1 < kBK / 16) {
#pragma unroll
        for (int i = 0; i < 2; ++i) af[n][i] = AOp::frag(As, wm * 64 + 32 * i, kc + 1, lane);
#pragma unroll
        for (int j = 0; j < NJ; ++j) bfr[n][j] = BOp::frag(Bs, wn * (BN / 2) + 32 * j, kc + 1, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[c][j], af[c][i], acc[i][j], 0, 0, 0);
      if (kc + 1 < kBK / 16) {
        // interleave: one LDS read after each MFMA
#pragma unroll
        for (int q = 0; q < 2 * NJ; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
    }
  }
  p.epilogue(t, acc, wm, wn, lane);
}

}  // namespace g2
}  // namespace usaf
