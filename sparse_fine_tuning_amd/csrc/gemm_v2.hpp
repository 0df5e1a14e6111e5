// bf16 MFMA grouped GEMM for gfx950 with direct global->LDS staging.
//
// Block tile BM x BN x 64, WM x WN waves (4 or 8); each wave computes
// BM/WM x BN/WN with v_mfma_f32_32x32x16_bf16
// (fp32 accumulate).  Operand tiles are copied straight from global memory
// into an NS-deep ring of LDS stages with 16-byte global_load_lds_dwordx4
// (no register staging), so the loads of stages kt+1 .. kt+NS-1 are in flight
// while stage kt feeds the matrix cores.
//
// Two operand forms:
//   k-major  (contraction index contiguous in memory, e.g. X rows, a weight
//            used as [N][K]): LDS [row][64 k] in 128-byte rows; 16-byte chunk
//            q of row r sits at slot q ^ ((r / 2) mod 8), so the 16 rows that
//            the 64-bank LDS serves together in a 16-byte read hit distinct
//            banks (measured: 4 LDS cycles per ds_read_b128, no conflicts).
//            Fragments are read with ds_read_b128.
//   mn-major (row index contiguous, e.g. a weight used as [K][N], or
//            activations contracted over slots): LDS [64 k][R rows]; chunk c
//            of k-row k sits at slot c ^ (4 (k & 3)), which puts the 4 k-rows
//            read together in different 64-byte bank quarters.  Fragments are
//            read with two ds_read_b64_tr_b16 (gfx950's transposing LDS read),
//            which hand each lane 4 consecutive k of one row.
// Rows past the tile and k past the end read clamped, valid addresses; the
// k tail of the last stage is zeroed in LDS before it is used, and rows or
// columns past the tile are never stored.
//
// The MFMA is issued with the operands swapped (the B fragment as the
// instruction's first operand), so each lane's accumulator holds one row of
// the tile and runs of 4 consecutive columns: for block (i, j), lane l and
// element r = 4 g + e:
//   row = wm*RW + 32 i + (l % 32),  col = wn*CW + 32 j + 8 g + 4 (l / 32) + e.
// Epilogues therefore read and write 4-column vectors per lane.
#pragma once

#include <climits>
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "gemm_mfma.hpp"
#include "lds_dma.hpp"

namespace usaf {
namespace g2 {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kBM = 128;

// Blocks per CU and waves per SIMD of a BM x BN tile with NS stages of BK
// and NW waves: two blocks share a CU when both rings fit the 160 KiB LDS and
// each block has at most 4 waves (so one block's epilogue overlaps the other's
// main loop); otherwise one.
template <int BM, int BN, int BK, int NS, int NW>
struct Occupancy {
  static constexpr int kLds = NS * (BM + BN) * BK * 2;
  static constexpr int kBlocksPerCU = (2 * kLds + 1024 <= 160 * 1024 && NW <= 4) ? 2 : 1;
  static constexpr int kWavesPerEU = (kBlocksPerCU * NW + 3) / 4;
};

// Logical tile L -> (expert, column tile, row tile of BM rows) over device
// offsets[E+1]; tiles ordered expert-major, then column tile, then row tile.
// When BM is an odd number of 32-row blocks, a group of cnt rows takes
// ceil(cnt / BM) row tiles of equal size in whole blocks (the last one
// shorter): 256 rows under BM = 160 make two tiles of 128, not 160 + 96.
// Wave 0 scans the experts 64 at a time; false for the whole block past the end.
template <int BM>
__device__ __forceinline__ int row_tile(int cnt) {
  if constexpr ((BM / 32) % 2 == 0) return BM;
  const int n = (cnt + BM - 1) / BM;
  return n > 0 ? ((cnt + n - 1) / n + 31) / 32 * 32 : BM;
}
template <int BM>
__device__ __forceinline__ bool grouped_tile(const int32_t* __restrict__ offsets, int E, int NT,
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
      const int tiles = ((cnt + row_tile<BM>(cnt) - 1) / row_tile<BM>(cnt)) * NT;
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
  const int q = row_tile<BM>(cnt), mts = (cnt + q - 1) / q;
  t.nt = rem / mts;
  t.m0 = (rem - t.nt * mts) * q;
  t.mc = min(q, cnt - t.m0);
  t.off = sh[3];
  return true;
}

// Tiles of all groups (the grouped_tile numbering), block-uniform.
template <int BM>
__device__ __forceinline__ int grouped_count(const int32_t* __restrict__ offsets, int E, int NT) {
  __shared__ int total;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int sum = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
      int tiles = cnt > 0 ? ((cnt + row_tile<BM>(cnt) - 1) / row_tile<BM>(cnt)) * NT : 0;
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) tiles += __shfl_xor(tiles, d, 64);
      sum += tiles;
    }
    if (lane == 0) total = sum;
  }
  __syncthreads();
  const int t = total;
  __syncthreads();  // the next call may overwrite it
  return t;
}

// Problems that opt in (static constexpr bool kTailSplit = true) provide
// SplitWs sk, TailSplit split() and tile(L, t, plan), which numbers split
// units; the kernels compute the plan once per block.
template <class P, class = void>
struct TailSplitOf {
  static constexpr bool value = false;
};
template <class P>
struct TailSplitOf<P, std::void_t<decltype(P::kTailSplit)>> {
  static constexpr bool value = P::kTailSplit;
};

// Tail split of a persistent launch of G blocks over T tiles: when at least
// one full round of G tiles runs and the last round is at most half full,
// its tail = T mod G tiles are each cut into S <= 4 contraction parts (S tail
// <= G, S tail <= cap, S <= the tile's stages), so that the idle blocks of
// the last round share them.  Units: the full rounds' tiles in order, then
// tail tile i's parts as units full + S i + part.
// The plan depends on the persistent grid's size G.  No split: full = INT_MAX.
struct TailSplit {
  int full, tail, S;
};
// Partial buffer of a split launch: cap units of one tile's fp32
// accumulators; grid: the persistent launch's block count; hdr: where the
// launch leaves its plan (full, tail, S) for the reduction.
struct SplitWs {
  float* ws = nullptr;
  int cap = 0;
  int grid = 0;
  int* hdr = nullptr;
};
template <int BM, int BK>
__device__ __forceinline__ TailSplit grouped_split_plan(const int32_t* __restrict__ offsets, int E,
                                                        int NT, int K, const SplitWs& sk) {
  TailSplit p{INT_MAX, 0, 1};
  const int cap = sk.cap;
  if (cap < 2) return p;  // uniform
  const int T = grouped_count<BM>(offsets, E, NT), G = sk.grid;
  const int nk = (K + BK - 1) / BK;
  const int R = T / G, rem = T - R * G;
  if (R >= 1 && rem > 0 && 2 * rem <= G) {
    const int S = min(min(4, G / rem), min(cap / rem, nk));
    if (S >= 2) p = TailSplit{R * G, rem, S};
  }
  return p;
}
// Unit L of a grouped problem with contraction K (stages of BK) split by
// plan sp; false past the last unit.  A part covers stages
// [part nk / S, (part + 1) nk / S) of the tile, as [kb, ke).
template <int BM, int BK>
__device__ __forceinline__ bool grouped_split_tile(const int32_t* __restrict__ offsets, int E, int NT,
                                                   int L, int K, const TailSplit& sp, MTile& t) {
  const int nk = (K + BK - 1) / BK;
  int tl = L, part = 0;
  if (L >= sp.full) {
    const int j = L - sp.full;
    if (j >= sp.tail * sp.S) return false;
    tl = sp.full + j / sp.S;
    part = j % sp.S;
  }
  if (!grouped_tile<BM>(offsets, E, NT, tl, t)) return false;
  t.kb = 0;
  t.ke = K;
  t.nparts = 1;
  if (tl >= sp.full) {
    t.nparts = sp.S;
    t.part = part;
    t.tidx = tl - sp.full;
    t.kb = BK * (part * nk / sp.S);
    t.ke = min(K, BK * ((part + 1) * nk / sp.S));
  }
  return true;
}

// A split part's fp32 accumulators, raw (the MFMA layout, per thread), at
// unit u = tidx S + part of the partial buffer: float4 f of thread x at
// ((u F4 + f) NTHR + x), F4 = IM NJ 4 per thread.
template <int NTHR, int IM, int NJ>
__device__ __forceinline__ void store_partial(float* ws, int u, const f32x16_t (&acc)[IM][NJ], int tid) {
  constexpr int F4 = IM * NJ * 4;
  float4* dst = reinterpret_cast<float4*>(ws) + int64_t(u) * F4 * NTHR + tid;
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dst[((i * NJ + j) * 4 + q) * NTHR] =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
}
template <int NTHR, int IM, int NJ>
__device__ __forceinline__ void add_partial(const float* ws, int u, f32x16_t (&acc)[IM][NJ], int tid) {
  constexpr int F4 = IM * NJ * 4;
  const float4* src = reinterpret_cast<const float4*>(ws) + int64_t(u) * F4 * NTHR + tid;
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = src[((i * NJ + j) * 4 + q) * NTHR];
        acc[i][j][4 * q] += v.x;
        acc[i][j][4 * q + 1] += v.y;
        acc[i][j][4 * q + 2] += v.z;
        acc[i][j][4 * q + 3] += v.w;
      }
}

// CW: columns of the tile held by one wave
// first of the 4 consecutive columns of group g of block j
__device__ __forceinline__ int out_col(int CW, int wn, int j, int g, int lane) {
  return wn * CW + 32 * j + 8 * g + 4 * (lane >> 5);
}
// First tile row r0 and valid 32-row blocks vb of wave-row wm for a tile of
// mc rows.  kSplit (two wave-rows): the tile's blocks are shared evenly,
// wave-row 0 taking the odd one, so a 128-row tile under RW = 96 runs 2 + 2
// blocks; otherwise wave-row wm holds rows [wm RW, (wm + 1) RW).
template <bool kSplit, int RW, int IM>
__device__ __forceinline__ void wave_rows(int mc, int wm, int& r0, int& vb) {
  if constexpr (kSplit) {
    const int nb = (mc + 31) / 32, h = (nb + 1) / 2;
    r0 = wm ? 32 * h : 0;
    vb = min(IM, wm ? nb - h : h);
  } else {
    r0 = wm * RW;
    vb = min(IM, max(0, (mc - r0 + 31) / 32));
  }
}

// ---------------------------------------------------------------------------
// Operand staging.  A k-major operand of R rows supplies row(r) (element
// (r, 0); r < R, always a valid row).  An mn-major operand of R rows supplies
// kptr(k) (element (row 0, k); k < kend, always valid) and ncols (valid rows,
// a multiple of 8).
// ---------------------------------------------------------------------------
template <int R, int NW = 4, int BK = 64>
struct KMajor {
  static_assert(BK == 32 || BK == 64, "64- or 128-byte rows");
  static constexpr int kBK = BK;
  static constexpr int kRowB = BK * 2;       // bytes per staged row
  static constexpr int kCh = BK / 8;         // 16-byte chunks per row
  static constexpr int kRPI = 64 / kCh;      // rows per dma instruction
  static constexpr int kGroups = R / kRPI;   // dma instructions per stage (all waves)
  static constexpr int kFragReads = 1;       // LDS read instructions per fragment
  // dma instructions per wave per stage: when the waves cannot share the
  // row groups evenly, group g = i NW + w goes to wave w, and the first
  // kGroups % NW waves issue one more than the rest (kInstMin)
  static constexpr bool kEven = kGroups % NW == 0;
  static constexpr int kInst = (kGroups + NW - 1) / NW;
  static constexpr int kInstMin = kGroups / NW;
  static constexpr int kBytes = R * kRowB;
  static_assert(kGroups * kRPI == R && kInstMin > 0, "row groups");
  // first row of the wave's i-th instruction
  __device__ __forceinline__ static int group_row(int w, int i) {
    return kRPI * (kEven ? w * kInst + i : i * NW + w);
  }
  __device__ __forceinline__ static bool has_inst(int w, int i) {
    return kEven || i < kInstMin || w < kGroups - kInstMin * NW;
  }
  // slot of 16-byte chunk q in row r: 64 banks serve 16 lanes of a 16-byte
  // read together, i.e. 16 consecutive rows; 256 / kRowB consecutive rows
  // share a 256-byte bank line, so the chunk position is XOR-ed with the
  // line index mod kCh
  __device__ __forceinline__ static int sw(int r) { return (r / (256 / kRowB)) & (kCh - 1); }
  const bf16_t* p[kInst];
  int chunk[kInst];
  int kend;
  template <class Src>
  __device__ __forceinline__ void init(const Src& s, int kend_, int w, int lane) {
    kend = kend_;
#pragma unroll
    for (int i = 0; i < kInst; ++i) {
      const int r = (kEven ? group_row(w, i) : min(group_row(w, i), R - kRPI)) + lane / kCh;
      chunk[i] = (lane % kCh) ^ sw(r);
      p[i] = s.row(r) + 8 * chunk[i];
    }
  }
  // stage kt into lds (operand tile base)
  template <class Src>
  __device__ __forceinline__ void issue(const Src&, int kt, unsigned char* lds, int w, int) const {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < kInst; ++i) {
      if (!has_inst(w, i)) break;  // wave-uniform
      // a chunk past kend (kend % BK != 0, last stage) reads the row's last
      // chunk instead; it is zeroed before use
      const int over = k0 + 8 * chunk[i] + 8 - kend;
      const int koff = over > 0 ? k0 - over : k0;
      dma16(p[i] + koff, lds + group_row(w, i) * kRowB);
    }
  }
  // zero k >= kvalid (kvalid a multiple of 8) in a stage
  __device__ __forceinline__ static void zero_tail(unsigned char* lds, int kvalid, int tid) {
    for (int x = tid; x < R * kCh; x += 64 * NW) {
      const int r = x / kCh, q = x % kCh;
      if (8 * q >= kvalid)
        *reinterpret_cast<uint4*>(lds + r * kRowB + 16 * (q ^ sw(r))) = make_uint4(0, 0, 0, 0);
    }
  }
  static constexpr bool kPrep = false;  // nothing staged per tile
  static constexpr bool kConvert = false;
  __device__ __forceinline__ void convert(int, int) const {}
  // fragment rows base..base+31 (base a multiple of 32), k-substep kc
  __device__ __forceinline__ static bf16x8_t frag(const unsigned char* lds, int base, int kc, int lane,
                                                  int /*kt*/ = 0) {
    const int r = base + (lane & 31);
    const int q = (2 * kc + (lane >> 5)) ^ sw(r);
    return *reinterpret_cast<const bf16x8_t*>(lds + r * kRowB + 16 * q);
  }
};

template <int R, int NW = 4, int BK = 64>
struct MNMajor {
  static constexpr int kBK = BK;
  static constexpr int kCPR = R / 8;         // 16-byte chunks per k-row
  static constexpr int kKPI = 64 / kCPR;     // k-rows per dma instruction
  static constexpr int kFragReads = 2;       // LDS read instructions per fragment
  static constexpr int kInst = BK * kCPR / (64 * NW);  // dma instructions per wave per stage
  static constexpr int kInstMin = kInst;
  static constexpr int kBytes = BK * R * 2;
  static_assert(kInst * 64 * NW == BK * kCPR, "k-rows per wave");
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
      const int chunk = min(slot ^ (4 * (kr & 3)), last);
      const int k = min(kt * BK + kr, kend - 1);
      dma16(s.kptr(k) + 8 * chunk, lds + (w * kInst + i) * kKPI * R * 2);
    }
  }
  __device__ __forceinline__ static void zero_tail(unsigned char* lds, int kvalid, int tid) {
    for (int x = tid + kvalid * kCPR; x < BK * kCPR; x += 64 * NW)
      *reinterpret_cast<uint4*>(lds + x * 16) = make_uint4(0, 0, 0, 0);
  }
  static constexpr bool kPrep = false;  // nothing staged per tile
  static constexpr bool kConvert = false;
  __device__ __forceinline__ void convert(int, int) const {}
  // fragment rows base..base+31 (the contiguous dimension), k-substep kc
  __device__ __forceinline__ static bf16x8_t frag(const unsigned char* lds, int base, int kc, int lane,
                                                  int /*kt*/ = 0) {
    const int g = lane >> 4, pq = lane & 15, jj = pq >> 2, q = pq & 3;
    const int n = base + 16 * (g & 1) + 4 * q;
    const int k = 16 * kc + 8 * (g >> 1) + jj;
    const int off = k * (R * 2) + 16 * ((n >> 3) ^ (4 * jj)) + 8 * (q & 1);
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds + off));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds + off + 4 * R * 2));
    typedef short s16x8_t __attribute__((ext_vector_type(8)));
    const s16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
  }
};


// A k-major operand of R rows held as affine 4-bit codes in groups of G = 2^gshift
// along k (w = bf16(fp32(fp32(q - z) * s)), element 2i in the low nibble of
// byte i), dequantised in LDS one stage ahead of the MFMAs.  The codes do not
// go through the ring: a stage's 32 code bytes per row and its scale and
// zero pairs (the two fp16 of the aligned group pair holding the stage's
// group, 4 bytes each) arrive by DMA in a batch of their own, one stage
// further ahead than the other operand's stage in the same batch, into one
// of three code / scale buffers.  While the MFMAs of stage kt read the bf16
// tile of stage kt, the whole block converts stage kt + 1 (its loads landed
// with stage kt's wait) into the other of two bf16 tiles (KMajor's layout),
// in four parts between the MFMA substeps; the next stage's barrier
// publishes it.  A tile's first stage is converted before its main loop.
// Buffer reuse: the batch issued during stage kt fills code buffer
// (kt + NS) mod 3, last read while stage kt + NS - 3 <= kt was converted:
// during stage kt - 1, or (NS = 3, kt = 0) at the tile's start, which is
// why a first stage's conversion precedes its batch; tile (kt + 1) mod 2
// was last read by stage kt - 1.  Every
// batch issues the same loads (stages past the last reload the last), so
// the ring's vmcnt waits count them exactly.  Requirements: R = 32 NW (each
// wave loads 32 rows of codes and 64 scale or zero pairs per stage), the
// contraction a whole number of stages, G a multiple of 64, an even number
// kg of groups per row.  Src: code_row(r) -> global code row of tile row r
// (r < R, always valid); q, s, z; qpitch (bytes per code row), kg (groups
// per row), gshift.
template <int R, int NW>
struct KMajorQ4 {
  static constexpr int kBK = 64;
  static constexpr bool kConvert = true;
  using Tile = KMajor<R, NW, 64>;
  static constexpr int kFragReads = 1;
  static constexpr bool kPrep = false;
  static constexpr int kBytes = 0;     // nothing in the ring
  static constexpr int kInstMin = 2;   // per batch and wave: 32 code rows, 64 scale or zero pairs
  static constexpr int kCodeBuf = R * 32;
  static constexpr int kScaleBuf = 2 * R * 4;   // [s, z][row][the group pair]
  static constexpr int kTileBuf = R * 128;
  static_assert(R == 32 * NW && NW >= 2 && NW % 2 == 0, "one code and one scale instruction per wave");
  __device__ __forceinline__ static unsigned char* code_lds() {
    __shared__ __attribute__((aligned(16))) unsigned char buf[3 * kCodeBuf];
    return buf;
  }
  __device__ __forceinline__ static unsigned char* scale_lds() {
    __shared__ __attribute__((aligned(16))) unsigned char buf[3 * kScaleBuf];
    return buf;
  }
  __device__ __forceinline__ static unsigned char* tile_lds() {
    __shared__ __attribute__((aligned(16))) unsigned char buf[2 * kTileBuf];
    return buf;
  }
  // 8 weights from 4 code bytes: w = bf16(fp32(fp32(q - z) * s)), the low
  // and high nibbles of the four bytes each converted as a byte
  __device__ __forceinline__ static uint4 dequant8(uint32_t code, float sc, float zr) {
    const uint32_t lo = code & 0x0f0f0f0fu, hi = (code >> 4) & 0x0f0f0f0fu;
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float d0 = float((lo >> (8 * j)) & 0xffu) - zr;
      const float d1 = float((hi >> (8 * j)) & 0xffu) - zr;
      o[j] = f2bf2(d0 * sc, d1 * sc);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  }
  // The same weights by one fused multiply-add each, w = bf16(fma(q, s, -z s)),
  // for rows where it is exact: with s > 0 finite and z finite, 0 or
  // |z| >= 2^-10, q - z (q <= 15, z with at most 11 significant bits at
  // weight >= 2^-20), z s (22 bits) and q s (15 bits) are all exact in
  // fp32, so fma rounds the exact (q - z) s once, as fp32(fp32(q - z) s)
  // does, and an exact zero comes out +0 in both (s > 0).
  __device__ __forceinline__ static uint4 dequant8_fma(uint32_t code, float sc, float zs) {
    const uint32_t lo = code & 0x0f0f0f0fu, hi = (code >> 4) & 0x0f0f0f0fu;
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = f2bf2(__builtin_fmaf(float((lo >> (8 * j)) & 0xffu), sc, -zs),
                   __builtin_fmaf(float((hi >> (8 * j)) & 0xffu), sc, -zs));
    return make_uint4(o[0], o[1], o[2], o[3]);
  }
  __device__ __forceinline__ static bool fma_exact(float sc, float zr) {
    const float az = __builtin_fabsf(zr);
    return sc > 0.f && sc <= 65504.f && az <= 65504.f && (az == 0.f || az >= 0x1p-10f);
  }
  // A thread's share of converting a stage: R rows x 2 halves of the
  // stage's 64 k over the block's 64 NW = 2 R threads, one each; load()
  // reads its 16 code bytes and the row's scale and zero, part(j) writes
  // 8 weights (bf16 chunk 4 h + j of the row)
  struct Conv {
    uint4 q;
    float sc, zr, zs;
    unsigned char* dst;
    int r, h;
    bool fast;  // wave-uniform: every lane's row takes the fused form
  };
  __device__ __forceinline__ Conv conv_load(int st, int tid) const {
    Conv c;
    c.r = tid >> 1;
    c.h = tid & 1;
    const int b = st % 3;
    c.q = *reinterpret_cast<const uint4*>(code_lds() + b * kCodeBuf + c.r * 32 + 16 * c.h);
    const int half = (((st + kst0) << 6) >> gshift) & 1;  // the stage's group within its pair
    const unsigned char* sb = scale_lds() + b * kScaleBuf + c.r * 4 + 2 * half;
    c.sc = float(__builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t*>(sb)));
    c.zr = float(__builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t*>(sb + R * 4)));
    c.dst = tile_lds() + (st & 1) * kTileBuf + c.r * 128;
    c.zs = c.zr * c.sc;
    c.fast = __all(fma_exact(c.sc, c.zr));
    return c;
  }
  __device__ __forceinline__ static void conv_part(const Conv& c, int j) {
    const uint32_t qw = j == 0 ? c.q.x : j == 1 ? c.q.y : j == 2 ? c.q.z : c.q.w;
    *reinterpret_cast<uint4*>(c.dst + 16 * ((4 * c.h + j) ^ Tile::sw(c.r))) =
        c.fast ? dequant8_fma(qw, c.sc, c.zs) : dequant8(qw, c.sc, c.zr);
  }
  __device__ __forceinline__ void convert(int st, int tid) const {
    const Conv c = conv_load(st, tid);
#pragma unroll
    for (int j = 0; j < 4; ++j) conv_part(c, j);
  }
  const unsigned char* cptr;   // the lane's code row at its 16-byte chunk
  const uint16_t* sptr;        // the lane's scale or zero row
  int gshift, kg, last;        // last: the tile's last stage
  int kst0;                    // the row's stage of the tile's stage 0 (a contraction part's start)
  template <class Src>
  __device__ __forceinline__ void init(const Src& s, int kend, int w, int lane) {
    gshift = s.gshift;
    kg = s.kg;
    last = kend / 64 - 1;
    kst0 = s.kst0;
    cptr = s.q + s.code_row(32 * w + (lane >> 1)) * s.qpitch + 32 * kst0 + 16 * (lane & 1);
    const int sr = 64 * (w % (NW / 2)) + lane;  // scales: waves 0 .. NW/2 - 1, zeros: the rest
    sptr = (w < NW / 2 ? s.s : s.z) + s.code_row(sr % R) * s.kg;
  }
  // the code and scale loads of stage st (clamped to the last) into buffer st mod 3
  __device__ __forceinline__ void load_stage(int st, int w) const {
    const int b = st % 3;
    const int sc = min(st, last);
    dma16(cptr + 32 * sc, code_lds() + b * kCodeBuf + w * 1024);
    const int pair = (((sc + kst0) << 6) >> gshift) & ~1;
    dma4(sptr + pair, scale_lds() + b * kScaleBuf + (w >= NW / 2 ? R * 4 : 0) + (w % (NW / 2)) * 256);
  }
  // the batch of ring stage kt carries stage kt + 1's codes
  template <class Src>
  __device__ __forceinline__ void issue(const Src&, int kt, unsigned char*, int w, int) const {
    load_stage(kt + 1, w);
  }
  // before a tile's first batch: stage 0's codes
  template <class Src>
  __device__ __forceinline__ void issue_first(const Src&, int w) const { load_stage(0, w); }
  __device__ __forceinline__ static void zero_tail(unsigned char*, int, int) {}
  // fragment rows base..base+31, k-substep kc of stage kt: from stage kt's tile
  __device__ __forceinline__ bf16x8_t frag(const unsigned char*, int base, int kc, int lane, int kt) const {
    return Tile::frag(tile_lds() + (kt & 1) * kTileBuf, base, kc, lane);
  }
};

// lgkmcnt(0): this wave's LDS accesses have completed (the compiler cannot
// see the cross-lane dependence of the staging below).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15 << 0) | (7 << 4) | (0 << 8) | (3 << 14));
  asm volatile("" ::: "memory");
}

// Output staging through LDS.  A wave holds, for its 32-row block i, 32 rows
// x 32*NJ columns in the swapped MFMA layout (lane: one row, 4-column runs).
// These helpers write that block into the wave's own LDS region and read it
// back row-major, so that each global store instruction covers whole row
// segments (consecutive lanes, consecutive 16 bytes).  The caller must have
// finished every LDS read of the main loop (a block barrier) first.
//
// fp32: calls st(row, col4, float4) for rows 0..31 and col4 = 4*(lane%32)
// (a multiple of 4 below 32*NJ; rows 2q + lane/32).
// With region == nullptr the lane stores its own 4-column runs instead
// (st(row = lane%32, col4, float4)).
template <int NJ, class St>
__device__ __forceinline__ void stage_f32(unsigned char* region, const f32x16_t (&accr)[NJ], int lane,
                                          St&& st) {
  constexpr int kPitch = 32 * NJ * 4 + 16;  // bytes per staged row
  const int r = lane & 31, h = lane >> 5;
  if (NJ != 4 || region == nullptr) {  // staging needs 128 columns = 32 lanes x 4
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        st(r, 32 * j + 8 * g + 4 * h,
           make_float4(accr[j][4 * g], accr[j][4 * g + 1], accr[j][4 * g + 2], accr[j][4 * g + 3]));
    return;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(region + r * kPitch + 4 * (32 * j + 8 * g + 4 * h)) =
          make_float4(accr[j][4 * g], accr[j][4 * g + 1], accr[j][4 * g + 2], accr[j][4 * g + 3]);
  wave_lds_sync();
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int row = 2 * q + h;
    st(row, 4 * r, *reinterpret_cast<const float4*>(region + row * kPitch + 16 * r));
  }
  wave_lds_sync();
}

// One wave's block of 32 rows x NC bf16 columns (NC = 32 or 64) through a
// region of LDS private to the wave: the writers put packed words (4 columns)
// in the MFMA output layout; the block then leaves in 16-byte row pieces,
// NC/8 lanes per row, so one store instruction covers 64*8/NC whole row
// segments instead of 32 rows x 8 bytes.
template <int NC>
struct WaveRows {
  static_assert(NC == 32 || NC == 64, "16-byte pieces, at most 8 lanes per row");
  static constexpr int kPitch = NC * 2 + 16;
  static constexpr int kBytes = 32 * kPitch;
  static constexpr int kLanesPerRow = NC / 8, kRowsPerStore = 64 / kLanesPerRow;
  __device__ __forceinline__ static void put2(unsigned char* region, int row, int col, uint32_t w0,
                                              uint32_t w1) {
    *reinterpret_cast<uint2*>(region + row * kPitch + 2 * col) = make_uint2(w0, w1);
  }
  // st(row, col8, uint4): 8 columns from col8 of row; every row of the block
  template <class St>
  __device__ __forceinline__ static void drain(unsigned char* region, int lane, St&& st) {
    wave_lds_sync();  // the wave's puts have landed
    const int lr = lane / kLanesPerRow, lc = lane % kLanesPerRow;
#pragma unroll
    for (int q = 0; q < 32 / kRowsPerStore; ++q) {
      const int row = kRowsPerStore * q + lr;
      st(row, 8 * lc, *reinterpret_cast<const uint4*>(region + row * kPitch + 16 * lc));
    }
    wave_lds_sync();  // read back before the region is written again
  }
};

// ---------------------------------------------------------------------------
// The kernel.  P supplies
//   static constexpr int BM, BN, NS, WM, WN (wave grid), NTHR = 64 WM WN,
//   RW = BM/WM, CW = BN/WN, IM = RW/32, NJ = CW/32; types AOp, BOp
//   (KMajor<BM, NW> / MNMajor<BM, NW>, KMajor<BN, NW> / MNMajor<BN, NW>)
//   bool tile(int L, MTile&)      (uniform per block; contraction [0, t.ke))
//   a_src(t), b_src(t): row(r) for a k-major operand, kptr(k) + ncols for an
//   mn-major one
//   void epilogue(const MTile&, f32x16_t (&acc)[IM][NJ], int wm, int wn, int lane,
//                 unsigned char* stage)   (stage: kStageBytes of LDS private to the wave)
// Each wave computes RW x CW.
// ---------------------------------------------------------------------------
// The per-thread conversion state of an operand converted in LDS (none for
// the others).
template <class Op, class = void>
struct ConvOf {
  struct type {};
};
template <class Op>
struct ConvOf<Op, std::void_t<typename Op::Conv>> {
  using type = typename Op::Conv;
};

// Scheduling request for one substep of the main loop: its NM MFMAs, each
// followed by a share of the NR LDS fragment reads of the next substep, so
// every fragment is read about one substep before its MFMA needs it.
template <int NM, int NR>
__device__ __forceinline__ void interleave_mfma_reads() {
  static_for<NM>([&](auto m) {
    constexpr int mm = decltype(m)::value;
    constexpr int r = (NR * (mm + 1)) / NM - (NR * mm) / NM;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // r LDS reads
  });
}

template <class P, int VB, int IM, int NJ, class AOp, class BOp, class AS, class BS>
__device__ __forceinline__ void main_loop(const AOp& ao, const BOp& bo, const AS& as, const BS& bs,
                                          unsigned char (*lds)[AOp::kBytes + BOp::kBytes], int K,
                                          int nk, int tid, int w, int r0, int wn, int lane,
                                          f32x16_t (&acc)[IM][NJ]) {
  constexpr int NS = P::NS, CW = P::CW;
  constexpr int A_BYTES = AOp::kBytes;
  constexpr int NLOAD = AOp::kInstMin + BOp::kInstMin;  // the fewest any wave issues per stage
  constexpr int BK = AOp::kBK;
  static_assert(BOp::kBK == BK, "operands share the stage depth");
  constexpr int KC = BK / 16;
  constexpr int NM = VB * NJ;                                       // MFMAs per substep
  constexpr int NR = VB * AOp::kFragReads + NJ * BOp::kFragReads;   // LDS reads per substep
  // The MFMAs of a stage's last substep are issued after the next stage's
  // barrier, from fragments already in registers, so they cover the barrier
  // and the latency of the next stage's first LDS reads.  Stage 0 is peeled
  // (it has no such MFMAs), which keeps every stage body one basic block.
  bf16x8_t pa[VB > 0 ? VB : 1], pb[NJ];
  auto mfmas = [&](const bf16x8_t* a, const bf16x8_t* b) {
#pragma unroll
    for (int i = 0; i < VB; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
  };
  auto stage = [&](int kt, auto first) {
    constexpr bool kFirst = decltype(first)::value;
    if (kt + NS - 2 < nk) wait_vmcnt<(NS - 2) * NLOAD>(); else wait_vmcnt<0>();
    __syncthreads();
    unsigned char* cur = lds[kt % NS];
    const int kvalid = K - kt * BK;
    if (kvalid < BK) {  // uniform: only the last stage
      AOp::zero_tail(cur, kvalid, tid);
      BOp::zero_tail(cur + A_BYTES, kvalid, tid);
      __syncthreads();
    }
    // an operand converted in LDS: a tile's first stage before its MFMAs
    // (and before this stage's batch, whose loads may refill the buffer it
    // reads), then stage kt + 1 in four parts between this stage's substeps
    if constexpr (BOp::kConvert && kFirst) {
      bo.convert(0, tid);
      __syncthreads();
    }
    if (kt + NS - 1 < nk) {
      unsigned char* nxt = lds[(kt + NS - 1) % NS];
      ao.issue(as, kt + NS - 1, nxt, w, lane);
      bo.issue(bs, kt + NS - 1, nxt + A_BYTES, w, lane);
    }
    // (the last stage converts the reloaded last stage into the tile no
    // stage of this tile reads, which keeps the stage body free of branches)
    typename ConvOf<BOp>::type cv{};
    if constexpr (BOp::kConvert) cv = bo.conv_load(kt + 1, tid);
    auto conv_part = [&](int j) {
      if constexpr (BOp::kConvert) BOp::conv_part(cv, j);
    };
    if constexpr (VB > 0) {
      const unsigned char* As = cur;
      const unsigned char* Bs = cur + A_BYTES;
      // fragments of substep kc+1 are read while the MFMAs of kc run
      bf16x8_t af[2][VB], bfr[2][NJ];
#pragma unroll
      for (int i = 0; i < VB; ++i) af[0][i] = AOp::frag(As, r0 + 32 * i, 0, lane);
#pragma unroll
      for (int j = 0; j < NJ; ++j) bfr[0][j] = bo.frag(Bs, wn * CW + 32 * j, 0, lane, kt);
      if constexpr (!kFirst) {
        mfmas(pa, pb);  // the previous stage's last substep
        interleave_mfma_reads<NM, NR>();
      }
#pragma unroll
      for (int kc = 0; kc < KC - 1; ++kc) {
        const int c = kc & 1, n = c ^ 1;
#pragma unroll
        for (int i = 0; i < VB; ++i) af[n][i] = AOp::frag(As, r0 + 32 * i, kc + 1, lane);
#pragma unroll
        for (int j = 0; j < NJ; ++j) bfr[n][j] = bo.frag(Bs, wn * CW + 32 * j, kc + 1, lane, kt);
        mfmas(af[c], bfr[c]);
        interleave_mfma_reads<NM, NR>();
        if constexpr (KC == 4) conv_part(kc);
      }
      if constexpr (KC == 4) conv_part(3);
      constexpr int last = (KC - 1) & 1;
      static_assert(!BOp::kConvert || KC == 4, "the conversion is split over four substeps");
#pragma unroll
      for (int i = 0; i < VB; ++i) pa[i] = af[last][i];
#pragma unroll
      for (int j = 0; j < NJ; ++j) pb[j] = bfr[last][j];
    } else {
      // a wave with no rows in this tile still converts its share
#pragma unroll
      for (int j = 0; j < 4; ++j) conv_part(j);
    }
  };
  if (nk > 0) {
    stage(0, std::true_type{});
    for (int kt = 1; kt < nk; ++kt) stage(kt, std::false_type{});
    if constexpr (VB > 0) mfmas(pa, pb);
  }
}

template <class P>
__global__ __launch_bounds__(P::NTHR, P::kWavesPerEU) void gemm2_kernel(P p) {
  constexpr int NS = P::NS, IM = P::IM, NJ = P::NJ;
  using AOp = typename P::AOp;
  using BOp = typename P::BOp;
  constexpr int A_BYTES = AOp::kBytes, B_BYTES = BOp::kBytes;
  constexpr int NLOAD = AOp::kInstMin + BOp::kInstMin;  // the fewest any wave issues per stage
  static_assert((NS - 2) * NLOAD < 64, "vmcnt");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[NS][A_BYTES + B_BYTES];
  static_assert(P::kStageBytes * (P::NTHR / 64) <= NS * (A_BYTES + B_BYTES),
                "every wave's epilogue staging region lies in the ring");
  MTile t;
  if (!p.tile(xcd_remap_blocks(blockIdx.x, gridDim.x), t)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / P::WN, wn = w % P::WN;
  const int K = t.ke;  // contraction range [0, ke)
  const auto as = p.a_src(t);
  const auto bs = p.b_src(t);
  AOp ao;
  BOp bo;
  ao.init(as, K, w, lane);
  bo.init(bs, K, w, lane);
  const int nk = (K + AOp::kBK - 1) / AOp::kBK;
  if constexpr (BOp::kConvert) bo.issue_first(bs, w);
  f32x16_t acc[IM][NJ];
#pragma unroll
  for (int i = 0; i < IM; ++i)
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
  if constexpr (BOp::kPrep) bo.prep(bs, tid);  // per-tile operand state, published by the first stage's barrier
  main_loop<P, IM, IM, NJ>(ao, bo, as, bs, lds, K, nk, tid, w, wm * P::RW, wn, lane, acc);
  __syncthreads();  // the ring is free: epilogues may stage through it
  p.epilogue(t, acc, wm, wn, lane, &lds[0][0] + w * P::kStageBytes);
}

// Persistent form: a grid of about one block per CU walks the tile list
// (block b takes logical tiles x(b), x(b) + G, x(b) + 2G, ... with the
// XCD-aware x), and the first stages of the next tile are in flight while
// the current tile's epilogue stores.  Epilogues get no LDS staging area
// here (the ring holds the next tile's stages).
template <class P>
__global__ __launch_bounds__(P::NTHR, P::kWavesPerEU) void gemm2_persistent(P p) {
  constexpr int NS = P::NS, IM = P::IM, NJ = P::NJ;
  using AOp = typename P::AOp;
  using BOp = typename P::BOp;
  constexpr int A_BYTES = AOp::kBytes, B_BYTES = BOp::kBytes;
  constexpr int NLOAD = AOp::kInstMin + BOp::kInstMin;  // the fewest any wave issues per stage
  static_assert((NS - 2) * NLOAD < 64, "vmcnt");
  static_assert(P::kPStage * (P::NTHR / 64) <= A_BYTES + B_BYTES, "epilogue staging fits one ring stage");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[NS][A_BYTES + B_BYTES];
  const int G = gridDim.x;
  int L = xcd_remap_blocks(blockIdx.x, G);
  TailSplit plan{INT_MAX, 0, 1};
  if constexpr (TailSplitOf<P>::value) {
    plan = p.split();
    if (blockIdx.x == 0 && threadIdx.x == 0 && p.sk.hdr) {
      p.sk.hdr[0] = plan.full;
      p.sk.hdr[1] = plan.tail;
      p.sk.hdr[2] = plan.S;
    }
  }
  auto tile = [&](int l, MTile& tt) {
    if constexpr (TailSplitOf<P>::value) return p.tile(l, tt, plan);
    else return p.tile(l, tt);
  };
  MTile t;
  if (!tile(L, t)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / P::WN, wn = w % P::WN;
  // a tile's contraction is [kb, ke): the sources start at kb
  auto as = p.a_src(t);
  auto bs = p.b_src(t);
  AOp ao;
  BOp bo;
  int klen = t.ke - t.kb;
  ao.init(as, klen, w, lane);
  bo.init(bs, klen, w, lane);
  int nk = (klen + AOp::kBK - 1) / AOp::kBK;
  if constexpr (BOp::kConvert) bo.issue_first(bs, w);
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) {
      ao.issue(as, s, lds[s], w, lane);
      bo.issue(bs, s, lds[s] + A_BYTES, w, lane);
    }
  while (true) {
    // per-tile operand state (after the previous tile's last reads: the
    // barrier below its main loop), published by the first stage's barrier
    if constexpr (BOp::kPrep) bo.prep(bs, tid);
    f32x16_t acc[IM][NJ];
#pragma unroll
    for (int i = 0; i < IM; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    // 32-row blocks of this wave inside the tile's valid rows: a ragged
    // group's last tile issues MFMAs only for its valid row blocks
    int r0 = wm * P::RW, vb;
    if constexpr (P::kSplit) {
      wave_rows<true, P::RW, IM>(t.mc, wm, r0, vb);
      r0 = __builtin_amdgcn_readfirstlane(r0);
    } else {
      vb = min(IM, max(0, (t.mc - r0 + 31) / 32));
    }
    vb = __builtin_amdgcn_readfirstlane(vb);
    static_for<IM + 1>([&](auto V_) {
      constexpr int v = decltype(V_)::value;
      if (vb == v) main_loop<P, v, IM, NJ>(ao, bo, as, bs, lds, klen, nk, tid, w, r0, wn, lane, acc);
    });
    __syncthreads();  // every wave is done with the ring
    MTile tn;
    L += G;
    const bool more = tile(L, tn);
    if (more) {
      as = p.a_src(tn);
      bs = p.b_src(tn);
      klen = tn.ke - tn.kb;
      ao.init(as, klen, w, lane);
      bo.init(bs, klen, w, lane);
      nk = (klen + AOp::kBK - 1) / AOp::kBK;
      if constexpr (BOp::kConvert) bo.issue_first(bs, w);
#pragma unroll
      for (int s = 0; s < NS - 1; ++s)
        if (s < nk) {
          ao.issue(as, s, lds[s], w, lane);
          bo.issue(bs, s, lds[s] + A_BYTES, w, lane);
        }
    }
    // the epilogue stages through ring stage NS-1, which the next tile's
    // prologue leaves free (its first stage refills it only after a barrier
    // every wave reaches after its epilogue)
    unsigned char* pst = P::kPStage ? &lds[NS - 1][0] + w * P::kPStage : nullptr;
    if constexpr (TailSplitOf<P>::value) {
      // a part of a split tile leaves its raw sums for gemm2_split_reduce
      if (t.nparts > 1)
        store_partial<P::NTHR, IM, NJ>(p.sk.ws, t.tidx * t.nparts + t.part, acc, tid);
      else
        p.epilogue(t, acc, wm, wn, lane, pst);
    } else {
      p.epilogue(t, acc, wm, wn, lane, pst);
    }
    if (!more) break;
    t = tn;
  }
}

// The tiles a persistent launch split (grouped_split_plan, as the launch
// recorded it in sk.hdr; no tail: every block returns at once): one wave per
// block, block x = NW b + w for wave w of tail tile b (at most G NW blocks),
// adds that wave's accumulators over the tile's parts in part order and
// runs its share of the problem's epilogue (epilogues work per wave).
template <class P>
__global__ __launch_bounds__(64) void gemm2_split_reduce(P p) {
  constexpr int IM = P::IM, NJ = P::NJ, NW = P::NTHR / 64;
  constexpr int kStage = P::kPStage > 0 ? P::kPStage : 16;
  __shared__ __attribute__((aligned(16))) unsigned char stage[kStage];
  const TailSplit sp{p.sk.hdr[0], p.sk.hdr[1], p.sk.hdr[2]};
  const int b = blockIdx.x / NW, w = blockIdx.x % NW;
  if (b >= sp.tail) return;
  MTile t;
  if (!p.tile(sp.full + b * sp.S, t, sp)) return;
  const int lane = threadIdx.x, tid = 64 * w + lane;
  f32x16_t acc[IM][NJ];
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int q = 0; q < sp.S; ++q) add_partial<P::NTHR, IM, NJ>(p.sk.ws, b * sp.S + q, acc, tid);
  p.epilogue(t, acc, w / P::WN, w % P::WN, lane, P::kPStage > 0 ? stage : nullptr);
}

}  // namespace g2
}  // namespace usaf
