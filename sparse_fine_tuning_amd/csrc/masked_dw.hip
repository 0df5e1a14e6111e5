// Masked expert-weight gradient for bf16 layers: the gradient only at the
// selected ~0.5% of expert weights (usaf README intro and A100 per-operation
// table: gradients and optimiser state exist only for the selected subset).
//
// For one (tensor, expert) the selected entries are a sampled subset of
//   gate_up: G[r, c] = sum_p dGU[p, r] * X[tok(p), c]          (r < 2I, c < H)
//   down:    G[r, c] = sum_p (w_p dY[tok(p), r]) * a[p, c]     (r < H,  c < I)
// over the expert's slots p.  The work is cut into tiles of one expert's
// rows [r_lo, r_hi) x one column tile: a builder kernel splits each
// (expert, column tile)'s rows at quantiles of its entries, within the LDS
// row limit, so the tiles stay balanced however the selected entries cluster
// (an importance-selected list is far from uniform: a few rows carry hundreds
// of entries).  A block takes tiles in turn and streams the expert's slots in
// chunks of 8: the staging threads keep the loads of the next chunks in
// registers and transpose chunk c+1 into one of two slot-contiguous LDS
// buffers ([element][8 slots] bf16, one 16-byte read yields an entry's 8
// slot values) while every thread multiplies chunk c from the other, one
// barrier per chunk.  Entries are interleaved over the lanes of a wave;
// each thread accumulates its entries in branch-free groups of 4 with bf16
// dot2 (fp32 accumulation).  down stages bf16(w_p * dY), the product rounded
// once, as a bf16 autograd forms the down projection's output gradient.
#include <algorithm>
#include <cmath>

#include "common.hpp"
#include "moe_internal.hpp"
#include "timing.hpp"

namespace usaf {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kSlots = 8;        // slots per staged chunk
constexpr int kThreads = 512;    // 8 waves per block
constexpr int kMaxEnt = 24;      // entries per thread per pass
constexpr int kMaxCB = 2048;     // max columns per tile
template <bool kDown>
constexpr int kEnt = kMaxEnt;  // entries per thread per pass
template <bool kDown>
constexpr int kCap = kThreads * kEnt<kDown>;          // entries of one tile: one pass of a block
template <bool kDown>
constexpr int kTokTab = kDown ? 1024 : 2048;  // slots per token-table window (down: LDS for 2048 rows)
// staged chunks whose loads are in flight (register sets of the staging threads)
constexpr int kPreGateUp = 2;
constexpr int kPreDown = 1;
template <bool kDown>
constexpr int kPre = kDown ? kPreDown : kPreGateUp;
// max rows per tile: what the row operand's two LDS buffers allow (bf16,
// staged from r_lo rounded down to 8); down holds all 2048 rows of a
// Qwen3-sized expert, so a light expert takes one tile.  The host lowers the
// limit where rows and columns together would need more staging blocks than
// threads.
template <bool kDown>
constexpr int kMaxRows = kDown ? 2048 : 1536;
template <bool kDown>
constexpr int kLsBytes = (kMaxRows<kDown> + 8) * kSlots * 2;
// row limit for CB columns: LDS and one staging block per thread.  The
// column operand's CB / 8 blocks take whole waves, the row operand's blocks
// (rows staged from r_lo rounded down to 8, at most (RB + 14) / 8 of them)
// the threads after them.
template <bool kDown>
constexpr int row_limit(int CB) {
  const int col_threads = 64 * ((CB / 8 + 63) / 64);
  const int by_threads = (8 * (kThreads - col_threads) - 16) & ~7;
  return kMaxRows<kDown> < by_threads ? kMaxRows<kDown> : by_threads;
}
static_assert(row_limit<false>(kMaxCB) >= 8 && row_limit<true>(kMaxCB) >= 8, "rows per tile");
constexpr int kRsBytes = kMaxCB * kSlots * 2;
constexpr int kMaxCUs = 1024;  // bound on the CU count in plan sizes
static_assert(kMaxCB <= kThreads * kMaxEnt, "a single row fits a tile");

struct MaskedArgs {
  const uint32_t* idx; int64_t nnz;
  const bf16_t* L;        // gate_up: dGU [S, 2I]; down: dY [T, H]
  const bf16_t* Rm;       // gate_up: X [T, H];    down: a [S, I]
  const int32_t* offsets; const int32_t* perm; const float* topk_w;
  int K;
  int R, C;               // rows / columns of the per-expert gradient
  int CB, nct;            // column tiling
  int E;
  int64_t base;           // flat index of expert 0's (0,0) entry for this tensor
  float* dW; int32_t* nonfinite;
  const uint32_t* seg;    // plan: start in idx of every (expert, row, column tile) segment
  int64_t qbase;          // first segment id of this tensor
};

// Segments of the plan: tensor-major, then expert, row, column tile, so
// that segment q+1 starts where q ends (the flat order of the list).
struct SegLayout {
  int R0, C0, nct0, R1, C1, nct1, CB0, CB1, E;
  int64_t ngu, q1, Q;  // flat start of down, first down segment, segment count
};

// Words of the plan's 256-byte counter block: the two tensors' tile counts,
// their entry targets, then what identifies the list the plan was built
// for (its length, its address, its first and last entry).  The gradient
// kernel compares these with the list it is given before it reads a tile.
constexpr int kHdrTiles = 0, kHdrTarget = 2, kHdrNnz = 4, kHdrPtr = 6, kHdrFirst = 8,
              kHdrLast = 9;

__global__ __launch_bounds__(256) void masked_plan_kernel(const uint32_t* __restrict__ idx,
                                                          int64_t nnz, SegLayout Lq,
                                                          uint32_t* __restrict__ seg,
                                                          int* __restrict__ tile_counters,
                                                          int* __restrict__ ng, int ngroups) {
  const int64_t q = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q < 2) tile_counters[kHdrTiles + q] = 0;  // the tile builders append after this kernel
  if (q < ngroups) ng[q] = 0;                   // the group totals add into these
  if (q == 0) {
    uint32_t* hdr = reinterpret_cast<uint32_t*>(tile_counters);
    hdr[kHdrNnz] = uint32_t(uint64_t(nnz));
    hdr[kHdrNnz + 1] = uint32_t(uint64_t(nnz) >> 32);
    hdr[kHdrPtr] = uint32_t(reinterpret_cast<uintptr_t>(idx));
    hdr[kHdrPtr + 1] = uint32_t(uint64_t(reinterpret_cast<uintptr_t>(idx)) >> 32);
    hdr[kHdrFirst] = idx[0];
    hdr[kHdrLast] = idx[nnz - 1];
  }
  if (q > Lq.Q) return;
  int64_t key;  // flat index where segment q begins
  if (q == Lq.Q) {
    key = int64_t(1) << 40;
  } else if (q < Lq.q1) {
    const int64_t row = q / Lq.nct0, ct = q - row * Lq.nct0;  // row = e*R0 + r
    key = row * Lq.C0 + ct * Lq.CB0;
  } else {
    const int64_t qq = q - Lq.q1;
    const int64_t row = qq / Lq.nct1, ct = qq - row * Lq.nct1;
    key = Lq.ngu + row * Lq.C1 + ct * Lq.CB1;
  }
  int64_t lo = 0, hi = nnz;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (int64_t(idx[mid]) < key) lo = mid + 1; else hi = mid;
  }
  seg[q] = uint32_t(lo);
}

__device__ __forceinline__ int64_t lb_idx(const uint32_t* a, int64_t lo, int64_t hi, int64_t v) {
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (int64_t(a[mid]) < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Transpose 8 rows (slots) x 8 bf16 (one uint4 per slot) into 8 uint4 of
// 8 slot values each (one per element).  Output word d of element j pairs
// element j of slots 2d (low half) and 2d+1 (high half); both sit in word
// j/2 of their slot, in its low half for even j, high half for odd j.  One
// byte permute per output word: v_perm_b32 indexes the bytes of {S0, S1}
// with S1 as bytes 0-3 and S0 as bytes 4-7.
__device__ __forceinline__ uint32_t word_of(const uint4& v, int w) {
  return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
}
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
      w[d] = __builtin_amdgcn_perm(word_of(in[2 * d + 1], j >> 1), word_of(in[2 * d], j >> 1), sel);
    out[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// LDS slot swizzles.  Staging writes 16-byte units for consecutive lanes at
// a 128-byte stride (8 units apart); XOR-ing bits of the unit index into its
// low 3 bits spreads those lanes over all 16 bank groups of a 256-byte window.
// 32-byte units (fp32 staging) are 8 apart in the same way.
__device__ __forceinline__ uint32_t sw16(uint32_t u) { return u ^ ((u >> 4) & 7u); }

// One staging block: 8 slots x 8 consecutive elements of one operand row.
struct StageRegs {
  uint4 v[kSlots];
  float w[kSlots];
};

// Staging roles.  The waves [0, ncw) stage the column operand (lane b: the
// block of columns 8b..8b+7 of the tile), the waves after them the row
// operand (rows from r_lo rounded down to 8); lanes past their operand's
// blocks load its last block again and store nothing.  An operand's rows are
// tokens (gate_up X, down dY) or the expert's slots (gate_up dGU, down a), so
// within a wave the base pointer and the row pitch are uniform and each
// lane's load is that base plus a 32-bit offset.
struct StageRole {
  const unsigned char* base;  // wave-uniform: the operand's first element of the tile
  uint32_t ld2;               // wave-uniform: bytes per operand row
  bool col;                   // wave-uniform: the column operand
  bool by_tok;                // wave-uniform: operand rows are tokens
  bool stores;                // the lane's block lies in the tile
  uint32_t lane_off;          // bytes from base to the lane's block
  uint32_t unit;              // the block's first 16-byte LDS unit
};

// The loads of a chunk are issued without branches: a slot past the
// window's end reloads a valid row (the row tables are padded to a whole
// chunk; such slots are zeroed when stored), so every thread issues exactly
// kSlots loads per chunk and the waits before a store need only cover the
// oldest chunk in flight.
template <bool kDown>
__device__ __forceinline__ void stage_fetch(const StageRole& R, int p0, const int* tok_tab,
                                            const int* slot_tab, const float* w_tab,
                                            StageRegs& sr) {
  // p0 (a multiple of 8) indexes the window's tables
  if constexpr (kDown) {
    if (!R.col) {  // dY rows are scaled by the slots' routing weights when stored
      const float4 wa = *reinterpret_cast<const float4*>(w_tab + p0);
      const float4 wb = *reinterpret_cast<const float4*>(w_tab + p0 + 4);
      sr.w[0] = wa.x; sr.w[1] = wa.y; sr.w[2] = wa.z; sr.w[3] = wa.w;
      sr.w[4] = wb.x; sr.w[5] = wb.y; sr.w[6] = wb.z; sr.w[7] = wb.w;
    }
  }
  // the chunk's 8 operand rows: tokens, or slots from slot0 (the row
  // table of the wave's operand; two 16-byte LDS reads), then 8 loads from
  // the wave-uniform base at 32-bit offsets
  const int* rt = R.by_tok ? tok_tab : slot_tab;
  const int4 ta = *reinterpret_cast<const int4*>(rt + p0);
  const int4 tb = *reinterpret_cast<const int4*>(rt + p0 + 4);
  const int row[8] = {ta.x, ta.y, ta.z, ta.w, tb.x, tb.y, tb.z, tb.w};
#pragma unroll
  for (int t = 0; t < kSlots; ++t)
    sr.v[t] = *reinterpret_cast<const uint4*>(R.base + (__umul24(uint32_t(row[t]), R.ld2) + R.lane_off));
}

template <bool kDown>
__device__ __forceinline__ void stage_store(const StageRole& R, StageRegs sr, int p0, int pend,
                                            unsigned char* lds_l, unsigned char* lds_r) {
  if (p0 + kSlots > pend) {  // uniform: the window's last chunk, its slots past the end zeroed
    asm volatile("");  // kept a branch: the other chunks skip the masking
#pragma unroll
    for (int t = 0; t < kSlots; ++t) {
      const uint32_t m = p0 + t < pend ? 0xffffffffu : 0u;
      sr.v[t] = make_uint4(sr.v[t].x & m, sr.v[t].y & m, sr.v[t].z & m, sr.v[t].w & m);
      sr.w[t] = __uint_as_float(__float_as_uint(sr.w[t]) & m);
    }
  }
  uint4 out[8];
  if (!kDown || R.col) {
    transpose8x8(sr.v, out);
  } else {
    // down: bf16(w_p * dY) for the 8 slots of each element, slots 2d and
    // 2d+1 in word d (the product rounded once, as a bf16 autograd forms
    // the down projection's output gradient)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t w[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t a = word_of(sr.v[2 * d], j >> 1), c = word_of(sr.v[2 * d + 1], j >> 1);
        const float x0 = (j & 1) ? bfhi(a) : bflo(a), x1 = (j & 1) ? bfhi(c) : bflo(c);
        w[d] = f2bf2(sr.w[2 * d] * x0, sr.w[2 * d + 1] * x1);
      }
      out[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  unsigned char* dst = R.col ? lds_r : lds_l;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<uint4*>(dst + size_t(sw16(R.unit + uint32_t(j))) * 16) = out[j];
}

// Entries of each group g = (expert e, column tile ct) of one tensor.  With
// one column tile a group's rows are consecutive segments (one difference);
// otherwise block (g, sub) adds the counts of its share of the group's rows
// (each thread kUnroll independent loads at a time, rows past the share
// clamped and counted as empty) into ng[g], which the plan kernel zeroed.
__global__ __launch_bounds__(256) void masked_group_totals_kernel(const uint32_t* __restrict__ seg,
                                                                  int64_t qbase, int E, int R, int nct,
                                                                  int* __restrict__ ng) {
  const int g = blockIdx.x, tid = threadIdx.x;
  const int e = g / nct, ct = g - e * nct;
  const int64_t q0 = qbase + int64_t(e) * R * nct + ct;
  if (nct == 1) {
    if (blockIdx.y == 0 && tid == 0) ng[g] = int(seg[q0 + R] - seg[q0]);
    return;
  }
  constexpr int kUnroll = 8;
  const int per = (R + int(gridDim.y) - 1) / int(gridDim.y);
  const int r_lo = int(blockIdx.y) * per, r_hi = min(R, r_lo + per);
  int part = 0;
  for (int r0 = r_lo; r0 < r_hi; r0 += 256 * kUnroll) {
    uint2 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const uint32_t* p = seg + q0 + int64_t(min(r0 + 256 * j + tid, R - 1)) * nct;
      v[j] = make_uint2(p[0], p[1]);
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) part += int(v[j].y - v[j].x) & -int(r0 + 256 * j + tid < r_hi);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) part += __shfl_xor(part, d, 64);
  __shared__ int red[4];
  if ((tid & 63) == 0) red[tid >> 6] = part;
  __syncthreads();
  if (tid == 0) atomicAdd(ng + g, (red[0] + red[1]) + (red[2] + red[3]));
}

// The tensor-wide entry target of a tile: the smallest t <= cap with
// sum over groups of max(ceil(R/RB), ceil(n_g / t)) <= rounds * cus, where
// rounds is the number of CU rounds that full tiles (t = cap) take.  A light
// list then takes one tile per row range and expert while a heavy expert's
// entries are spread over the CUs the light ones leave idle, and a list too
// large for one round fills its last round instead of leaving it part
// empty.  Either way t < cap adds fewer than cus tiles.  One block.
__global__ __launch_bounds__(256) void masked_target_kernel(const int* __restrict__ ng, int G, int R,
                                                            int RB, int cap, int cus,
                                                            int* __restrict__ target) {
  __shared__ int red[4];
  const int tid = threadIdx.x;
  const int nr = (R + RB - 1) / RB;
  auto tiles_at = [&](int t) {
    int c = 0;
    for (int g = tid; g < G; g += 256) {
      const int n = ng[g];
      if (n > 0) c += max(nr, int((int64_t(n) + t - 1) / t));
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d, 64);
    __syncthreads();  // red is free
    if ((tid & 63) == 0) red[tid >> 6] = c;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
  };
  // whole rounds of the CUs: when even full tiles need more than one round,
  // the smallest target that still fits the same number of rounds spreads
  // the entries evenly instead of leaving a part-filled last round
  const int rounds = max(1, (tiles_at(cap) + cus - 1) / cus);
  const int bound = rounds * cus;
  int lo = 1, hi = cap;  // invariant: tiles_at(hi) <= bound
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    if (tiles_at(mid) <= bound) hi = mid; else lo = mid + 1;
  }
  if (tid == 0) *target = lo;
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts by 1, 2,
// 4 and 8 (lanes without a source add 0) give each 16-lane row its own
// prefix; the row-15 broadcast adds row 0's total into row 1 and row 2's
// into row 3, the row-31 broadcast adds rows 0-1 into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  int v = x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return v;
}

// Tiles of one tensor.  Group g = (expert e, column tile ct), e-major; its
// rows' entry counts come from the plan's segment starts (per group fewer
// than 2^31 entries).  The group is split into nt = max(ceil(R / RB),
// ceil(n / min(cap, target))) tiles of about n / nt entries each (n: the
// group's entries, target: the tensor-wide entry target): one wave per group walks the rows 64 at a time and closes the
// open tile [open_r, r) before row r when it holds RB rows, when row r would
// take it past cap entries, or when the entries before r reach the next
// multiple of n / nt and the rows from r on fit in the tiles still planned
// (so that a row-limited split is not followed by a sliver).  A single row never exceeds cap (at most kMaxCB
// entries), so every tile is one pass of a block.  Splitting at the
// quantiles keeps the tiles of a group even however its entries cluster (an
// importance-selected list puts hundreds of entries in a few rows and leaves
// others empty) and gives a light expert a single tile.  A group's tiles are
// appended together at an atomically reserved position: the order of the
// groups in the list changes no result, since every tile's entries are
// computed the same way by whichever block takes it.
// Tile: x = e | ct << 16, y = r_lo | r_hi << 16.
__global__ __launch_bounds__(256) void masked_tiles_kernel(const uint32_t* __restrict__ seg,
                                                           int64_t qbase, int E, int R, int nct,
                                                           int RB, int cap, const int* __restrict__ ng,
                                                           const int* __restrict__ target,
                                                           uint2* __restrict__ tiles,
                                                           int* __restrict__ ntiles) {
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= E * nct) return;  // uniform per wave
  const int e = g / nct, ct = g - e * nct;
  const uint32_t tx = uint32_t(e) | (uint32_t(ct) << 16);
  // segment of row r: q0 + r*nct; its entries: seg[q+1] - seg[q]
  const int64_t q0 = qbase + int64_t(e) * R * nct + ct;
  const int total = ng[g];
  if (total == 0) return;  // uniform
  // tiles of about total / nt entries: at most cap (one pass of a block) and
  // at most the tensor-wide target, which spreads the work over the CUs
  const int tcap = min(cap, *target);
  const int nt = max(int((R + RB - 1) / RB), int((int64_t(total) + tcap - 1) / tcap));
  // One walk over the rows records the group's tiles in registers (tile i
  // in lane i mod 64 of rec[i / 64]); the group then reserves them at once,
  // so its tiles stay consecutive in the list, and its lanes write them.  A
  // group with more than kRec tiles walks a second time to write them.  The
  // walk reads the counts of kSpan chunks of 64 rows with independent loads
  // (rows past R clamped to a valid segment and counted as empty), the next
  // span's while it scans the current one chunk by chunk.
  constexpr int kSpan = 16, kRecRegs = 4, kRec = 64 * kRecRegs;
  // (the counts are formed where they are used, so that nothing waits for
  // the loads before the scan that precedes their use)
  auto load_span = [&](int s0, uint2 (&cnts)[kSpan]) {
#pragma unroll
    for (int j = 0; j < kSpan; ++j) {
      const int r = min(s0 + 64 * j + lane, R - 1);
      const uint32_t* p = seg + q0 + int64_t(r) * nct;
      cnts[j] = make_uint2(p[0], p[1]);
    }
    __builtin_amdgcn_sched_barrier(0);  // issued here, not next to their use
  };
  uint32_t rec[kRecRegs];
#pragma unroll
  for (int i = 0; i < kRecRegs; ++i) rec[i] = 0;
  int base = 0;
#pragma unroll 1
  for (int walk = 0; walk < 2; ++walk) {
    int open_r = 0, open_x = 0;  // first row of the open tile, its exclusive prefix
    int carry = 0;               // exclusive prefix of the chunk's first row
    int n = 0;                   // tiles with entries so far
    int ncut = 0;                // cuts so far
    // the first multiple of total / nt beyond the open tile's start (it
    // changes only at a cut)
    auto next_quant = [&](int ox) {
      const int64_t k = int64_t(ox) * nt / total + 1;
      return (k * total + nt - 1) / nt;
    };
    int64_t quant = next_quant(0);
    auto emit = [&](int r_lo, int r_hi) {
      const uint32_t y = uint32_t(r_lo) | (uint32_t(r_hi) << 16);
      if (walk == 0) {
#pragma unroll
        for (int i = 0; i < kRecRegs; ++i)
          if (n == 64 * i + lane) rec[i] = y;
      } else if (lane == 0) {
        tiles[base + n] = make_uint2(tx, y);
      }
      ++n;
    };
    auto scan_span = [&](int s0, const uint2 (&cnts)[kSpan]) {
#pragma unroll
      for (int j = 0; j < kSpan; ++j) {
        const int r0 = s0 + 64 * j;
        if (r0 >= R) break;  // uniform
        const int r = r0 + lane;
        const int cnt = int(cnts[j].y - cnts[j].x) & -int(r < R);
        const int incl = wave_incl_scan(cnt);
        const int excl = carry + incl - cnt;
        // at most one cut per row, taken in row order
        while (true) {
          // a cut at the quantile only once the rows after it fit the tiles left
          const bool cut = r < R && r > open_r &&
                           (r - open_r >= RB || excl + cnt - open_x > cap ||
                            (int64_t(excl) >= quant && int64_t(R - r) <= int64_t(nt - ncut - 1) * RB));
          const uint64_t m = __ballot(cut);
          if (!m) break;
          const int c = __ffsll((long long)m) - 1;
          const int cr = r0 + c;
          const int cx = __builtin_amdgcn_readlane(excl, c);
          if (cx > open_x) emit(open_r, cr);
          open_r = cr;
          open_x = cx;
          quant = next_quant(open_x);
          ++ncut;
        }
        carry += __builtin_amdgcn_readlane(incl, 63);
      }
    };
    // two span buffers, each refilled right after it is scanned (the last
    // refills read clamped rows and go unused)
    uint2 ca[kSpan], cb[kSpan];
    load_span(0, ca);
    for (int s0 = 0; s0 < R; s0 += 2 * 64 * kSpan) {
      load_span(s0 + 64 * kSpan, cb);
      scan_span(s0, ca);
      load_span(s0 + 2 * 64 * kSpan, ca);
      if (s0 + 64 * kSpan < R) scan_span(s0 + 64 * kSpan, cb);  // uniform
    }
    if (carry > open_x) emit(open_r, R);
    if (walk == 0) {
      if (lane == 0) base = atomicAdd(ntiles, n);
      base = __shfl(base, 0, 64);
      if (n <= kRec) {
#pragma unroll
        for (int i = 0; i < kRecRegs; ++i)
          if (64 * i + lane < n) tiles[base + 64 * i + lane] = make_uint2(tx, rec[i]);
        return;
      }
    }
  }
}

// Tiles of the list, one at a time per block: the rows [r_lo, r_hi) of
// expert e in column tile ct, all the tile's entries in one pass (at most
// kCap<kDown>).
// Whether the plan's counter block describes the list the kernel is given
// (same length, address, first and last entry).  A plan kept across a change
// of the list would otherwise send the tiles to list positions that hold
// other entries.
__device__ __forceinline__ bool plan_matches(const uint32_t* __restrict__ hdr, const MaskedArgs& A) {
  const uint64_t p = uint64_t(reinterpret_cast<uintptr_t>(A.idx));
  return hdr[kHdrNnz] == uint32_t(uint64_t(A.nnz)) && hdr[kHdrNnz + 1] == uint32_t(uint64_t(A.nnz) >> 32) &&
         hdr[kHdrPtr] == uint32_t(p) && hdr[kHdrPtr + 1] == uint32_t(p >> 32) &&
         hdr[kHdrFirst] == A.idx[0] && hdr[kHdrLast] == A.idx[A.nnz - 1];
}

template <bool kDown>
__global__ __launch_bounds__(kThreads) void masked_dw_sddmm_kernel(MaskedArgs A, const uint2* __restrict__ tiles,
                                                                  const int* __restrict__ counters,
                                                                  int tensor) {
  __shared__ __attribute__((aligned(16))) unsigned char lds_l[2][kLsBytes<kDown>];
  __shared__ __attribute__((aligned(16))) unsigned char lds_r[2][kRsBytes];
  __shared__ int rowpre[kMaxRows<kDown> + 1];
  __shared__ uint32_t rstart[kMaxRows<kDown>];
  __shared__ __attribute__((aligned(16))) int tok_tab[kTokTab<kDown>];
  __shared__ __attribute__((aligned(16))) int slot_tab[kTokTab<kDown>];
  __shared__ __attribute__((aligned(16))) float w_tab[kDown ? kTokTab<kDown> : 4];

  constexpr int kE = kEnt<kDown>;
  const int tid = threadIdx.x;
  if (!plan_matches(reinterpret_cast<const uint32_t*>(counters), A)) {
    // a plan of another list: no gradient is written, and the non-finite
    // count the optimiser checks is raised so that the step is skipped
    if (blockIdx.x == 0 && tid == 0 && A.nonfinite) atomicAdd(A.nonfinite, 1);
    return;
  }
  const int nt = counters[kHdrTiles + tensor];
  // persistent: block b takes tiles x(b), x(b) + G, ... (x: the XCD-aware
  // order, so that a group's consecutive tiles share an XCD's L2)
  for (int L = xcd_remap_blocks(blockIdx.x, gridDim.x); L < nt; L += gridDim.x) {
  __syncthreads();  // the previous tile's tables are no longer read
  const uint2 td = tiles[L];
  const int e = int(td.x & 0xffffu), ct = int(td.x >> 16);
  const int r_lo = int(td.y & 0xffffu), r_hi = int(td.y >> 16), nr = r_hi - r_lo;
  // rows are staged from r_al (16-byte aligned loads); an entry of local
  // row i (from r_lo) sits at staged row i + shift
  const int r_al = r_lo & ~7, shift = r_lo - r_al;
  const int c0 = ct * A.CB, c1 = min(A.C, c0 + A.CB), ncol = c1 - c0;
  const int lane = tid & 63;

  // entries of this tile: per row r, the plan segment (e, r, ct)
  const int64_t q_r0 = A.qbase + (int64_t(e) * A.R + r_lo) * A.nct + ct;
  const uint32_t nnz32 = uint32_t(A.nnz);  // list positions are below 2^32
  int nent;
  uint32_t rs0;  // list position of the tile's first entry
  if (A.nct == 1) {
    // one column tile: the tile's entries are one run of the list (rows
    // r_lo..r_hi-1 are consecutive segments) and an entry's row follows
    // from its flat index, so no per-row table is built
    rs0 = min(A.seg[q_r0], nnz32);
    nent = int(max(min(A.seg[q_r0 + nr], nnz32), rs0) - rs0);
  } else {
    for (int r = tid; r < nr; r += kThreads) {
      const int64_t q = q_r0 + int64_t(r) * A.nct;
      const uint32_t s0 = min(A.seg[q], nnz32);
      rstart[r] = s0;
      rowpre[r + 1] = int(max(min(A.seg[q + 1], nnz32), s0) - s0);
    }
    if (tid == 0) rowpre[0] = 0;
    __syncthreads();
    if (tid < 64) {  // inclusive scan of rowpre[1..nr] by wave 0
      int carry = 0;
      for (int b = 0; b < nr; b += 64) {
        int v = (b + lane < nr) ? rowpre[b + lane + 1] : 0;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int u = __shfl_up(v, d, 64);
          if (lane >= d) v += u;
        }
        if (b + lane < nr) rowpre[b + lane + 1] = v + carry;
        carry += __shfl(v, 63, 64);
      }
    }
    __syncthreads();
    nent = rowpre[nr];
    rs0 = rstart[0];
  }
  if (nent == 0) continue;  // uniform

  const int off = A.offsets[e];
  const int ne = A.offsets[e + 1] - off;
  const int nblk_r = (ncol + 7) >> 3, nblk_l = (nr + shift + 7) >> 3;

  for (int q0 = 0, per = 0; q0 < nent; q0 += kThreads * per) {
    // this pass: per entries for every thread (spread evenly, at most kE).
    // Wave w takes the 64*per entries from q0 + 64*per*w, lane-interleaved:
    // lane l's i-th entry is that base + 64 i + l, so the lanes of a wave
    // read neighbouring entries at once (mostly one row: one broadcast LDS
    // read of the row operand; coalesced list loads and gradient stores).
    per = min(kE, (nent - q0 + kThreads - 1) / kThreads);
    uint32_t offs[kE];  // LDS byte offsets of the entry's row (high half) and column (low half)
    uint32_t opos[kE];  // list position of the entry, ~0 when unused
    float acc[kE];
    {
      const int qw = q0 + (tid >> 6) * 64 * per + lane;
      uint32_t rows[kE], val[kE];
      const int64_t rb0 = A.base + (int64_t(e) * A.R + r_lo) * A.C + c0;
      if (A.nct == 1) {
        // one column tile: the tile's rows are one run of the list from
        // rs0, and an entry's row follows from its flat index
        // (offset x < nr*C < 2^24 from the tile's first row; the float
        // quotient is off by at most one and corrected exactly)
#pragma unroll
        for (int i = 0; i < kE; ++i) {
          const int qi = qw + 64 * i;
          const bool used = i < per && qi < nent;
          opos[i] = used ? rs0 + uint32_t(qi) : 0xffffffffu;
          val[i] = used ? opos[i] : rs0;
        }
#pragma unroll
        for (int i = 0; i < kE; ++i) val[i] = A.idx[val[i]];
        const uint32_t C = uint32_t(A.C);
        const float invC = 1.0f / float(A.C);
#pragma unroll
        for (int i = 0; i < kE; ++i) {
          const uint32_t x = opos[i] != 0xffffffffu ? uint32_t(int64_t(val[i]) - rb0) : 0u;
          uint32_t rr = uint32_t(float(x) * invC);
          if (rr * C > x) --rr; else if ((rr + 1) * C <= x) ++rr;
          rows[i] = rr;
        }
      } else {
        // rows by binary search over the row prefix (the lane's entries
        // ascend, so each search starts at the previous row), list
        // positions, then every list load at once
        int r = 0;
#pragma unroll
        for (int i = 0; i < kE; ++i) {
          const int qi = qw + 64 * i;
          opos[i] = 0xffffffffu;
          rows[i] = 0;
          val[i] = rs0;
          if (i < per && qi < nent) {
            int hi = nr - 1;
            while (r < hi) {  // last row with rowpre <= qi
              const int mid = (r + hi + 1) >> 1;
              if (rowpre[mid] <= qi) r = mid; else hi = mid - 1;
            }
            rows[i] = uint32_t(r);
            opos[i] = rstart[r] + uint32_t(qi - rowpre[r]);
            val[i] = opos[i];
          }
        }
#pragma unroll
        for (int i = 0; i < kE; ++i) val[i] = A.idx[val[i]];
      }
#pragma unroll
      for (int i = 0; i < kE; ++i) {
        acc[i] = 0.f;
        offs[i] = 0;  // unused: row 0, column 0
        if (opos[i] != 0xffffffffu) {
          const uint32_t col = uint32_t(int64_t(val[i]) - (rb0 + int64_t(rows[i]) * A.C));
          const uint32_t lrow = rows[i] + uint32_t(shift);
          const uint32_t loff = sw16(lrow) * 16;
          offs[i] = (loff << 16) | (sw16(col) * 16);
        }
      }
      // Bank-aware lane order: the 16 lanes of a quarter-wave read LDS
      // together, and their column reads conflict when two fall in one
      // 16-byte bank group (random columns meet ~3 per group).  For each i
      // the wave sorts its 64 entries by the column's bank group (a
      // counting sort on the group's 4 bits, by ballots) and deals the
      // sorted order across the quarters (sorted position p goes to lane
      // 16 (p mod 4) + p / 4), so equal groups land in different quarters;
      // rows stay within the 64 neighbouring entries, mostly one broadcast
      // row per quarter.  Results do not depend on the order.
      const uint64_t below = (uint64_t(1) << lane) - 1;
#pragma unroll
      for (int i = 0; i < kE; ++i) {
        if (i >= per) break;  // uniform
        const uint32_t g = ((offs[i] & 0xffffu) >> 4) & 15u;
        uint64_t eq = ~uint64_t(0);
        uint32_t less = 0;
#pragma unroll
        for (int b = 3; b >= 0; --b) {
          const uint64_t B = __ballot((g >> b) & 1u);
          if ((g >> b) & 1u) {
            less += uint32_t(__popcll(eq & ~B));
            eq &= B;
          } else {
            eq &= ~B;
          }
        }
        const uint32_t p = less + uint32_t(__popcll(eq & below));
        const int dst = int(((p & 3u) << 4) | (p >> 2));
        offs[i] = uint32_t(__builtin_amdgcn_ds_permute(dst << 2, int(offs[i])));
        opos[i] = uint32_t(__builtin_amdgcn_ds_permute(dst << 2, int(opos[i])));
      }
    }
    // Products over one staged chunk, entries in branch-free groups of 4 (an
    // unused entry reads row 0 and column 0): bf16 dot2 with fp32
    // accumulation.  The LDS reads of group g+1 are issued before the
    // products of group g and no further ahead (a scheduling barrier after
    // each group), which keeps the operands of two groups in registers.
    constexpr int kG = 4;
    constexpr int kNG = kE / kG;
    struct Ops {
      uint4 rv[kG];
      uint4 lv[kG];
    };
    auto load_group = [&](auto G_, const unsigned char* Ls, const unsigned char* Rs, Ops& o) {
      constexpr int g0 = kG * decltype(G_)::value;
#pragma unroll
      for (int k = 0; k < kG; ++k) {
        const uint32_t lo = offs[g0 + k] >> 16, ro = offs[g0 + k] & 0xffffu;
        o.rv[k] = *reinterpret_cast<const uint4*>(Rs + ro);
        o.lv[k] = *reinterpret_cast<const uint4*>(Ls + lo);
      }
    };
    auto math_group = [&](auto G_, const Ops& o) {
      constexpr int g0 = kG * decltype(G_)::value;
#pragma unroll
      for (int k = 0; k < kG; ++k) {
        float a = acc[g0 + k];
        const uint4 rv = o.rv[k], lb = o.lv[k];
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lb.x),
                                            __builtin_bit_cast(bf16x2_t, rv.x), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lb.y),
                                            __builtin_bit_cast(bf16x2_t, rv.y), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lb.z),
                                            __builtin_bit_cast(bf16x2_t, rv.z), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lb.w),
                                            __builtin_bit_cast(bf16x2_t, rv.w), a, false);
        acc[g0 + k] = a;
      }
    };
    auto compute = [&](const unsigned char* Ls, const unsigned char* Rs) {
      Ops o[2];
      load_group(std::integral_constant<int, 0>{}, Ls, Rs, o[0]);  // per >= 1
      static_for<kNG>([&](auto G_) {
        constexpr int g = decltype(G_)::value;
        if (kG * g >= per) return;
        if constexpr (g + 1 < kNG) {
          if (kG * (g + 1) < per) load_group(std::integral_constant<int, g + 1>{}, Ls, Rs, o[(g + 1) & 1]);
        }
        math_group(G_, o[g & 1]);
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // stream the expert's slots, a token-table window at a time
    StageRole role;
    {
      const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
      const int ncw = (nblk_r + 63) >> 6;
      role.col = wv < ncw;
      const int nb = role.col ? nblk_r : nblk_l;
      const int b = role.col ? tid : tid - 64 * ncw;
      role.stores = b < nb;
      const int bc = min(b, nb - 1);
      role.ld2 = 2u * uint32_t(role.col ? A.C : A.R);
      role.by_tok = role.col != kDown;
      // operand rows by slot start at the expert's first slot
      const unsigned char* b0 = role.col ? reinterpret_cast<const unsigned char*>(A.Rm + c0)
                                         : reinterpret_cast<const unsigned char*>(A.L + r_al);
      role.base = role.by_tok ? b0 : b0 + int64_t(off) * role.ld2;
      role.lane_off = 16u * uint32_t(bc);
      role.unit = 8u * uint32_t(bc);
    }
    for (int w0 = 0; w0 < ne; w0 += kTokTab<kDown>) {
      const int wn = min(kTokTab<kDown>, ne - w0);
      __syncthreads();  // previous window's tables and buffers consumed
      // row tables: the slot's token, and its slot row (from the window's
      // first), padded to a whole chunk with valid rows
      for (int p = tid; p < wn; p += kThreads) {
        const int sid = A.perm[off + w0 + p];
        tok_tab[p] = sid / A.K;
        slot_tab[p] = w0 + p;
        if (kDown) w_tab[p] = A.topk_w[sid];
      }
      if (tid < kSlots && wn + tid < ((wn + kSlots - 1) & ~(kSlots - 1))) {
        tok_tab[wn + tid] = 0;
        slot_tab[wn + tid] = w0 + wn - 1;
        if (kDown) w_tab[wn + tid] = 0.f;
      }
      __syncthreads();
      const int nch = (wn + kSlots - 1) / kSlots;
      // chunk c is multiplied from buffer c & 1.  Every thread holds the
      // loads of kPre chunks in registers (chunk m in set m % kPre): while
      // chunk c is multiplied the staging threads write chunk c+1 into the
      // other buffer, and every thread reuses its registers to load chunk
      // c+1+kPre, so every load has kPre chunk steps to arrive.  Loads are
      // unconditional (chunks past the last reload it), and the chunk loop
      // runs a whole number of kPre steps (the steps past the last chunk
      // store what no product reads and multiply nothing), so the waits
      // before a store count exactly the chunks in flight.
      constexpr int kP = kPre<kDown>;
      StageRegs sr[kP];
      stage_fetch<kDown>(role, 0, tok_tab, slot_tab, w_tab, sr[0]);
      if (role.stores) stage_store<kDown>(role, sr[0], 0, wn, lds_l[0], lds_r[0]);
      static_for<kP>([&](auto J) {
        constexpr int m = decltype(J)::value + 1;
        stage_fetch<kDown>(role, min(m, nch - 1) * kSlots, tok_tab, slot_tab, w_tab, sr[m % kP]);
      });
      for (int cb = 0; cb < nch; cb += kP) {
        static_for<kP>([&](auto J) {
          constexpr int j = decltype(J)::value;
          constexpr int s = (j + 1) % kP;  // set of chunk c + 1 (cb is a multiple of kP)
          const int c = cb + j;
          __syncthreads();  // buffer c & 1 written; buffer (c+1) & 1 no longer read
          if (role.stores)
            stage_store<kDown>(role, sr[s], (c + 1) * kSlots, wn, lds_l[(c + 1) & 1],
                               lds_r[(c + 1) & 1]);
          stage_fetch<kDown>(role, min(c + 1 + kP, nch - 1) * kSlots, tok_tab, slot_tab, w_tab,
                             sr[s]);
          if (c < nch) compute(lds_l[c & 1], lds_r[c & 1]);  // uniform
        });
      }
    }
    // write this thread's entries
    {
      int nbad = 0;
#pragma unroll
      for (int i = 0; i < kE; ++i) {
        if (opos[i] == 0xffffffffu) continue;
        A.dW[opos[i]] = acc[i];
        nbad += !finite_f(acc[i]);
      }
      if (A.nonfinite && nbad) atomicAdd(A.nonfinite, nbad);
    }
  }
  }
}

// Column tiling of one tensor: balanced tiles of at most kMaxCB columns
// (a multiple of 8); depends on the shape only.
static void col_tiles(int C, int& CB, int& nct) {
  nct = int(ceil_div(C, kMaxCB));
  CB = int(ceil_div(ceil_div(C, nct), 8) * 8);
  nct = int(ceil_div(C, CB));
}

// Upper bound on the tiles of one tensor (R rows, C columns per expert)
// holding at most nnz entries, for row limit RB.  A group of n entries has
// at most R/RB row cuts, 2n/cap + 1 entry cuts (two consecutive entry-cut
// tiles hold more than cap entries together) and at most one quantile cut
// per multiple of n/nt, nt <= ceil(R/RB) + ceil(n/cap) of them, so at most
// 2 ceil(R/RB) + 3 ceil(n/cap) + 2 tiles; summed over the groups with
// sum ceil(n/cap) <= nnz/cap + groups; a target below cap adds fewer than
// cus <= kMaxCUs (the quantile tiles fit the rounds that full tiles take).
static int64_t tile_bound(const usaf_moe_shape& s, int R, int C, int64_t nnz, int RB, int cap) {
  int CB, nct;
  col_tiles(C, CB, nct);
  return int64_t(s.E) * nct * (2 * ceil_div(R, RB) + 5) + 3 * ceil_div(nnz, cap) + kMaxCUs;
}

// Plan layout (bytes): segment starts [Q+1] u32 (256-aligned), 256 bytes of
// counters (the two tensors' tile counts, then their entry targets), the
// gate_up tile list, the down tile list, the groups' entry counts.
struct PlanLayout {
  SegLayout Lq;
  int RB0, RB1;
  int64_t b0, b1;   // tile bounds for this nnz (block counts)
  size_t counters, tiles0, tiles1, ngrp, total;
};

static PlanLayout plan_layout(const usaf_moe_shape& s, int64_t nnz) {
  PlanLayout P;
  SegLayout& Lq = P.Lq;
  Lq.E = s.E;
  Lq.R0 = 2 * s.I; Lq.C0 = s.H;
  Lq.R1 = s.H; Lq.C1 = s.I;
  col_tiles(Lq.C0, Lq.CB0, Lq.nct0);
  col_tiles(Lq.C1, Lq.CB1, Lq.nct1);
  Lq.ngu = int64_t(s.E) * 2 * s.I * s.H;
  Lq.q1 = int64_t(s.E) * Lq.R0 * Lq.nct0;
  Lq.Q = Lq.q1 + int64_t(s.E) * Lq.R1 * Lq.nct1;
  const int64_t N = n_weights(s);
  P.RB0 = std::min(Lq.R0, row_limit<false>(Lq.CB0));
  P.RB1 = std::min(Lq.R1, row_limit<true>(Lq.CB1));
  P.b0 = tile_bound(s, Lq.R0, Lq.C0, std::min<int64_t>(nnz, Lq.ngu), P.RB0, kCap<false>);
  P.b1 = tile_bound(s, Lq.R1, Lq.C1, std::min<int64_t>(nnz, N - Lq.ngu), P.RB1, kCap<true>);
  P.counters = ((size_t(Lq.Q + 1) * 4 + 255) / 256) * 256;
  P.tiles0 = P.counters + 256;
  P.tiles1 = P.tiles0 + 8 * size_t(tile_bound(s, Lq.R0, Lq.C0, Lq.ngu, P.RB0, kCap<false>));
  P.ngrp = P.tiles1 + ((8 * size_t(tile_bound(s, Lq.R1, Lq.C1, N - Lq.ngu, P.RB1, kCap<true>)) + 255) / 256) * 256;
  P.total = P.ngrp + ((size_t(s.E) * (Lq.nct0 + Lq.nct1) * 4 + 255) / 256) * 256;
  return P;
}

int64_t masked_plan_bytes(const usaf_moe_shape& s) { return int64_t(plan_layout(s, 1).total); }

// The gradient kernels address an operand row by a 24-bit row index times
// the row pitch, as a 32-bit byte offset from the tile's base (token rows
// from the tensor's start, slot rows from the expert's first slot): the
// token-row tensors (X, dY: T x H) and the slot-row tensors (dGU: S x 2I)
// must stay below 4 GiB, and T, S below 2^24.
bool masked_dw_fits(const usaf_moe_shape& s) {
  const int64_t S = int64_t(s.T) * s.K, lim = int64_t(1) << 32;
  return S < (int64_t(1) << 24) && int64_t(s.T) * s.H * 2 < lim && S * 2 * s.I * 2 < lim;
}

// The plan of a list: segment starts, then each tensor's tiles.  Depends on
// idx and the shape only, so one plan serves every step until the list
// changes.
usaf_status masked_plan_bf16(const usaf_moe_shape& s, const uint32_t* idx, int64_t nnz, void* plan,
                             hipStream_t st) {
  if (nnz == 0) return USAF_OK;
  const PlanLayout P = plan_layout(s, nnz);
  if (P.b0 >= (int64_t(1) << 31) || P.b1 >= (int64_t(1) << 31)) return USAF_ERR_UNSUPPORTED;
  unsigned char* base = static_cast<unsigned char*>(plan);
  uint32_t* seg = reinterpret_cast<uint32_t*>(base);
  int* counters = reinterpret_cast<int*>(base + P.counters);
  int* ng = reinterpret_cast<int*>(base + P.ngrp);
  const int ngroups = s.E * (P.Lq.nct0 + P.Lq.nct1);  // <= Q + 1 threads
  hipLaunchKernelGGL(masked_plan_kernel, dim3(unsigned(ceil_div(P.Lq.Q + 1, 256))), dim3(256), 0, st,
                     idx, nnz, P.Lq, seg, counters, ng, ngroups);
  USAF_LAUNCH_CHECK();
  const int cus = std::min(device_cus(), kMaxCUs);
  for (int tensor = 0; tensor < 2; ++tensor) {
    const int nct = tensor == 0 ? P.Lq.nct0 : P.Lq.nct1;
    const int groups = s.E * nct;
    const int64_t qb = tensor == 0 ? int64_t(0) : P.Lq.q1;
    const int R = tensor == 0 ? P.Lq.R0 : P.Lq.R1, RB = tensor == 0 ? P.RB0 : P.RB1;
    const int cap = tensor == 0 ? kCap<false> : kCap<true>;
    int* ngt = ng + (tensor == 0 ? 0 : s.E * P.Lq.nct0);
    // about 2048 rows per block (at most 16 blocks per group)
    const int nsub = nct == 1 ? 1 : std::min(16, int(ceil_div(R, 2048)));
    hipLaunchKernelGGL(masked_group_totals_kernel, dim3(unsigned(groups), unsigned(nsub)), dim3(256), 0, st,
                       seg, qb, s.E, R, nct, ngt);
    USAF_LAUNCH_CHECK();
    hipLaunchKernelGGL(masked_target_kernel, dim3(1), dim3(256), 0, st, ngt, groups, R, RB, cap, cus,
                       counters + kHdrTarget + tensor);
    USAF_LAUNCH_CHECK();
    hipLaunchKernelGGL(masked_tiles_kernel, dim3(unsigned(ceil_div(groups, 4))), dim3(256), 0, st,
                       seg, qb, s.E, R, nct, RB, cap, ngt, counters + kHdrTarget + tensor,
                       reinterpret_cast<uint2*>(base + (tensor == 0 ? P.tiles0 : P.tiles1)),
                       counters + kHdrTiles + tensor);
    USAF_LAUNCH_CHECK();
  }
  return USAF_OK;
}

usaf_status masked_dw_bf16(const usaf_moe_shape& s, const uint32_t* idx, int64_t nnz,
                           const bf16_t* X, const bf16_t* dY, const bf16_t* dgu, const bf16_t* a,
                           const float* topk_w, const int32_t* offsets, const int32_t* perm,
                           float* dW, int32_t* nonfinite, const void* plan, void* ws_plan,
                           hipStream_t st) {
  if (nnz == 0) return USAF_OK;
  if (!masked_dw_fits(s)) return USAF_ERR_UNSUPPORTED;
  const PlanLayout P = plan_layout(s, nnz);
  if (P.b0 >= (int64_t(1) << 31) || P.b1 >= (int64_t(1) << 31)) return USAF_ERR_UNSUPPORTED;
  timer_begin(USAF_K_MASKED_DW, st);
  if (!plan) {  // no plan kept by the caller: build one in the workspace
    USAF_TRY(masked_plan_bf16(s, idx, nnz, ws_plan, st));
    plan = ws_plan;
  }
  const unsigned char* base = static_cast<const unsigned char*>(plan);
  const uint32_t* seg = reinterpret_cast<const uint32_t*>(base);
  const int* counters = reinterpret_cast<const int*>(base + P.counters);
  for (int tensor = 0; tensor < 2; ++tensor) {
    MaskedArgs A;
    A.idx = idx; A.nnz = nnz;
    A.offsets = offsets; A.perm = perm; A.topk_w = topk_w; A.K = s.K; A.E = s.E;
    A.dW = dW; A.nonfinite = nonfinite; A.seg = seg;
    if (tensor == 0) {
      A.L = dgu; A.Rm = X; A.R = P.Lq.R0; A.C = P.Lq.C0; A.base = 0;
      A.CB = P.Lq.CB0; A.nct = P.Lq.nct0; A.qbase = 0;
    } else {
      A.L = dY; A.Rm = a; A.R = P.Lq.R1; A.C = P.Lq.C1; A.base = P.Lq.ngu;
      A.CB = P.Lq.CB1; A.nct = P.Lq.nct1; A.qbase = P.Lq.q1;
    }
    const uint2* tl = reinterpret_cast<const uint2*>(base + (tensor == 0 ? P.tiles0 : P.tiles1));
    const int64_t bound = tensor == 0 ? P.b0 : P.b1;
    const int64_t blocks = (std::min<int64_t>(bound, device_cus()) + 7) / 8 * 8;
    if (tensor == 0)
      hipLaunchKernelGGL(masked_dw_sddmm_kernel<false>, dim3(unsigned(blocks)), dim3(kThreads), 0, st, A, tl,
                         counters, 0);
    else
      hipLaunchKernelGGL(masked_dw_sddmm_kernel<true>, dim3(unsigned(blocks)), dim3(kThreads), 0, st, A, tl,
                         counters, 1);
    USAF_LAUNCH_CHECK();
  }
  timer_end(USAF_K_MASKED_DW, st);
  return USAF_OK;
}

}  // namespace usaf
