// Masked expert-weight gradient for bf16 layers: the gradient only at the
// selected ~0.5% of expert weights (usaf README intro and A100 per-operation
// table: gradients and optimiser state exist only for the selected subset).
//
// For one (tensor, expert) the selected entries are a sampled subset of
//   gate_up: G[r, c] = sum_p dGU[p, r] * X[tok(p), c]          (r < 2I, c < H)
//   down:    G[r, c] = sum_p (w_p dY[tok(p), r]) * a[p, c]     (r < H,  c < I)
// over the expert's slots p.  A block owns a (row tile x column tile) of one
// expert and streams the expert's slots through LDS in chunks of 8, staged
// slot-contiguous ([row][8 slots]) by 8x8 register transposes, so that one
// 16-byte LDS read yields an entry's 8 slot values.  Each thread accumulates
// a contiguous run of the block's entries (consecutive entries mostly share
// a row, whose staged values stay in registers).  gate_up uses bf16 dot2
// (fp32 accumulate); down stages w_p * dY in fp32 and uses fp32 FMA.
#include <cmath>

#include "common.hpp"
#include "moe_internal.hpp"
#include "timing.hpp"

namespace usaf {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kSlots = 8;        // slots per staged chunk
constexpr int kThreads = 512;    // 8 waves per block, one block per CU
constexpr int kMaxEnt = 24;      // entries per thread per pass
constexpr int kMaxRB = 1024;     // max rows per block
constexpr int kMaxCB = 2048;     // max columns per block (kMaxCB/8 + kMaxRB/8 <= kThreads)
constexpr int kTokTab = 2048;    // slots per token-table window
constexpr int kLsBytes = kMaxRB * kSlots * 4;
constexpr int kRsBytes = kMaxCB * kSlots * 2;

struct MaskedArgs {
  const uint32_t* idx; int64_t nnz;
  const bf16_t* L;        // gate_up: dGU [S, 2I]; down: dY [T, H]
  const bf16_t* Rm;       // gate_up: X [T, H];    down: a [S, I]
  const int32_t* offsets; const int32_t* perm; const float* topk_w;
  int K;
  int R, C;               // rows / columns of the per-expert gradient
  int RB, CB, nrt, nct;   // tiling
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

__global__ __launch_bounds__(256) void masked_plan_kernel(const uint32_t* __restrict__ idx,
                                                          int64_t nnz, SegLayout Lq,
                                                          uint32_t* __restrict__ seg) {
  const int64_t q = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
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
// 8 slot values each (one per element).
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint4 a4 = in[2 * d], b4 = in[2 * d + 1];
      const uint32_t a = (j < 2) ? a4.x : (j < 4) ? a4.y : (j < 6) ? a4.z : a4.w;
      const uint32_t b = (j < 2) ? b4.x : (j < 4) ? b4.y : (j < 6) ? b4.z : b4.w;
      w[d] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    out[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// LDS slot swizzles.  Staging writes 16-byte units for consecutive lanes at
// a 128-byte stride (8 units apart); XOR-ing bits of the unit index into its
// low 3 bits spreads those lanes over all 16 bank groups of a 256-byte window.
// 32-byte units (fp32 staging) are 8 apart in the same way.
__device__ __forceinline__ uint32_t sw16(uint32_t u) { return u ^ ((u >> 4) & 7u); }
__device__ __forceinline__ uint32_t sw32(uint32_t u) { return u ^ ((u >> 3) & 7u); }

// One staging block: 8 slots x 8 consecutive elements of one operand row.
struct StageRegs {
  uint4 v[kSlots];
  float w[kSlots];
};

template <bool kDown>
__device__ __forceinline__ void stage_fetch(const MaskedArgs& A, int b, int nblk_r, int p0,
                                            int pend, int slot0, int r_lo, int c0,
                                            const int* tok_tab, const float* w_tab,
                                            StageRegs& sr) {
  // p0 indexes the token table window; slot0 + p is the expert-major slot row
  const bool isR = b < nblk_r;
  const int j0 = (isR ? b : b - nblk_r) * 8;
#pragma unroll
  for (int t = 0; t < kSlots; ++t) {
    const int p = p0 + t;
    sr.v[t] = make_uint4(0, 0, 0, 0);
    sr.w[t] = 0.f;
    if (p < pend) {
      const bf16_t* src;
      if (isR) {
        src = kDown ? A.Rm + int64_t(slot0 + p) * A.C + c0
                    : A.Rm + int64_t(tok_tab[p]) * A.C + c0;
      } else {
        src = kDown ? A.L + int64_t(tok_tab[p]) * A.R + r_lo
                    : A.L + int64_t(slot0 + p) * A.R + r_lo;
        if (kDown) sr.w[t] = w_tab[p];
      }
      sr.v[t] = *reinterpret_cast<const uint4*>(src + j0);
    }
  }
}

template <bool kDown>
__device__ __forceinline__ void stage_store(int b, int nblk_r, const StageRegs& sr,
                                            unsigned char* lds_l, unsigned char* lds_r) {
  const bool isR = b < nblk_r;
  const int j0 = (isR ? b : b - nblk_r) * 8;
  if (isR || !kDown) {
    uint4 out[8];
    transpose8x8(sr.v, out);
    unsigned char* dst = isR ? lds_r : lds_l;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<uint4*>(dst + size_t(sw16(uint32_t(j0 + j))) * 16) = out[j];
  } else {
    // down: w_p * dY in fp32, [row][8 slots]
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v[8];
#pragma unroll
      for (int t = 0; t < kSlots; ++t) {
        const uint32_t wd = (j < 2) ? sr.v[t].x : (j < 4) ? sr.v[t].y : (j < 6) ? sr.v[t].z : sr.v[t].w;
        v[t] = sr.w[t] * ((j & 1) ? bfhi(wd) : bflo(wd));
      }
      float4* dst = reinterpret_cast<float4*>(lds_l + size_t(sw32(uint32_t(j0 + j))) * 32);
      dst[0] = make_float4(v[0], v[1], v[2], v[3]);
      dst[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

template <bool kDown>
__global__ __launch_bounds__(kThreads) void masked_dw_sddmm_kernel(MaskedArgs A) {
  __shared__ __attribute__((aligned(16))) unsigned char lds_l[kLsBytes];
  __shared__ __attribute__((aligned(16))) unsigned char lds_r[kRsBytes];
  __shared__ int rowpre[kMaxRB + 1];
  __shared__ uint32_t rstart[kMaxRB];
  __shared__ int tok_tab[kTokTab];
  __shared__ float w_tab[kDown ? kTokTab : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int per_e = A.nrt * A.nct;
  const int L = xcd_remap_blocks(blockIdx.x, gridDim.x);
  const int e = L / per_e;
  if (e >= A.E) return;
  const int rem = L - e * per_e;
  const int rt = rem / A.nct, ct = rem - rt * A.nct;
  const int r_lo = rt * A.RB, r_hi = min(A.R, r_lo + A.RB), nr = r_hi - r_lo;
  const int c0 = ct * A.CB, c1 = min(A.C, c0 + A.CB), ncol = c1 - c0;
  const int64_t ebase = A.base + int64_t(e) * A.R * A.C;
  (void)ebase;

  // entries of this tile: per row r, the plan segment (e, r, ct)
  const int64_t q_r0 = A.qbase + (int64_t(e) * A.R + r_lo) * A.nct + ct;
  for (int r = tid; r < nr; r += kThreads) {
    const int64_t q = q_r0 + int64_t(r) * A.nct;
    const uint32_t s0 = A.seg[q];
    rstart[r] = s0;
    rowpre[r + 1] = int(A.seg[q + 1] - s0);
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
  const int nent = rowpre[nr];
  if (nent == 0) return;  // nothing selected in this tile (uniform)

  const int off = A.offsets[e];
  const int ne = A.offsets[e + 1] - off;
  const int nblk_r = (ncol + 7) >> 3, nblk_l = (nr + 7) >> 3;

  for (int q0 = 0, per = 0; q0 < nent; q0 += kThreads * per) {
    // this pass: per entries for every thread (spread evenly, at most
    // kMaxEnt), thread tid taking q0 + tid*per + i
    per = min(kMaxEnt, (nent - q0 + kThreads - 1) / kThreads);
    uint32_t coord[kMaxEnt];  // (row - r_lo) << 16 | (col - c0), or ~0 when unused
    float acc[kMaxEnt];
    {
      const int q = q0 + tid * per;
      // row of entry q: last r with rowpre[r] <= q
      int lo = 0, hi = nr;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (rowpre[mid] <= q) lo = mid; else hi = mid - 1;
      }
      int r = lo;
#pragma unroll
      for (int i = 0; i < kMaxEnt; ++i) {
        acc[i] = 0.f;
        coord[i] = 0xffffffffu;
        const int qi = q + i;
        if (i < per && qi < nent) {
          while (rowpre[r + 1] <= qi) ++r;
          const int64_t rb = A.base + (int64_t(e) * A.R + r_lo + r) * A.C;
          const int c = int(int64_t(A.idx[rstart[r] + (qi - rowpre[r])]) - rb);
          coord[i] = (uint32_t(r) << 16) | uint32_t(c - c0);
        }
      }
    }
    // stream the expert's slots, a token-table window at a time, in chunks
    // of kSlots staged through LDS
    const bool stager = tid < nblk_r + nblk_l;  // <= kThreads staging blocks: one per thread
    for (int w0 = 0; w0 < ne; w0 += kTokTab) {
      const int wn = min(kTokTab, ne - w0);
      __syncthreads();  // previous window fully consumed
      for (int p = tid; p < wn; p += kThreads) {
        const int sid = A.perm[off + w0 + p];
        tok_tab[p] = sid / A.K;
        if (kDown) w_tab[p] = A.topk_w[sid];
      }
      __syncthreads();
      // chunk c+1 is fetched into registers while chunk c is consumed
      auto compute = [&]() {
        uint32_t prow = 0xffffffffu;
        uint4 lb16 = make_uint4(0, 0, 0, 0);
        float lf[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) lf[t] = 0.f;
#pragma unroll
        for (int i = 0; i < kMaxEnt; ++i) {
          const uint32_t cd = coord[i];
          if (cd == 0xffffffffu) continue;
          const uint32_t lr = cd >> 16, lc = cd & 0xffffu;
          if (lr != prow) {
            prow = lr;
            if (kDown) {
              const float4* src = reinterpret_cast<const float4*>(lds_l + size_t(sw32(lr)) * 32);
              const float4 x = src[0], y = src[1];
              lf[0] = x.x; lf[1] = x.y; lf[2] = x.z; lf[3] = x.w;
              lf[4] = y.x; lf[5] = y.y; lf[6] = y.z; lf[7] = y.w;
            } else {
              lb16 = *reinterpret_cast<const uint4*>(lds_l + size_t(sw16(lr)) * 16);
            }
          }
          const uint4 rv = *reinterpret_cast<const uint4*>(lds_r + size_t(sw16(lc)) * 16);
          float a = acc[i];
          if (kDown) {
            a = fmaf(lf[0], bflo(rv.x), a); a = fmaf(lf[1], bfhi(rv.x), a);
            a = fmaf(lf[2], bflo(rv.y), a); a = fmaf(lf[3], bfhi(rv.y), a);
            a = fmaf(lf[4], bflo(rv.z), a); a = fmaf(lf[5], bfhi(rv.z), a);
            a = fmaf(lf[6], bflo(rv.w), a); a = fmaf(lf[7], bfhi(rv.w), a);
          } else {
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lb16.x),
                                                __builtin_bit_cast(bf16x2_t, rv.x), a, false);
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lb16.y),
                                                __builtin_bit_cast(bf16x2_t, rv.y), a, false);
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lb16.z),
                                                __builtin_bit_cast(bf16x2_t, rv.z), a, false);
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lb16.w),
                                                __builtin_bit_cast(bf16x2_t, rv.w), a, false);
          }
          acc[i] = a;
        }
      };
      StageRegs sr;
      if (stager) stage_fetch<kDown>(A, tid, nblk_r, 0, wn, off + w0, r_lo, c0, tok_tab, w_tab, sr);
      for (int p0 = 0; p0 < wn; p0 += kSlots) {
        __syncthreads();  // previous chunk fully consumed
        if (stager) stage_store<kDown>(tid, nblk_r, sr, lds_l, lds_r);
        __syncthreads();
        if (stager && p0 + kSlots < wn)
          stage_fetch<kDown>(A, tid, nblk_r, p0 + kSlots, wn, off + w0, r_lo, c0, tok_tab, w_tab, sr);
        compute();
      }
    }
    // write this thread's entries (contiguous positions in idx within a row run;
    // recompute positions row by row)
    {
      const int q = q0 + tid * per;
      int nbad = 0;
#pragma unroll
      for (int i = 0; i < kMaxEnt; ++i) {
        const uint32_t cd = coord[i];
        if (cd == 0xffffffffu) continue;
        const int ri = int(cd >> 16);
        const float v = acc[i];
        A.dW[int64_t(rstart[ri]) + (q + i - rowpre[ri])] = v;
        nbad += !finite_f(v);
      }
      if (A.nonfinite && nbad) atomicAdd(A.nonfinite, nbad);
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

int64_t masked_plan_segments(const usaf_moe_shape& s) {
  int CB0, nct0, CB1, nct1;
  col_tiles(s.H, CB0, nct0);
  col_tiles(s.I, CB1, nct1);
  return int64_t(s.E) * 2 * s.I * nct0 + int64_t(s.E) * s.H * nct1;
}

// Row tiling: as few row tiles as the LDS staging allows (the expert's slot
// stream is re-read once per tile), but enough that each block's entries
// fit one pass of about 20 per thread.  Returns the tile height (a multiple
// of 8).
static int row_tile(int R, int CB, double density) {
  const double per_row = double(CB) * (density > 0 ? density : 1e-9);
  int64_t nrt = ceil_div(int64_t(R), int64_t(kMaxRB));
  const int64_t by_entries = int64_t(std::ceil(double(R) * per_row / (20.0 * kThreads)));
  if (by_entries > nrt) nrt = by_entries;
  const int64_t rb = ceil_div(ceil_div(int64_t(R), nrt), int64_t(8)) * 8;
  return int(rb < R ? rb : R);
}

usaf_status masked_dw_bf16(const usaf_moe_shape& s, const uint32_t* idx, int64_t nnz,
                           const bf16_t* X, const bf16_t* dY, const bf16_t* dgu, const bf16_t* a,
                           const float* topk_w, const int32_t* offsets, const int32_t* perm,
                           float* dW, int32_t* nonfinite, uint32_t* seg, hipStream_t st) {
  if (nnz == 0) return USAF_OK;
  const double density = double(nnz) / double(n_weights(s));
  SegLayout Lq;
  Lq.E = s.E;
  Lq.R0 = 2 * s.I; Lq.C0 = s.H;
  Lq.R1 = s.H; Lq.C1 = s.I;
  col_tiles(Lq.C0, Lq.CB0, Lq.nct0);
  col_tiles(Lq.C1, Lq.CB1, Lq.nct1);
  Lq.ngu = int64_t(s.E) * 2 * s.I * s.H;
  Lq.q1 = int64_t(s.E) * Lq.R0 * Lq.nct0;
  Lq.Q = Lq.q1 + int64_t(s.E) * Lq.R1 * Lq.nct1;
  timer_begin(USAF_K_MASKED_DW, st);
  hipLaunchKernelGGL(masked_plan_kernel, dim3(unsigned(ceil_div(Lq.Q + 1, 256))), dim3(256), 0, st,
                     idx, nnz, Lq, seg);
  USAF_LAUNCH_CHECK();
  for (int tensor = 0; tensor < 2; ++tensor) {
    MaskedArgs A;
    A.idx = idx; A.nnz = nnz;
    A.offsets = offsets; A.perm = perm; A.topk_w = topk_w; A.K = s.K; A.E = s.E;
    A.dW = dW; A.nonfinite = nonfinite; A.seg = seg;
    if (tensor == 0) {
      A.L = dgu; A.Rm = X; A.R = Lq.R0; A.C = Lq.C0; A.base = 0;
      A.CB = Lq.CB0; A.nct = Lq.nct0; A.qbase = 0;
    } else {
      A.L = dY; A.Rm = a; A.R = Lq.R1; A.C = Lq.C1; A.base = Lq.ngu;
      A.CB = Lq.CB1; A.nct = Lq.nct1; A.qbase = Lq.q1;
    }
    A.RB = row_tile(A.R, A.CB, density);
    A.nrt = int(ceil_div(A.R, A.RB));
    const int64_t blocks = (int64_t(s.E) * A.nrt * A.nct + 7) / 8 * 8;
    if (tensor == 0)
      hipLaunchKernelGGL(masked_dw_sddmm_kernel<false>, dim3(unsigned(blocks)), dim3(kThreads), 0, st, A);
    else
      hipLaunchKernelGGL(masked_dw_sddmm_kernel<true>, dim3(unsigned(blocks)), dim3(kThreads), 0, st, A);
    USAF_LAUNCH_CHECK();
  }
  timer_end(USAF_K_MASKED_DW, st);
  return USAF_OK;
}

}  // namespace usaf
