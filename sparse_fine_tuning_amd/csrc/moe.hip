// MoE layer forward / masked backward for the USAF sparse fine-tuning step.
//
// Method: the usaf README ("tsuyu122/usaf"): tokens are routed to a few
// experts, the router (gating network) is trained densely, and expert weights
// get gradients only at the selected ~0.5% ("how it works" bullets, A100
// per-operation table).  The expert MLP is SwiGLU over the fused gate_up /
// down tensors of the README's quantisation recipe.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "gemm_fma.hpp"
#include "moe_internal.hpp"
#include "timing.hpp"

namespace usaf {

// ---------------------------------------------------------------------------
// Routing
// ---------------------------------------------------------------------------

// Order-preserving map of an fp32 logit to uint32 (larger = better).  NaN
// ranks below -inf; -0 and +0 are equal.
__device__ __forceinline__ uint32_t logit_key(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Maximum over the wave of a 64-bit key, the same in every lane: within each
// row of 16 lanes by DPP (swap neighbours, swap pairs, mirror the halves,
// mirror the row), then over the four rows' first lanes.
template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(v)), kCtrl, 0xf, 0xf, false));
  const uint32_t hi = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(v >> 32)), kCtrl, 0xf, 0xf, false));
  return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), l));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), l));
  return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o = dpp_u64<0xB1>(v);   // quad_perm 1,0,3,2
  v = o > v ? o : v;
  o = dpp_u64<0x4E>(v);            // quad_perm 2,3,0,1
  v = o > v ? o : v;
  o = dpp_u64<0x141>(v);           // row_half_mirror
  v = o > v ? o : v;
  o = dpp_u64<0x140>(v);           // row_mirror
  v = o > v ? o : v;
  const uint64_t r0 = readlane_u64(v, 0), r1 = readlane_u64(v, 16);
  const uint64_t r2 = readlane_u64(v, 32), r3 = readlane_u64(v, 48);
  const uint64_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
}

// One wave per token: K rounds of a wave-wide max over (key, -expert id),
// then softmax over the K chosen logits.  E <= 64 NV, K <= 64: lane l holds
// experts l, l + 64, ... in NV registers.
// With nparts > 1 the logits arrive as split-K partial sums [nparts][T][E];
// they are added in fixed part order and the sums written to `logits`.
template <int NV>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ parts,
                                                         int nparts, float* __restrict__ logits,
                                                         int T, int E, int K,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* lt = logits + int64_t(t) * E;
  uint64_t comp[NV];
  float val[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    val[i] = 0.f;
    if (e < E) {
      float v;
      if (nparts > 1) {
        // the parts' loads are issued together, then added in part order
        float pv[kMaxRouterParts];
#pragma unroll
        for (int q = 0; q < kMaxRouterParts; ++q)
          pv[q] = q < nparts ? parts[(int64_t(q) * T + t) * E + e] : 0.f;
        v = pv[0];
#pragma unroll
        for (int q = 1; q < kMaxRouterParts; ++q)
          if (q < nparts) v += pv[q];
        logits[int64_t(t) * E + e] = v;
      } else {
        v = lt[e];
      }
      val[i] = v;
      comp[i] = (uint64_t(logit_key(v)) << 32) | uint64_t(0xffffffffu - uint32_t(e));
    } else {
      comp[i] = 0ull;
    }
  }
  int my_id = 0;
  float my_l = 0.f;
  for (int j = 0; j < K; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) best = comp[i] > best ? comp[i] : best;
    best = wave_max_u64(best);
    const int e = int(0xffffffffu - uint32_t(best & 0xffffffffull));
    // the owner lane (e % 64) retires the expert; its logit is read from it
    float le = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i == e) {
        comp[i] = 0;
        le = val[i];
      }
    le = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(le), e & 63));
    if (lane == j) {
      my_id = e;
      my_l = le;
    }
  }
  const float l0 = __shfl(my_l, 0, 64);
  float z = lane < K ? expf(my_l - l0) : 0.f;
  float sum = z;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane < K) {
    ids[int64_t(t) * K + lane] = my_id;
    w[int64_t(t) * K + lane] = z / sum;
  }
}

// Stable grouping of slots by expert.  Block e (1024 threads) counts the
// slots routed to experts < e (its offset) and == e, each thread over a
// contiguous run of slots; one block-wide scan of the per-thread matches then
// places every thread's matches in ascending slot order.
__global__ __launch_bounds__(1024) void expert_sort_kernel(const int32_t* __restrict__ ids, int S,
                                                           int E, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ slot_pos) {
  // Block e reads the ids twice, 1024 consecutive slots per round: first
  // counting the slots of lower experts (the group's offset), then placing
  // its own slots in slot order (ballot prefix within a wave, LDS prefix
  // over the 16 waves, a running base across rounds).
  __shared__ int red[16];
  __shared__ int wcnt[16];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int lt = 0;
  for (int s = tid; s < S; s += 1024) lt += ids[s] < e;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lt += __shfl_xor(lt, off, 64);
  if (lane == 0) red[wid] = lt;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) base += red[w];
  if (tid == 0) {
    offsets[e] = base;
    if (e == E - 1) offsets[E] = S;
  }
  const uint64_t below = (uint64_t(1) << lane) - 1;
  for (int s0 = 0; s0 < S; s0 += 1024) {
    const int s = s0 + tid;
    const bool mine = s < S && ids[s] == e;
    const uint64_t m = __ballot(mine);
    if (lane == 0) wcnt[wid] = __popcll(m);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int c = wcnt[w];
      before += w < wid ? c : 0;
      total += c;
    }
    if (mine) {
      const int p = base + before + __popcll(m & below);
      perm[p] = s;
      slot_pos[s] = p;
    }
    base += total;
    __syncthreads();  // wcnt is rewritten next round
  }
}

// The same stable grouping in three launches of constant depth, for S >=
// ceil(S / 1024) * E (the per-chunk counts borrow perm as scratch):
//  1. chunk b of 1024 slots ranks each slot among the chunk's earlier slots
//     of its expert (wave peers from one ballot per id bit, then the counts
//     of the chunk's earlier waves) into slot_pos, and its per-expert counts
//     into perm[b*E + e];
//  2. every chunk derives the expert offsets and its own per-expert base
//     from all chunks' counts, and turns its ranks into final positions;
//  3. perm[slot_pos[s]] = s.
constexpr int kSortChunk = 1024;
__global__ __launch_bounds__(kSortChunk) void expert_rank_kernel(const int32_t* __restrict__ ids,
                                                                 int S, int E, int nbits,
                                                                 int32_t* __restrict__ cnt_out,
                                                                 int32_t* __restrict__ rank) {
  extern __shared__ int wc[];  // [16 waves][E]
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int i = tid; i < 16 * E; i += kSortChunk) wc[i] = 0;
  const int s = blockIdx.x * kSortChunk + tid;
  const bool live = s < S;
  const int id = live ? ids[s] : 0;
  uint64_t peers = __ballot(live);
  if (!live) peers = 0;
  for (int b = 0; b < nbits; ++b) {
    const uint64_t m = __ballot(live && ((id >> b) & 1));
    peers &= ((id >> b) & 1) ? m : ~m;
  }
  const uint64_t below = (uint64_t(1) << lane) - 1;
  const int rw = __popcll(peers & below);
  __syncthreads();  // table zeroed
  if (live && rw == 0) wc[wid * E + id] = __popcll(peers);
  __syncthreads();
  for (int e = tid; e < E; e += kSortChunk) {  // exclusive scan over the waves
    int run = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int c = wc[w * E + e];
      wc[w * E + e] = run;
      run += c;
    }
    cnt_out[int64_t(blockIdx.x) * E + e] = run;
  }
  __syncthreads();
  if (live) rank[s] = wc[wid * E + id] + rw;
}

__global__ __launch_bounds__(kSortChunk) void expert_place_kernel(const int32_t* __restrict__ ids,
                                                                  int S, int E, int nchunk,
                                                                  const int32_t* __restrict__ cnt,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ slot_pos) {
  extern __shared__ int base[];  // [E] then wave sums [16]
  int* wsum = base + E;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  // per expert: total over all chunks and the chunks before this one; the
  // offsets are the exclusive scan of the totals over the experts, taken
  // 1024 experts at a time (E <= 1024)
  int total = 0, before = 0;
  if (tid < E) {
#pragma unroll 8
    for (int b = 0; b < nchunk; ++b) {
      const int c = cnt[int64_t(b) * E + tid];
      total += c;
      before += b < int(blockIdx.x) ? c : 0;
    }
  }
  int incl = total;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < wid; ++w) wbase += wsum[w];
  const int off = wbase + incl - total;
  if (tid < E) {
    base[tid] = off + before;
    if (blockIdx.x == 0) {
      offsets[tid] = off;
      if (tid == E - 1) offsets[E] = S;
    }
  }
  __syncthreads();
  const int s = blockIdx.x * kSortChunk + tid;
  if (s < S) slot_pos[s] = base[ids[s]] + slot_pos[s];
}

__global__ __launch_bounds__(256) void expert_scatter_kernel(const int32_t* __restrict__ slot_pos,
                                                             int S, int32_t* __restrict__ perm) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s < S) perm[slot_pos[s]] = s;
}

// ---------------------------------------------------------------------------
// fp32-FMA GEMM problems (see gemm_fma.hpp for the contract)
// ---------------------------------------------------------------------------

// logits[T, E] = X[T, H] * Wr'[E, H]^T
template <class T>
struct RouterGemm {
  const T* X;
  const float* Wr;
  float* logits;
  int Tn, H, E;
  struct Tile { int m0, mc, n0, nc; };
  __device__ bool get_tile(int bx, int by, int, Tile& t) const {
    t.m0 = bx * 64; t.n0 = by * 64;
    t.mc = min(64, Tn - t.m0); t.nc = min(64, E - t.n0);
    return t.mc > 0 && t.nc > 0;
  }
  __device__ int kbeg(const Tile&) const { return 0; }
  __device__ int kend(const Tile&) const { return H; }
  __device__ void load_a(const Tile& t, int k0, float (*S)[kFmaLd], int tid) const {
    load_kcontig(S, tid, t.mc, k0, H, [&](int r, int k) { return Act<T>::ld(X, int64_t(t.m0 + r) * H + k); });
  }
  __device__ void load_b(const Tile& t, int k0, float (*S)[kFmaLd], int tid) const {
    load_kcontig(S, tid, t.nc, k0, H, [&](int r, int k) { return router_w<T>(Wr, int64_t(t.n0 + r) * H + k); });
  }
  __device__ void epilogue(const Tile& t, float (&acc)[4][4], int tm, int tn) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = tm + 16 * i, n = tn + 16 * j;
        if (m < t.mc && n < t.nc) logits[int64_t(t.m0 + m) * E + t.n0 + n] = acc[i][j];
      }
  }
};

// gate_up forward for expert e: [g | u] = X[tokens of e] * W_gu[e]^T with the
// SwiGLU epilogue.  A tile covers 32 gate features and the same 32 up
// features, so each thread holds matching (g, u) pairs.
template <class T>
struct GateUpFwd {
  const T* X; const T* Wgu; const int32_t* offsets; const int32_t* perm;
  T* gu; T* a;
  int H, E, K, I;
  struct Tile { int e, m0, mc, f0, off; };
  __device__ bool get_tile(int bx, int by, int, Tile& t) const {
    if (!find_mtile(offsets, E, bx, 64, t.e, t.m0, t.mc)) return false;
    t.off = offsets[t.e];
    t.f0 = by * 32;
    return true;
  }
  __device__ int kbeg(const Tile&) const { return 0; }
  __device__ int kend(const Tile&) const { return H; }
  __device__ void load_a(const Tile& t, int k0, float (*S)[kFmaLd], int tid) const {
    load_kcontig(S, tid, t.mc, k0, H, [&](int r, int k) {
      const int tok = perm[t.off + t.m0 + r] / K;
      return Act<T>::ld(X, int64_t(tok) * H + k);
    });
  }
  __device__ void load_b(const Tile& t, int k0, float (*S)[kFmaLd], int tid) const {
    load_kcontig(S, tid, 64, k0, H, [&](int c, int k) {
      const int row = c < 32 ? t.f0 + c : I + t.f0 + (c - 32);
      return Act<T>::ld(Wgu, (int64_t(t.e) * 2 * I + row) * H + k);
    });
  }
  __device__ void epilogue(const Tile& t, float (&acc)[4][4], int tm, int tn) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = tm + 16 * i;
      if (m >= t.mc) continue;
      const int64_t p = t.off + t.m0 + m;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int f = t.f0 + tn + 16 * jj;
        const float g = Act<T>::round(acc[i][jj]);
        const float u = Act<T>::round(acc[i][jj + 2]);
        Act<T>::st(gu, p * 2 * I + f, g);
        Act<T>::st(gu, p * 2 * I + I + f, u);
        Act<T>::st(a, p * I + f, silu_f(g) * u);
      }
    }
  }
};

// down forward: ybuf[p, :] = a[p, :] * W_d[e]^T  (activation dtype, expert-major rows)
template <class T>
struct DownFwd {
  const T* a; const T* Wd; const int32_t* offsets; T* ybuf;
  int H, E, I;
  struct Tile { int e, m0, mc, n0, off; };
  __device__ bool get_tile(int bx, int by, int, Tile& t) const {
    if (!find_mtile(offsets, E, bx, 64, t.e, t.m0, t.mc)) return false;
    t.off = offsets[t.e];
    t.n0 = by * 64;
    return true;
  }
  __device__ int kbeg(const Tile&) const { return 0; }
  __device__ int kend(const Tile&) const { return I; }
  __device__ void load_a(const Tile& t, int k0, float (*S)[kFmaLd], int tid) const {
    load_kcontig(S, tid, t.mc, k0, I, [&](int r, int k) { return Act<T>::ld(a, int64_t(t.off + t.m0 + r) * I + k); });
  }
  __device__ void load_b(const Tile& t, int k0, float (*S)[kFmaLd], int tid) const {
    load_kcontig(S, tid, 64, k0, I, [&](int r, int k) { return Act<T>::ld(Wd, (int64_t(t.e) * H + t.n0 + r) * I + k); });
  }
  __device__ void epilogue(const Tile& t, float (&acc)[4][4], int tm, int tn) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = tm + 16 * i;
      if (m >= t.mc) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) Act<T>::st(ybuf, int64_t(t.off + t.m0 + m) * H + t.n0 + tn + 16 * j, acc[i][j]);
    }
  }
};

// dA backward: U = dY[tokens of e] * W_d[e]; epilogue forms dGU (SwiGLU
// derivative, scaled by the routing weight) and per-tile partial dw sums.
template <class T>
struct DaBwd {
  const T* dY; const T* Wd; const int32_t* offsets; const int32_t* perm; const float* topk_w;
  const T* gu; const T* a; T* dgu; float* dwpart;
  int H, E, K, I, NT;
  struct Tile { int e, m0, mc, n0, nc, off, nt; };
  __device__ bool get_tile(int bx, int by, int, Tile& t) const {
    if (!find_mtile(offsets, E, bx, 64, t.e, t.m0, t.mc)) return false;
    t.off = offsets[t.e];
    t.n0 = by * 64;
    t.nc = min(64, I - t.n0);
    t.nt = by;
    return true;
  }
  __device__ int kbeg(const Tile&) const { return 0; }
  __device__ int kend(const Tile&) const { return H; }
  __device__ void load_a(const Tile& t, int k0, float (*S)[kFmaLd], int tid) const {
    load_kcontig(S, tid, t.mc, k0, H, [&](int r, int k) {
      const int tok = perm[t.off + t.m0 + r] / K;
      return Act<T>::ld(dY, int64_t(tok) * H + k);
    });
  }
  __device__ void load_b(const Tile& t, int k0, float (*S)[kFmaLd], int tid) const {
    load_rcontig(S, tid, t.nc, k0, H, [&](int n, int k) { return Act<T>::ld(Wd, (int64_t(t.e) * H + k) * I + t.n0 + n); });
  }
  __device__ void epilogue(const Tile& t, float (&acc)[4][4], int tm, int tn) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = tm + 16 * i;
      const bool valid = m < t.mc;
      const int64_t p = t.off + t.m0 + (valid ? m : 0);
      const float wt = valid ? topk_w[perm[p]] : 0.f;
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = tn + 16 * j;
        if (valid && n < t.nc) {
          const int f = t.n0 + n;
          const float U = acc[i][j];
          part = fmaf(U, Act<T>::ld(a, p * I + f), part);
          const float da = wt * U;
          const float g = Act<T>::ld(gu, p * 2 * I + f);
          const float u = Act<T>::ld(gu, p * 2 * I + I + f);
          const float sg = sigmoid_f(g);
          Act<T>::st(dgu, p * 2 * I + f, da * u * sg * (1.f + g * (1.f - sg)));
          Act<T>::st(dgu, p * 2 * I + I + f, da * g * sg);
        }
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) part += __shfl_xor(part, off, 16);
      if (tn == 0 && valid) dwpart[p * NT + t.nt] = part;
    }
  }
};

// dX backward: vbuf[p, :] = dGU[p, :] * W_gu[e]   (activation dtype, expert-major rows)
template <class T>
struct DxBwd {
  const T* dgu; const T* Wgu; const int32_t* offsets; T* vbuf;
  int H, E, I;
  struct Tile { int e, m0, mc, n0, off; };
  __device__ bool get_tile(int bx, int by, int, Tile& t) const {
    if (!find_mtile(offsets, E, bx, 64, t.e, t.m0, t.mc)) return false;
    t.off = offsets[t.e];
    t.n0 = by * 64;
    return true;
  }
  __device__ int kbeg(const Tile&) const { return 0; }
  __device__ int kend(const Tile&) const { return 2 * I; }
  __device__ void load_a(const Tile& t, int k0, float (*S)[kFmaLd], int tid) const {
    load_kcontig(S, tid, t.mc, k0, 2 * I, [&](int r, int k) { return Act<T>::ld(dgu, int64_t(t.off + t.m0 + r) * 2 * I + k); });
  }
  __device__ void load_b(const Tile& t, int k0, float (*S)[kFmaLd], int tid) const {
    load_rcontig(S, tid, 64, k0, 2 * I, [&](int n, int k) { return Act<T>::ld(Wgu, (int64_t(t.e) * 2 * I + k) * H + t.n0 + n); });
  }
  __device__ void epilogue(const Tile& t, float (&acc)[4][4], int tm, int tn) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = tm + 16 * i;
      if (m >= t.mc) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) Act<T>::st(vbuf, int64_t(t.off + t.m0 + m) * H + t.n0 + tn + 16 * j, acc[i][j]);
    }
  }
};

// Dense gate_up weight gradient of expert e: dW[r, c] = sum_p dGU[p, r] X[t(p), c]
template <class T>
struct DenseDwGu {
  const T* dgu; const T* X; const int32_t* offsets; const int32_t* perm; float* dW;
  int H, E, K, I;
  struct Tile { int e, r0, n0, off, ne; };
  __device__ bool get_tile(int bx, int by, int bz, Tile& t) const {
    t.e = bz; t.n0 = bx * 64; t.r0 = by * 64;
    t.off = offsets[t.e]; t.ne = offsets[t.e + 1] - t.off;
    return true;
  }
  __device__ int kbeg(const Tile&) const { return 0; }
  __device__ int kend(const Tile& t) const { return t.ne; }
  __device__ void load_a(const Tile& t, int k0, float (*S)[kFmaLd], int tid) const {
    load_rcontig(S, tid, 64, k0, t.ne, [&](int r, int k) { return Act<T>::ld(dgu, int64_t(t.off + k) * 2 * I + t.r0 + r); });
  }
  __device__ void load_b(const Tile& t, int k0, float (*S)[kFmaLd], int tid) const {
    load_rcontig(S, tid, 64, k0, t.ne, [&](int c, int k) {
      const int tok = perm[t.off + k] / K;
      return Act<T>::ld(X, int64_t(tok) * H + t.n0 + c);
    });
  }
  __device__ void epilogue(const Tile& t, float (&acc)[4][4], int tm, int tn) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dW[(int64_t(t.e) * 2 * I + t.r0 + tm + 16 * i) * H + t.n0 + tn + 16 * j] = acc[i][j];
  }
};

// Dense down weight gradient of expert e: dW[r, c] = sum_p w_p dY[t(p), r] a[p, c]
template <class T>
struct DenseDwD {
  const T* dY; const float* topk_w; const T* a; const int32_t* offsets; const int32_t* perm;
  float* dW;
  int H, E, K, I;
  int64_t ngu;
  struct Tile { int e, r0, n0, nc, off, ne; };
  __device__ bool get_tile(int bx, int by, int bz, Tile& t) const {
    t.e = bz; t.n0 = bx * 64; t.r0 = by * 64; t.nc = min(64, I - t.n0);
    t.off = offsets[t.e]; t.ne = offsets[t.e + 1] - t.off;
    return true;
  }
  __device__ int kbeg(const Tile&) const { return 0; }
  __device__ int kend(const Tile& t) const { return t.ne; }
  __device__ void load_a(const Tile& t, int k0, float (*S)[kFmaLd], int tid) const {
    load_rcontig(S, tid, 64, k0, t.ne, [&](int r, int k) {
      const int s = perm[t.off + k];
      return topk_w[s] * Act<T>::ld(dY, int64_t(s / K) * H + t.r0 + r);
    });
  }
  __device__ void load_b(const Tile& t, int k0, float (*S)[kFmaLd], int tid) const {
    load_rcontig(S, tid, t.nc, k0, t.ne, [&](int c, int k) { return Act<T>::ld(a, int64_t(t.off + k) * I + t.n0 + c); });
  }
  __device__ void epilogue(const Tile& t, float (&acc)[4][4], int tm, int tn) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = tn + 16 * j;
        if (n < t.nc) dW[ngu + (int64_t(t.e) * H + t.r0 + tm + 16 * i) * I + t.n0 + n] = acc[i][j];
      }
  }
};

// ---------------------------------------------------------------------------
// Combines, router backward, masked dW, loss
// ---------------------------------------------------------------------------

template <class T>
__device__ __forceinline__ void store4(T* p, int64_t i, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, int64_t i, float4 v) {
  *reinterpret_cast<float4*>(p + i) = v;
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, int64_t i, float4 v) {
  *reinterpret_cast<uint2*>(p + i) = make_uint2(f2bf2(v.x, v.y),
                                                f2bf2(v.z, v.w));
}

// Four consecutive elements (16 bytes fp32, 8 bytes bf16) as fp32.
template <class T>
__device__ __forceinline__ float4 load4(const T* p);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
template <>
__device__ __forceinline__ float4 load4<bf16_t>(const bf16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}

// Y[t, :] = sum_{j=0..K-1} w[t, j] * y[slot t*K+j]   (fixed j order); four
// columns per thread (H % 64 == 0).
template <class T>
__global__ __launch_bounds__(256) void combine_y_kernel(const T* __restrict__ ybuf,
                                                        const float* __restrict__ topk_w,
                                                        const int32_t* __restrict__ slot_pos, int H,
                                                        int K, T* __restrict__ Y) {
  __shared__ const T* rows[64];
  __shared__ float wts[64];
  const int t = blockIdx.x;
  if (threadIdx.x < K) {
    const int s = t * K + threadIdx.x;
    rows[threadIdx.x] = ybuf + int64_t(slot_pos[s]) * H;
    wts[threadIdx.x] = topk_w[s];
  }
  __syncthreads();
  for (int h = 4 * threadIdx.x; h < H; h += 4 * blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int j = 0; j < K; ++j) {
      const float wj = wts[j];
      const float4 y = load4<T>(rows[j] + h);
      acc.x = fmaf(wj, y.x, acc.x);
      acc.y = fmaf(wj, y.y, acc.y);
      acc.z = fmaf(wj, y.z, acc.z);
      acc.w = fmaf(wj, y.w, acc.w);
    }
    store4<T>(Y, int64_t(t) * H + h, acc);
  }
}

// Per slot: dw[s] = sum of the dA tiles' partial dot products (fixed order).
// A block covers whole tokens (floor(256/K) of them); per token, dlogits of
// the chosen experts: w_j (dw_j - sum_m w_m dw_m), the sum in fixed m order.
// With wrb set it also writes bf16(Wr) [E*H] (the rounded router rows the
// dX combine multiplies), four elements per thread over the grid.
__global__ __launch_bounds__(256) void dw_router_kernel(const float* __restrict__ dwpart, int NT,
                                                        const float* __restrict__ topk_w,
                                                        const int32_t* __restrict__ slot_pos,
                                                        int T, int K, float* __restrict__ dw,
                                                        float* __restrict__ dl,
                                                        const float* __restrict__ Wr,
                                                        bf16_t* __restrict__ wrb, int64_t EH) {
  if (wrb) {
    for (int64_t i = 4 * (int64_t(blockIdx.x) * 256 + threadIdx.x); i < EH;
         i += 4 * int64_t(gridDim.x) * 256) {
      const uint32_t lo = f2bf2(Wr[i], Wr[i + 1]), hi = f2bf2(Wr[i + 2], Wr[i + 3]);
      *reinterpret_cast<uint2*>(wrb + i) = make_uint2(lo, hi);
    }
  }
  __shared__ float swd[256];
  const int tpb = 256 / K;
  const int lt = threadIdx.x / K, j = threadIdx.x - lt * K;
  const int t = blockIdx.x * tpb + lt;
  const bool live = lt < tpb && t < T;
  const int s = t * K + j;
  float d = 0.f, wj = 0.f;
  if (live) {
    const int64_t p = slot_pos[s];
#pragma unroll 4
    for (int nt = 0; nt < NT; ++nt) d += dwpart[p * NT + nt];
    dw[s] = d;
    wj = topk_w[s];
  }
  swd[threadIdx.x] = wj * d;
  __syncthreads();
  if (live) {
    float sw = 0.f;
    for (int m = 0; m < K; ++m) sw += swd[lt * K + m];
    dl[s] = wj * (d - sw);
  }
}

// Dense fp32 router gradient dWr[e, h] = sum over slots p of e of
// dlogits[s(p)] * X[t(p), h] (dlogits is zero off the chosen experts).  The
// expert's slot tokens and dlogits are staged in LDS; two columns per thread.
template <class T>
__global__ __launch_bounds__(256) void dwr_kernel(const float* __restrict__ dl,
                                                  const T* __restrict__ X,
                                                  const int32_t* __restrict__ offsets,
                                                  const int32_t* __restrict__ perm, int H, int K,
                                                  float* __restrict__ dWr,
                                                  int32_t* __restrict__ nonfinite) {
  __shared__ int tok[1024];
  __shared__ float dls[1024];
  const int e = blockIdx.x;
  const int h = 2 * (blockIdx.y * blockDim.x + threadIdx.x);
  const int p0 = offsets[e], p1 = offsets[e + 1];
  float a0 = 0.f, a1 = 0.f;
  for (int w0 = p0; w0 < p1; w0 += 1024) {
    const int wn = min(1024, p1 - w0);
    __syncthreads();
    for (int i = threadIdx.x; i < wn; i += blockDim.x) {
      const int s = perm[w0 + i];
      tok[i] = s / K;
      dls[i] = dl[s];
    }
    __syncthreads();
    if constexpr (std::is_same<T, bf16_t>::value) {
      // both columns in one 4-byte load (h even, H a multiple of 64), 16
      // slots' loads in flight; the same fma order as the generic loop
      if (h < H) {
        int i = 0;
        for (; i + 16 <= wn; i += 16) {
          uint32_t xv[16];
#pragma unroll
          for (int u = 0; u < 16; ++u)
            xv[u] = *reinterpret_cast<const uint32_t*>(X + int64_t(tok[i + u]) * H + h);
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            a0 = fmaf(dls[i + u], __uint_as_float(xv[u] << 16), a0);
            a1 = fmaf(dls[i + u], __uint_as_float(xv[u] & 0xffff0000u), a1);
          }
        }
        for (; i < wn; ++i) {
          const uint32_t xv = *reinterpret_cast<const uint32_t*>(X + int64_t(tok[i]) * H + h);
          a0 = fmaf(dls[i], __uint_as_float(xv << 16), a0);
          a1 = fmaf(dls[i], __uint_as_float(xv & 0xffff0000u), a1);
        }
      }
    } else if (h < H) {
      int i = 0;
      for (; i + 4 <= wn; i += 4) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t base = int64_t(tok[i + u]) * H + h;
          x[2 * u] = Act<T>::ld(X, base);
          x[2 * u + 1] = Act<T>::ld(X, base + 1);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a0 = fmaf(dls[i + u], x[2 * u], a0);
          a1 = fmaf(dls[i + u], x[2 * u + 1], a1);
        }
      }
      for (; i < wn; ++i) {
        const int64_t base = int64_t(tok[i]) * H + h;
        a0 = fmaf(dls[i], Act<T>::ld(X, base), a0);
        a1 = fmaf(dls[i], Act<T>::ld(X, base + 1), a1);
      }
    }
  }
  if (h < H) {
    dWr[int64_t(e) * H + h] = a0;
    dWr[int64_t(e) * H + h + 1] = a1;
    const int bad = !finite_f(a0) + !finite_f(a1);
    if (nonfinite && bad) atomicAdd(nonfinite, bad);
  }
}

// bf16 form of dwr_kernel for H % 8 == 0: a block takes 512 columns of one
// expert, each lane 8 columns (one 16-byte load per slot), and its four
// waves take every fourth slot of the expert, 8 slots' loads in flight.  The
// four partial sums are added in wave order, so the result is deterministic.
__global__ __launch_bounds__(256) void dwr_bf16_kernel(const float* __restrict__ dl,
                                                       const bf16_t* __restrict__ X,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ perm, int H,
                                                       int K, float* __restrict__ dWr,
                                                       int32_t* __restrict__ nonfinite) {
  __shared__ int tok[1024];
  __shared__ float dls[1024];
  __shared__ float part[3][512];
  const int e = blockIdx.x, lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int h = 512 * blockIdx.y + 8 * lane;
  const bool live = h < H;
  const int p0 = offsets[e], p1 = offsets[e + 1];
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
  for (int w0 = p0; w0 < p1; w0 += 1024) {
    const int wn = min(1024, p1 - w0);
    __syncthreads();
    for (int i = threadIdx.x; i < wn; i += blockDim.x) {
      const int s = perm[w0 + i];
      tok[i] = s / K;
      dls[i] = dl[s];
    }
    __syncthreads();
    if (!live) continue;
    int i = wid;
    for (; i + 28 < wn; i += 32) {
      uint4 xv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        xv[u] = *reinterpret_cast<const uint4*>(X + int64_t(tok[i + 4 * u]) * H + h);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float d = dls[i + 4 * u];
        const uint32_t wv[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[2 * c] = fmaf(d, __uint_as_float(wv[c] << 16), acc[2 * c]);
          acc[2 * c + 1] = fmaf(d, __uint_as_float(wv[c] & 0xffff0000u), acc[2 * c + 1]);
        }
      }
    }
    for (; i < wn; i += 4) {
      const uint4 x = *reinterpret_cast<const uint4*>(X + int64_t(tok[i]) * H + h);
      const float d = dls[i];
      const uint32_t wv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[2 * c] = fmaf(d, __uint_as_float(wv[c] << 16), acc[2 * c]);
        acc[2 * c + 1] = fmaf(d, __uint_as_float(wv[c] & 0xffff0000u), acc[2 * c + 1]);
      }
    }
  }
  if (wid > 0) {
#pragma unroll
    for (int c = 0; c < 8; ++c) part[wid - 1][8 * lane + c] = acc[c];
  }
  __syncthreads();
  if (wid == 0 && live) {
    int bad = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float v = ((acc[c] + part[0][8 * lane + c]) + part[1][8 * lane + c]) + part[2][8 * lane + c];
      dWr[int64_t(e) * H + h + c] = v;
      bad += !finite_f(v);
    }
    if (nonfinite && bad) atomicAdd(nonfinite, bad);
  }
}

// dX[t, :] = sum_j v[slot t*K+j] + sum_j dlogits[t, j] * Wr'[e_j, :]; four
// columns per thread.
template <class T>
__global__ __launch_bounds__(256) void combine_dx_kernel(const T* __restrict__ vbuf,
                                                         const float* __restrict__ dl,
                                                         const int32_t* __restrict__ ids,
                                                         const T* __restrict__ Wr,
                                                         const int32_t* __restrict__ slot_pos,
                                                         int H, int K, T* __restrict__ dX) {
  __shared__ const T* vrows[64];
  __shared__ const T* wrows[64];
  __shared__ float dls[64];
  const int t = blockIdx.x;
  if (threadIdx.x < K) {
    const int s = t * K + threadIdx.x;
    vrows[threadIdx.x] = vbuf + int64_t(slot_pos[s]) * H;
    wrows[threadIdx.x] = Wr + int64_t(ids[s]) * H;
    dls[threadIdx.x] = dl[s];
  }
  __syncthreads();
  for (int h = 4 * threadIdx.x; h < H; h += 4 * blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int j = 0; j < K; ++j) {
      const float4 v = load4<T>(vrows[j] + h);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
#pragma unroll 8
    for (int j = 0; j < K; ++j) {
      const float d = dls[j];
      const float4 w = load4<T>(wrows[j] + h);
      acc.x = fmaf(d, w.x, acc.x);
      acc.y = fmaf(d, w.y, acc.y);
      acc.z = fmaf(d, w.z, acc.z);
      acc.w = fmaf(d, w.w, acc.w);
    }
    store4<T>(dX, int64_t(t) * H + h, acc);
  }
}

// Expert-weight gradient at each listed flat index (one thread per entry).
template <class T>
__global__ __launch_bounds__(256) void masked_dw_kernel(
    const uint32_t* __restrict__ idx, int64_t nnz, const T* __restrict__ X,
    const T* __restrict__ dY, const T* __restrict__ dgu, const T* __restrict__ a,
    const float* __restrict__ topk_w, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, int H, int K, int I, uint32_t ngu, int64_t N,
    float* __restrict__ dW, int32_t* __restrict__ nonfinite) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= nnz) return;
  const uint32_t f = idx[i];
  if (int64_t(f) >= N) {  // not a valid flat index: flag it instead of reading out of range
    dW[i] = __int_as_float(0x7fc00000);
    if (nonfinite) atomicAdd(nonfinite, 1);
    return;
  }
  float acc = 0.f;
  if (f < ngu) {
    const uint32_t per = uint32_t(2 * I) * uint32_t(H);
    const int e = int(f / per);
    const uint32_t rem = f - uint32_t(e) * per;
    const int r = int(rem / uint32_t(H)), c = int(rem % uint32_t(H));
    for (int p = offsets[e]; p < offsets[e + 1]; ++p) {
      const int tok = perm[p] / K;
      acc = fmaf(Act<T>::ld(dgu, int64_t(p) * 2 * I + r), Act<T>::ld(X, int64_t(tok) * H + c), acc);
    }
  } else {
    const uint32_t g = f - ngu, per = uint32_t(H) * uint32_t(I);
    const int e = int(g / per);
    const uint32_t rem = g - uint32_t(e) * per;
    const int r = int(rem / uint32_t(I)), c = int(rem % uint32_t(I));
    for (int p = offsets[e]; p < offsets[e + 1]; ++p) {
      const int s = perm[p];
      const float l = topk_w[s] * Act<T>::ld(dY, int64_t(s / K) * H + r);
      acc = fmaf(l, Act<T>::ld(a, int64_t(p) * I + c), acc);
    }
  }
  dW[i] = acc;
  if (nonfinite && !finite_f(acc)) atomicAdd(nonfinite, 1);
}

// Residual stream of stacked layers: out = round(a + b) elementwise.  For
// bf16 operands the fp32 sum is exact unless the exponents differ by more
// than 15, and then b lies far below half an ulp of a, so rounding the fp32
// sum to bf16 gives the correctly rounded sum either way.  Eight elements per
// thread: 16-byte vector accesses when every pointer is 16-byte aligned and
// n is a multiple of 8 (kVec), element accesses otherwise.
template <class T, bool kVec>
__global__ __launch_bounds__(256) void residual_add_kernel(const T* __restrict__ a,
                                                           const T* __restrict__ b, T* __restrict__ out,
                                                           int64_t n) {
  const int64_t i0 = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i0 >= n) return;
  if constexpr (kVec) {
    constexpr int kU = 16 / sizeof(T);  // elements per 16-byte vector
#pragma unroll
    for (int v = 0; v < 8 / kU; ++v) {
      const uint4 x = *reinterpret_cast<const uint4*>(a + i0 + v * kU);
      const uint4 y = *reinterpret_cast<const uint4*>(b + i0 + v * kU);
      uint4 z;
      if constexpr (sizeof(T) == 2) {
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
        uint32_t zs[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = __uint_as_float(xs[q] << 16) + __uint_as_float(ys[q] << 16);
          const float hi = __uint_as_float(xs[q] & 0xffff0000u) + __uint_as_float(ys[q] & 0xffff0000u);
          zs[q] = f2bf2(lo, hi);
        }
        z = make_uint4(zs[0], zs[1], zs[2], zs[3]);
      } else {
        z = make_uint4(__float_as_uint(__uint_as_float(x.x) + __uint_as_float(y.x)),
                       __float_as_uint(__uint_as_float(x.y) + __uint_as_float(y.y)),
                       __float_as_uint(__uint_as_float(x.z) + __uint_as_float(y.z)),
                       __float_as_uint(__uint_as_float(x.w) + __uint_as_float(y.w)));
      }
      *reinterpret_cast<uint4*>(out + i0 + v * kU) = z;
    }
  } else {
    for (int64_t i = i0; i < n && i < i0 + 8; ++i) Act<T>::st(out, i, Act<T>::ld(a, i) + Act<T>::ld(b, i));
  }
}

// Loss: per-block partial sums of (Y - tgt)^2 over 4096 elements, dY written.
// kVec: bf16 operands 16-byte aligned, accessed 8 elements at a time.
template <class T, bool kVec>
__global__ __launch_bounds__(256) void mse_partial_kernel(const T* __restrict__ Y,
                                                          const T* __restrict__ tgt, int64_t n,
                                                          float scale, T* __restrict__ dY,
                                                          float* __restrict__ part) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int64_t base = int64_t(blockIdx.x) * 4096;
  float acc = 0.f;
  if constexpr (kVec) {
    // 8 elements per thread and step in 16-byte accesses (n is a multiple of 8)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int64_t i = base + r * 2048 + tid * 8;
      if (i < n) {
        const uint4 y = *reinterpret_cast<const uint4*>(Y + i);
        const uint4 g = *reinterpret_cast<const uint4*>(tgt + i);
        const uint32_t yw[4] = {y.x, y.y, y.z, y.w}, gw[4] = {g.x, g.y, g.z, g.w};
        uint32_t ow[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float d0 = __uint_as_float(yw[q] << 16) - __uint_as_float(gw[q] << 16);
          const float d1 = __uint_as_float(yw[q] & 0xffff0000u) - __uint_as_float(gw[q] & 0xffff0000u);
          acc = fmaf(d0, d0, acc);
          acc = fmaf(d1, d1, acc);
          ow[q] = f2bf2(scale * d0, scale * d1);
        }
        *reinterpret_cast<uint4*>(dY + i) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
      }
    }
  } else {
#pragma unroll 4
    for (int r = 0; r < 16; ++r) {
      const int64_t i = base + r * 256 + tid;
      if (i < n) {
        const float d = Act<T>::ld(Y, i) - Act<T>::ld(tgt, i);
        acc = fmaf(d, d, acc);
        Act<T>::st(dY, i, scale * d);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((tid & 63) == 0) red[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) part[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void mse_final_kernel(const float* __restrict__ part, int nb,
                                                        float inv_n, float* __restrict__ loss,
                                                        int32_t* __restrict__ nonfinite) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  float acc = 0.f;
  for (int b = tid; b < nb; b += 256) acc += part[b];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((tid & 63) == 0) red[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    const float l = ((red[0] + red[1]) + (red[2] + red[3])) * inv_n;
    *loss = l;
    if (nonfinite && !finite_f(l)) atomicAdd(nonfinite, 1);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
template <class P>
static usaf_status launch_fma(const P& p, dim3 grid, hipStream_t st, int kclass) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return USAF_OK;
  timer_begin(kclass, st);
  hipLaunchKernelGGL(gemm_fma_kernel<P>, grid, dim3(256), 0, st, p);
  timer_end(kclass, st);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

static inline unsigned mtiles_bound(const usaf_moe_shape& s) {
  return unsigned(ceil_div(int64_t(s.T) * s.K, 64) + s.E);
}

// Routing from logits: `parts` holds nparts split-K partial sums (summed
// into st.logits) or, with nparts == 1, the logits themselves.
static usaf_status route_impl(const usaf_moe_shape& s, const float* parts, int nparts,
                              const usaf_moe_state& st, hipStream_t stream) {
  if (nparts < 1 || nparts > kMaxRouterParts) return USAF_ERR_INVALID_ARG;
  const int S = s.T * s.K;
  timer_begin(USAF_K_ROUTE, stream);
  const dim3 tg(unsigned(ceil_div(s.T, 4)));
  float* lg = nparts > 1 ? st.logits : const_cast<float*>(parts);
  const int nv = int(ceil_div(s.E, 64));
  if (nv <= 1)
    hipLaunchKernelGGL(route_topk_kernel<1>, tg, dim3(256), 0, stream, parts, nparts, lg, s.T, s.E, s.K, st.topk_ids, st.topk_w);
  else if (nv <= 2)
    hipLaunchKernelGGL(route_topk_kernel<2>, tg, dim3(256), 0, stream, parts, nparts, lg, s.T, s.E, s.K, st.topk_ids, st.topk_w);
  else if (nv <= 4)
    hipLaunchKernelGGL(route_topk_kernel<4>, tg, dim3(256), 0, stream, parts, nparts, lg, s.T, s.E, s.K, st.topk_ids, st.topk_w);
  else if (nv <= 8)
    hipLaunchKernelGGL(route_topk_kernel<8>, tg, dim3(256), 0, stream, parts, nparts, lg, s.T, s.E, s.K, st.topk_ids, st.topk_w);
  else
    hipLaunchKernelGGL(route_topk_kernel<16>, tg, dim3(256), 0, stream, parts, nparts, lg, s.T, s.E, s.K, st.topk_ids, st.topk_w);
  USAF_LAUNCH_CHECK();
  const int nchunk = int(ceil_div(S, kSortChunk));
  if (int64_t(nchunk) * s.E <= S) {
    int nbits = 0;
    while ((1 << nbits) < s.E) ++nbits;
    hipLaunchKernelGGL(expert_rank_kernel, dim3(unsigned(nchunk)), dim3(kSortChunk),
                       size_t(16) * s.E * sizeof(int), stream, st.topk_ids, S, s.E, nbits, st.perm,
                       st.slot_pos);
    USAF_LAUNCH_CHECK();
    hipLaunchKernelGGL(expert_place_kernel, dim3(unsigned(nchunk)), dim3(kSortChunk),
                       size_t(s.E + 16) * sizeof(int), stream, st.topk_ids, S, s.E, nchunk, st.perm,
                       st.offsets, st.slot_pos);
    USAF_LAUNCH_CHECK();
    hipLaunchKernelGGL(expert_scatter_kernel, dim3(unsigned(ceil_div(S, 256))), dim3(256), 0, stream,
                       st.slot_pos, S, st.perm);
  } else {
    hipLaunchKernelGGL(expert_sort_kernel, dim3(unsigned(s.E)), dim3(1024), 0, stream, st.topk_ids,
                       S, s.E, st.offsets, st.perm, st.slot_pos);
  }
  timer_end(USAF_K_ROUTE, stream);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

template <class T>
static usaf_status forward_impl(const usaf_moe_shape& s, const T* X, const float* Wr, const T* W,
                                T* Y, const usaf_moe_state& st, char* ws, hipStream_t stream) {
  const WsForward L = ws_forward(s);
  T* ybuf = reinterpret_cast<T*>(ws + L.ybuf);
  const T* Wgu = W;
  const T* Wd = W + int64_t(s.E) * 2 * s.I * s.H;
  constexpr bool kMfma = std::is_same<T, bf16_t>::value;
  // router logits (bf16: split-K partial sums in the workspace, summed by
  // the routing kernel in fixed order)
  if constexpr (kMfma) {
    float* parts = reinterpret_cast<float*>(ws + L.ybuf);
    const int nparts = mfma_router_splits(s);
    USAF_TRY(mfma_router(s, X, Wr, parts, nparts, stream));
    USAF_TRY(route_impl(s, parts, nparts, st, stream));
  } else {
    RouterGemm<T> rg{X, Wr, st.logits, s.T, s.H, s.E};
    USAF_TRY(launch_fma(rg, dim3(unsigned(ceil_div(s.T, 64)), unsigned(ceil_div(s.E, 64))), stream,
                        USAF_K_ROUTER_GEMM));
    USAF_TRY(route_impl(s, st.logits, 1, st, stream));
  }
  // experts
  if constexpr (kMfma) {
    // the whole [S, H] fp32-sized region is free during gate_up (the
    // router partials are consumed, the down outputs not yet written)
    USAF_TRY(mfma_gate_up(s, X, Wgu, st.offsets, st.perm, static_cast<T*>(st.gu),
                          static_cast<T*>(st.a), reinterpret_cast<float*>(ws + L.ybuf),
                          2 * bf16_spare_offset(s), stream));
    USAF_TRY(mfma_down(s, static_cast<const T*>(st.a), Wd, st.offsets, ybuf,
                       reinterpret_cast<float*>(ws + L.ybuf + bf16_spare_offset(s)),
                       bf16_spare_offset(s), stream));
  } else {
    GateUpFwd<T> gp{X, Wgu, st.offsets, st.perm, static_cast<T*>(st.gu), static_cast<T*>(st.a),
                    s.H, s.E, s.K, s.I};
    USAF_TRY(launch_fma(gp, dim3(mtiles_bound(s), unsigned(s.I / 32)), stream, USAF_K_GATE_UP));
    DownFwd<T> dp{static_cast<const T*>(st.a), Wd, st.offsets, ybuf, s.H, s.E, s.I};
    USAF_TRY(launch_fma(dp, dim3(mtiles_bound(s), unsigned(s.H / 64)), stream, USAF_K_DOWN));
  }
  timer_begin(USAF_K_COMBINE_Y, stream);
  hipLaunchKernelGGL(combine_y_kernel<T>, dim3(unsigned(s.T)), dim3(256), 0, stream, ybuf,
                     st.topk_w, st.slot_pos, s.H, s.K, Y);
  timer_end(USAF_K_COMBINE_Y, stream);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

template <class T>
static usaf_status backward_impl(const usaf_moe_shape& s, const T* X, const float* Wr, const T* W,
                                 const usaf_moe_state& st, const T* dY, const uint32_t* idx,
                                 int64_t nnz, const void* plan, float* dW, float* dWr, T* dX,
                                 int32_t* nonfinite, char* ws, hipStream_t stream) {
  const WsBackward L = ws_backward(s);
  // sparse mode: a list of nnz entries, possibly empty (idx may then be NULL)
  const bool sparse = idx != nullptr || nnz == 0;
  T* vbuf = reinterpret_cast<T*>(ws + L.vbuf);
  float* dwpart = reinterpret_cast<float*>(ws + L.dwpart);
  float* dl = reinterpret_cast<float*>(ws + L.dl);
  constexpr bool kMfma = std::is_same<T, bf16_t>::value;
  const int NT = kMfma ? mfma_dw_partials(s) : int(ceil_div(s.I, 64));
  const T* Wgu = W;
  const T* Wd = W + int64_t(s.E) * 2 * s.I * s.H;
  T* dgu = static_cast<T*>(st.dgu);
  const T* gu = static_cast<const T*>(st.gu);
  const T* a = static_cast<const T*>(st.a);

  if constexpr (kMfma) {
    // vbuf is free during dA (dX writes it afterwards)
    USAF_TRY(mfma_da(s, dY, Wd, st.offsets, st.perm, st.topk_w, gu, a, dgu, dwpart,
                     reinterpret_cast<float*>(ws + L.vbuf), 2 * bf16_spare_offset(s), stream));
  } else {
    DaBwd<T> da{dY, Wd, st.offsets, st.perm, st.topk_w, gu, a, dgu, dwpart, s.H, s.E, s.K, s.I, NT};
    USAF_TRY(launch_fma(da, dim3(mtiles_bound(s), unsigned(NT)), stream, USAF_K_DA));
  }
  timer_begin(USAF_K_ROUTER_BWD, stream);
  // bf16 layers: the combine reads bf16(Wr), written here once per call
  bf16_t* wrb = nullptr;
  if constexpr (kMfma) wrb = reinterpret_cast<bf16_t*>(ws + L.wrb);
  hipLaunchKernelGGL(dw_router_kernel, dim3(unsigned(ceil_div(s.T, 256 / s.K))), dim3(256), 0,
                     stream, dwpart, NT, st.topk_w, st.slot_pos, s.T, s.K, st.dw, dl, Wr, wrb,
                     int64_t(s.E) * s.H);
  USAF_LAUNCH_CHECK();
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (s.H % 8 == 0 && (reinterpret_cast<uintptr_t>(X) & 15) == 0)
      hipLaunchKernelGGL(dwr_bf16_kernel, dim3(unsigned(s.E), unsigned(ceil_div(s.H, 512))), dim3(256),
                         0, stream, dl, X, st.offsets, st.perm, s.H, s.K, dWr,
                         sparse ? nonfinite : nullptr);
    else
      hipLaunchKernelGGL(dwr_kernel<T>, dim3(unsigned(s.E), unsigned(ceil_div(s.H, 512))), dim3(256),
                         0, stream, dl, X, st.offsets, st.perm, s.H, s.K, dWr,
                         sparse ? nonfinite : nullptr);
  } else {
    hipLaunchKernelGGL(dwr_kernel<T>, dim3(unsigned(s.E), unsigned(ceil_div(s.H, 512))), dim3(256),
                       0, stream, dl, X, st.offsets, st.perm, s.H, s.K, dWr,
                       sparse ? nonfinite : nullptr);
  }
  timer_end(USAF_K_ROUTER_BWD, stream);
  USAF_LAUNCH_CHECK();
  if (dX) {
    if constexpr (kMfma) {
      USAF_TRY(mfma_dx(s, dgu, Wgu, st.offsets, vbuf,
                       reinterpret_cast<float*>(ws + L.vbuf + bf16_spare_offset(s)),
                       bf16_spare_offset(s), stream));
    } else {
      DxBwd<T> dx{dgu, Wgu, st.offsets, vbuf, s.H, s.E, s.I};
      USAF_TRY(launch_fma(dx, dim3(mtiles_bound(s), unsigned(s.H / 64)), stream, USAF_K_DX));
    }
    timer_begin(USAF_K_COMBINE_DX, stream);
    const T* wr_act;
    if constexpr (kMfma) wr_act = wrb; else wr_act = Wr;
    hipLaunchKernelGGL(combine_dx_kernel<T>, dim3(unsigned(s.T)), dim3(256), 0, stream, vbuf, dl,
                       st.topk_ids, wr_act, st.slot_pos, s.H, s.K, dX);
    timer_end(USAF_K_COMBINE_DX, stream);
    USAF_LAUNCH_CHECK();
  }
  const int64_t ngu = int64_t(s.E) * 2 * s.I * s.H;
  if (sparse) {
    if constexpr (kMfma) {
      return masked_dw_bf16(s, idx, nnz, X, dY, dgu, a, st.topk_w, st.offsets, st.perm, dW,
                            nonfinite, plan, ws + L.seg, stream);
    }
    if (nnz > 0) {
      timer_begin(USAF_K_MASKED_DW, stream);
      hipLaunchKernelGGL(masked_dw_kernel<T>, dim3(unsigned(ceil_div(nnz, 256))), dim3(256), 0,
                         stream, idx, nnz, X, dY, dgu, a, st.topk_w, st.offsets, st.perm, s.H, s.K,
                         s.I, uint32_t(ngu), n_weights(s), dW, nonfinite);
      timer_end(USAF_K_MASKED_DW, stream);
      USAF_LAUNCH_CHECK();
    }
  } else {
    if constexpr (kMfma) {
      return mfma_dense_dw(s, X, dY, dgu, a, st.offsets, st.perm, st.topk_w,
                           reinterpret_cast<bf16_t*>(vbuf), dW, stream);
    }
    DenseDwGu<T> g1{dgu, X, st.offsets, st.perm, dW, s.H, s.E, s.K, s.I};
    USAF_TRY(launch_fma(g1, dim3(unsigned(s.H / 64), unsigned(2 * s.I / 64), unsigned(s.E)), stream, USAF_K_DENSE_DW));
    DenseDwD<T> g2{dY, st.topk_w, a, st.offsets, st.perm, dW, s.H, s.E, s.K, s.I, ngu};
    USAF_TRY(launch_fma(g2, dim3(unsigned(ceil_div(s.I, 64)), unsigned(s.H / 64), unsigned(s.E)), stream, USAF_K_DENSE_DW));
  }
  return USAF_OK;
}

template <class T>
static usaf_status mse_impl(const usaf_moe_shape& s, const T* Y, const T* tgt, T* dY, float* loss,
                            int32_t* nonfinite, char* ws, hipStream_t stream) {
  const int64_t n = int64_t(s.T) * s.H;
  const int nb = int(ceil_div(n, 4096));
  float* part = reinterpret_cast<float*>(ws);
  timer_begin(USAF_K_MSE, stream);
  const bool vec = std::is_same<T, bf16_t>::value && n % 8 == 0 &&
                   ((reinterpret_cast<uintptr_t>(Y) | reinterpret_cast<uintptr_t>(tgt) |
                     reinterpret_cast<uintptr_t>(dY)) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL((mse_partial_kernel<T, std::is_same<T, bf16_t>::value>), dim3(unsigned(nb)), dim3(256), 0,
                       stream, Y, tgt, n, float(2.0 / double(n)), dY, part);
  else
    hipLaunchKernelGGL((mse_partial_kernel<T, false>), dim3(unsigned(nb)), dim3(256), 0, stream, Y, tgt, n,
                       float(2.0 / double(n)), dY, part);
  USAF_LAUNCH_CHECK();
  hipLaunchKernelGGL(mse_final_kernel, dim3(1), dim3(256), 0, stream, part, nb,
                     float(1.0 / double(n)), loss, nonfinite);
  timer_end(USAF_K_MSE, stream);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

usaf_status mse_launch(const usaf_moe_shape& s, const void* Y, const void* tgt, void* dY,
                       float* loss, int32_t* nonfinite, float* part, hipStream_t stream) {
  char* ws = reinterpret_cast<char*>(part);
  if (s.act == USAF_BF16)
    return mse_impl<bf16_t>(s, static_cast<const bf16_t*>(Y), static_cast<const bf16_t*>(tgt),
                            static_cast<bf16_t*>(dY), loss, nonfinite, ws, stream);
  return mse_impl<float>(s, static_cast<const float*>(Y), static_cast<const float*>(tgt),
                         static_cast<float*>(dY), loss, nonfinite, ws, stream);
}

}  // namespace usaf

using namespace usaf;

static bool state_ok(const usaf_moe_state* st, bool bwd) {
  if (!st || !st->logits || !st->topk_ids || !st->topk_w || !st->offsets || !st->perm ||
      !st->slot_pos || !st->gu || !st->a)
    return false;
  if (bwd && (!st->dgu || !st->dw)) return false;
  return true;
}

extern "C" usaf_status usaf_moe_forward(const usaf_moe_shape* shape, const void* X, const float* Wr,
                                        const void* Wflat, void* Y, const usaf_moe_state* state,
                                        void* ws, size_t ws_bytes, hipStream_t stream) {
  USAF_TRY(check_shape(shape));
  if (!X || !Wr || !Wflat || !Y || !state_ok(state, false)) return USAF_ERR_INVALID_ARG;
  if (!ws || ws_bytes < ws_forward(*shape).total) return USAF_ERR_WORKSPACE;
  if (shape->act == USAF_BF16)
    return forward_impl<bf16_t>(*shape, static_cast<const bf16_t*>(X), Wr,
                                static_cast<const bf16_t*>(Wflat), static_cast<bf16_t*>(Y), *state,
                                static_cast<char*>(ws), stream);
  return forward_impl<float>(*shape, static_cast<const float*>(X), Wr,
                             static_cast<const float*>(Wflat), static_cast<float*>(Y), *state,
                             static_cast<char*>(ws), stream);
}

extern "C" usaf_status usaf_moe_forward_q4(const usaf_moe_shape* shape, const void* X,
                                           const float* Wr, const usaf_q4_experts* w, void* Y,
                                           const usaf_moe_state* state, void* ws, size_t ws_bytes,
                                           hipStream_t stream) {
  USAF_TRY(check_shape(shape));
  if (!X || !Wr || !w || !Y || !state_ok(state, false)) return USAF_ERR_INVALID_ARG;
  if (!w->q_gu || !w->s_gu || !w->z_gu || !w->q_d || !w->s_d || !w->z_d) return USAF_ERR_INVALID_ARG;
  const usaf_moe_shape& s = *shape;
  if (s.act != USAF_BF16) return USAF_ERR_UNSUPPORTED;
  if ((w->group != 64 && w->group != 128) || s.H % (2 * w->group) || s.I % (2 * w->group))
    return USAF_ERR_UNSUPPORTED;  // an even number of groups per row (4-byte scale pairs)
  if ((reinterpret_cast<uintptr_t>(w->q_gu) | reinterpret_cast<uintptr_t>(w->q_d)) & 15)
    return USAF_ERR_UNSUPPORTED;  // 16-byte code loads
  if ((reinterpret_cast<uintptr_t>(w->s_gu) | reinterpret_cast<uintptr_t>(w->z_gu) |
       reinterpret_cast<uintptr_t>(w->s_d) | reinterpret_cast<uintptr_t>(w->z_d)) & 3)
    return USAF_ERR_UNSUPPORTED;  // 4-byte scale and zero pairs
  if (!ws || ws_bytes < ws_forward(s).total) return USAF_ERR_WORKSPACE;
  const WsForward L = ws_forward(s);
  char* wsc = static_cast<char*>(ws);
  bf16_t* ybuf = reinterpret_cast<bf16_t*>(wsc + L.ybuf);
  const bf16_t* Xb = static_cast<const bf16_t*>(X);
  const usaf_moe_state& st = *state;
  float* parts = reinterpret_cast<float*>(wsc + L.ybuf);
  const int nparts = mfma_router_splits(s);
  USAF_TRY(mfma_router(s, Xb, Wr, parts, nparts, stream));
  USAF_TRY(route_impl(s, parts, nparts, st, stream));
  USAF_TRY(q4_gate_up(s, Xb, *w, st.offsets, st.perm, static_cast<bf16_t*>(st.gu),
                      static_cast<bf16_t*>(st.a), reinterpret_cast<float*>(wsc + L.ybuf),
                      2 * bf16_spare_offset(s), stream));
  USAF_TRY(q4_down(s, static_cast<const bf16_t*>(st.a), *w, st.offsets, ybuf,
                   reinterpret_cast<float*>(wsc + L.ybuf + bf16_spare_offset(s)),
                   bf16_spare_offset(s), stream));
  timer_begin(USAF_K_COMBINE_Y, stream);
  hipLaunchKernelGGL(combine_y_kernel<bf16_t>, dim3(unsigned(s.T)), dim3(256), 0, stream, ybuf,
                     st.topk_w, st.slot_pos, s.H, s.K, static_cast<bf16_t*>(Y));
  timer_end(USAF_K_COMBINE_Y, stream);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

extern "C" usaf_status usaf_masked_backward(const usaf_moe_shape* shape, const void* X,
                                            const float* Wr, const void* Wflat,
                                            const usaf_moe_state* state, const void* dY,
                                            const uint32_t* idx, int64_t nnz, const void* plan,
                                            float* dW, float* dWr, void* dX, int32_t* nonfinite,
                                            void* ws, size_t ws_bytes, hipStream_t stream) {
  USAF_TRY(check_shape(shape));
  if (!X || !Wr || !Wflat || !dY || !dWr || !state_ok(state, true)) return USAF_ERR_INVALID_ARG;
  const int64_t N = n_weights(*shape);
  if (nnz < 0 || nnz > N) return USAF_ERR_INVALID_ARG;
  if (!idx && nnz != N && nnz != 0) return USAF_ERR_INVALID_ARG;
  if (nnz > 0 && !dW) return USAF_ERR_INVALID_ARG;
  if (!ws || ws_bytes < ws_backward(*shape).total) return USAF_ERR_WORKSPACE;
  if (shape->act == USAF_BF16 && idx && nnz > 0 && !masked_dw_fits(*shape))
    return USAF_ERR_UNSUPPORTED;
  if (shape->act == USAF_BF16)
    return backward_impl<bf16_t>(*shape, static_cast<const bf16_t*>(X), Wr,
                                 static_cast<const bf16_t*>(Wflat), *state,
                                 static_cast<const bf16_t*>(dY), idx, nnz, idx ? plan : nullptr, dW,
                                 dWr, static_cast<bf16_t*>(dX), nonfinite, static_cast<char*>(ws),
                                 stream);
  return backward_impl<float>(*shape, static_cast<const float*>(X), Wr,
                              static_cast<const float*>(Wflat), *state,
                              static_cast<const float*>(dY), idx, nnz, nullptr, dW, dWr,
                              static_cast<float*>(dX), nonfinite, static_cast<char*>(ws), stream);
}

extern "C" usaf_status usaf_masked_plan(const usaf_moe_shape* shape, const uint32_t* idx,
                                        int64_t nnz, void* plan, size_t plan_bytes,
                                        hipStream_t stream) {
  USAF_TRY(check_shape(shape));
  if (nnz < 0 || nnz > n_weights(*shape) || (nnz > 0 && !idx)) return USAF_ERR_INVALID_ARG;
  if (shape->act != USAF_BF16) return USAF_OK;  // fp32 layers need no plan
  if (!plan || plan_bytes < size_t(masked_plan_bytes(*shape))) return USAF_ERR_WORKSPACE;
  return masked_plan_bf16(*shape, idx, nnz, plan, stream);
}

extern "C" usaf_status usaf_mse_grad(const usaf_moe_shape* shape, const void* Y, const void* tgt,
                                     void* dY, float* loss, int32_t* nonfinite, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  USAF_TRY(check_shape(shape));
  if (!Y || !tgt || !dY || !loss) return USAF_ERR_INVALID_ARG;
  const int64_t n = int64_t(shape->T) * shape->H;
  if (!ws || ws_bytes < size_t(ceil_div(n, 4096)) * 4 + 64) return USAF_ERR_WORKSPACE;
  return mse_launch(*shape, Y, tgt, dY, loss, nonfinite, static_cast<float*>(ws), stream);
}

extern "C" usaf_status usaf_residual_add(int32_t act, const void* a, const void* b, void* out,
                                         int64_t n, hipStream_t stream) {
  if (n < 0 || (act != USAF_BF16 && act != USAF_F32)) return USAF_ERR_INVALID_ARG;
  if (n == 0) return USAF_OK;
  if (!a || !b || !out) return USAF_ERR_INVALID_ARG;
  const int64_t blocks = ceil_div(ceil_div(n, 8), 256);
  if (blocks >= (int64_t(1) << 31)) return USAF_ERR_UNSUPPORTED;
  const bool vec = n % 8 == 0 && ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
                                    reinterpret_cast<uintptr_t>(out)) & 15) == 0;
  if (act == USAF_BF16) {
    auto* k = vec ? residual_add_kernel<bf16_t, true> : residual_add_kernel<bf16_t, false>;
    hipLaunchKernelGGL(k, dim3(unsigned(blocks)), dim3(256), 0, stream, static_cast<const bf16_t*>(a),
                       static_cast<const bf16_t*>(b), static_cast<bf16_t*>(out), n);
  } else {
    auto* k = vec ? residual_add_kernel<float, true> : residual_add_kernel<float, false>;
    hipLaunchKernelGGL(k, dim3(unsigned(blocks)), dim3(256), 0, stream, static_cast<const float*>(a),
                       static_cast<const float*>(b), static_cast<float*>(out), n);
  }
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

extern "C" usaf_status usaf_route(const usaf_moe_shape* shape, const float* logits,
                                  const usaf_moe_state* state, hipStream_t stream) {
  USAF_TRY(check_shape(shape));
  if (!logits || !state || !state->topk_ids || !state->topk_w || !state->offsets ||
      !state->perm || !state->slot_pos)
    return USAF_ERR_INVALID_ARG;
  return route_impl(*shape, logits, 1, *state, stream);
}
