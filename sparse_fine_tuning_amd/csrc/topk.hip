// Global top-k by |grad| (importance selection) and RigL drop / grow.
//
// Method: the usaf README ("tsuyu122/usaf"), "how it works": the importance
// phase keeps the ~0.5% of expert weights with the largest gradient
// magnitude; RigL reselection replaces part of the active set every 50 steps
// (RESELECT_EVERY in the env-var table).
//
// Selection is an exact radix select over 31-bit keys (|g| as fp32 bits, or
// an inverted |w| for RigL's drop), three digit passes (11, 11, 9 bits) that
// fix the k-th key K*, then an ordered compaction that keeps every key > K*
// and the lowest-index keys == K* until k are taken.  Output indices are
// therefore ascending and the result is unique: rank by (key desc, index asc).
#include "common.hpp"
#include "moe_internal.hpp"
#include "timing.hpp"

namespace usaf {

constexpr int kTopkTile = 4096;  // elements per block: 256 threads x 16 rounds
constexpr int kTopkBins = 2048;

struct KeyGrad {
  const float* g;
  __device__ __forceinline__ uint32_t operator()(int64_t i) const {
    return __float_as_uint(g[i]) & 0x7fffffffu;
  }
};
// Smaller |w| ranks first; bf16 magnitude bits are 15 wide.
struct KeyDropBf16 {
  const bf16_t* W;
  const uint32_t* idx;
  __device__ __forceinline__ uint32_t operator()(int64_t i) const {
    return 0x7fffu - (uint32_t(W[idx[i]]) & 0x7fffu);
  }
};
struct KeyDropF32 {
  const float* W;
  const uint32_t* idx;
  __device__ __forceinline__ uint32_t operator()(int64_t i) const {
    return 0x7fffffffu - (__float_as_uint(W[idx[i]]) & 0x7fffffffu);
  }
};

__device__ __forceinline__ int64_t lower_bound_u32(const uint32_t* a, int64_t n, uint64_t v) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (uint64_t(a[mid]) < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Marks, in an LDS bitmap of kTopkTile bits, the excluded indices of the tile
// starting at i0.  Ends with a barrier.
__device__ __forceinline__ void mark_excluded(uint32_t* bm, const uint32_t* ex, int64_t nex,
                                              int64_t i0) {
  __shared__ int64_t range[2];
  for (int w = threadIdx.x; w < kTopkTile / 32; w += blockDim.x) bm[w] = 0;
  if (ex && threadIdx.x < 2) range[threadIdx.x] = lower_bound_u32(ex, nex, uint64_t(i0) + threadIdx.x * kTopkTile);
  __syncthreads();
  if (ex) {
    for (int64_t q = range[0] + threadIdx.x; q < range[1]; q += blockDim.x) {
      const int64_t l = int64_t(ex[q]) - i0;
      if (l >= 0 && l < kTopkTile) atomicOr(&bm[l >> 5], 1u << (l & 31));
    }
  }
  __syncthreads();
}

__device__ __forceinline__ bool is_marked(const uint32_t* bm, int l) { return (bm[l >> 5] >> (l & 31)) & 1u; }

// state[0] = key prefix fixed so far, state[1] = how many of the keys that
// match the prefix are still to be taken.
__global__ void topk_init_kernel(uint32_t* hist, uint32_t* state, uint32_t k) {
  for (int b = threadIdx.x; b < kTopkBins; b += blockDim.x) hist[b] = 0;
  if (threadIdx.x == 0) {
    state[0] = 0;
    state[1] = k;
  }
}

template <class KF>
__global__ __launch_bounds__(256) void topk_hist_kernel(KF key, int64_t n, const uint32_t* ex,
                                                        int64_t nex, int shift, uint32_t dmask,
                                                        int cmp_shift,
                                                        const uint32_t* __restrict__ state,
                                                        uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[kTopkBins];
  __shared__ uint32_t bm[kTopkTile / 32];
  for (int b = threadIdx.x; b < kTopkBins; b += 256) h[b] = 0;
  const int64_t i0 = int64_t(blockIdx.x) * kTopkTile;
  mark_excluded(bm, ex, nex, i0);
  const uint32_t prefix = state[0];
  for (int r = 0; r < 16; ++r) {
    const int l = r * 256 + threadIdx.x;
    const int64_t i = i0 + l;
    if (i < n && !is_marked(bm, l)) {
      const uint32_t kv = key(i);
      if (cmp_shift >= 31 || (kv >> cmp_shift) == (prefix >> cmp_shift))
        atomicAdd(&h[(kv >> shift) & dmask], 1u);
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b <= int(dmask); b += 256)
    if (h[b]) atomicAdd(&hist[b], h[b]);
}

// One block: find the digit whose cumulative count from the top reaches
// state[1]; fold it into the prefix; clear the histogram for the next pass.
__global__ __launch_bounds__(256) void topk_select_kernel(uint32_t* __restrict__ hist, int nbins,
                                                          int shift, uint32_t* __restrict__ state) {
  __shared__ uint32_t csum[256];
  const int per = nbins / 256;
  uint32_t s = 0;
  for (int q = 0; q < per; ++q) s += hist[threadIdx.x * per + q];
  csum[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t krem = state[1];
    uint32_t above = 0;
    int c = 255;
    for (; c > 0; --c) {
      if (above + csum[c] >= krem) break;
      above += csum[c];
    }
    int b = c * per + per - 1;
    for (; b > c * per; --b) {
      const uint32_t hb = hist[b];
      if (above + hb >= krem) break;
      above += hb;
    }
    state[0] |= uint32_t(b) << shift;
    state[1] = krem - above;
  }
  __syncthreads();
  for (int b = threadIdx.x; b < nbins; b += 256) hist[b] = 0;
}

template <class KF>
__global__ __launch_bounds__(256) void topk_count_kernel(KF key, int64_t n, const uint32_t* ex,
                                                         int64_t nex,
                                                         const uint32_t* __restrict__ state,
                                                         uint32_t* __restrict__ gt_cnt,
                                                         uint32_t* __restrict__ eq_cnt) {
  __shared__ uint32_t bm[kTopkTile / 32];
  __shared__ uint32_t red[2][4];
  const int64_t i0 = int64_t(blockIdx.x) * kTopkTile;
  mark_excluded(bm, ex, nex, i0);
  const uint32_t thr = state[0];
  uint32_t gt = 0, eq = 0;
  for (int r = 0; r < 16; ++r) {
    const int l = r * 256 + threadIdx.x;
    const int64_t i = i0 + l;
    if (i < n && !is_marked(bm, l)) {
      const uint32_t kv = key(i);
      gt += kv > thr;
      eq += kv == thr;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    gt += __shfl_xor(gt, off, 64);
    eq += __shfl_xor(eq, off, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = gt;
    red[1][threadIdx.x >> 6] = eq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    gt_cnt[blockIdx.x] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    eq_cnt[blockIdx.x] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  }
}

// One block of 1024 threads: in-place exclusive scan of two u32 arrays.
__global__ __launch_bounds__(1024) void scan2_kernel(uint32_t* __restrict__ a,
                                                     uint32_t* __restrict__ b, int64_t n) {
  __shared__ uint32_t sa[1024], sb[1024];
  const int tid = threadIdx.x;
  const int64_t chunk = (n + 1023) / 1024;
  const int64_t lo = min(n, chunk * tid), hi = min(n, lo + chunk);
  uint32_t ta = 0, tb = 0;
  for (int64_t i = lo; i < hi; ++i) {
    ta += a[i];
    tb += b[i];
  }
  sa[tid] = ta;
  sb[tid] = tb;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const uint32_t va = tid >= off ? sa[tid - off] : 0;
    const uint32_t vb = tid >= off ? sb[tid - off] : 0;
    __syncthreads();
    sa[tid] += va;
    sb[tid] += vb;
    __syncthreads();
  }
  uint32_t ra = sa[tid] - ta, rb = sb[tid] - tb;
  for (int64_t i = lo; i < hi; ++i) {
    const uint32_t xa = a[i], xb = b[i];
    a[i] = ra;
    b[i] = rb;
    ra += xa;
    rb += xb;
  }
}

// Block-wide exclusive count of `flag` over 256 threads (4 waves).
__device__ __forceinline__ uint32_t block_excl(bool flag, uint32_t* wtot, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint64_t b = __ballot(flag);
  const uint32_t pre = __popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) wtot[wid] = __popcll(b);
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wid; ++w) base += wtot[w];
  total = wtot[0] + wtot[1] + wtot[2] + wtot[3];
  __syncthreads();
  return base + pre;
}

template <class KF>
__global__ __launch_bounds__(256) void topk_write_kernel(
    KF key, int64_t n, const uint32_t* ex, int64_t nex, const uint32_t* __restrict__ state,
    const uint32_t* __restrict__ gt_before, const uint32_t* __restrict__ eq_before,
    uint32_t* __restrict__ out_idx, float* __restrict__ out_val, const float* __restrict__ valsrc) {
  __shared__ uint32_t bm[kTopkTile / 32];
  __shared__ uint32_t wt[4];
  const int64_t i0 = int64_t(blockIdx.x) * kTopkTile;
  mark_excluded(bm, ex, nex, i0);
  const uint32_t thr = state[0], krem = state[1];
  uint32_t eqrun = eq_before[blockIdx.x];
  uint32_t pos = gt_before[blockIdx.x] + min(eqrun, krem);
  for (int r = 0; r < 16; ++r) {
    const int l = r * 256 + threadIdx.x;
    const int64_t i = i0 + l;
    const bool valid = i < n && !is_marked(bm, l);
    const uint32_t kv = valid ? key(i) : 0u;
    const bool gt = valid && kv > thr;
    const bool eq = valid && kv == thr;
    uint32_t eq_tot, sel_tot;
    const uint32_t eq_pre = block_excl(eq, wt, eq_tot);
    const bool sel = gt || (eq && eqrun + eq_pre < krem);
    const uint32_t sel_pre = block_excl(sel, wt, sel_tot);
    if (sel) {
      out_idx[pos + sel_pre] = uint32_t(i);
      if (out_val) out_val[pos + sel_pre] = valsrc[i];
    }
    eqrun += eq_tot;
    pos += sel_tot;
  }
}

size_t topk_ws_bytes(int64_t n) {
  const int64_t ntiles = ceil_div(n > 0 ? n : 1, kTopkTile);
  return align256(kTopkBins * 4) + align256(64 * 4) + 2 * align256(size_t(ntiles) * 4);
}

// Enqueue a full selection: the k keys ranked first by (key desc, index asc)
// among n (minus the excluded), written ascending to out_idx.
template <class KF>
usaf_status topk_run(KF key, int64_t n, int64_t k, const uint32_t* ex, int64_t nex,
                     uint32_t* out_idx, float* out_val, const float* valsrc, char* ws,
                     hipStream_t st) {
  if (k == 0 || n == 0) return USAF_OK;
  const int64_t ntiles = ceil_div(n, kTopkTile);
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws);
  uint32_t* state = reinterpret_cast<uint32_t*>(ws + align256(kTopkBins * 4));
  uint32_t* gt = reinterpret_cast<uint32_t*>(ws + align256(kTopkBins * 4) + align256(64 * 4));
  uint32_t* eq = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(gt) + align256(size_t(ntiles) * 4));
  const dim3 grid{unsigned(ntiles), 1, 1}, blk{256, 1, 1};
  timer_begin(USAF_K_TOPK, st);
  hipLaunchKernelGGL(topk_init_kernel, dim3(1), blk, 0, st, hist, state, uint32_t(k));
  USAF_LAUNCH_CHECK();
  struct Pass { int shift; uint32_t dmask; int cmp_shift; int nbins; };
  const Pass passes[3] = {{20, 0x7ffu, 31, 2048}, {9, 0x7ffu, 20, 2048}, {0, 0x1ffu, 9, 512}};
  for (const Pass& p : passes) {
    hipLaunchKernelGGL(topk_hist_kernel<KF>, grid, blk, 0, st, key, n, ex, nex, p.shift, p.dmask,
                       p.cmp_shift, state, hist);
    USAF_LAUNCH_CHECK();
    hipLaunchKernelGGL(topk_select_kernel, dim3(1), blk, 0, st, hist, p.nbins, p.shift, state);
    USAF_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(topk_count_kernel<KF>, grid, blk, 0, st, key, n, ex, nex, state, gt, eq);
  USAF_LAUNCH_CHECK();
  hipLaunchKernelGGL(scan2_kernel, dim3(1), dim3(1024), 0, st, gt, eq, ntiles);
  USAF_LAUNCH_CHECK();
  hipLaunchKernelGGL(topk_write_kernel<KF>, grid, blk, 0, st, key, n, ex, nex, state, gt, eq,
                     out_idx, out_val, valsrc);
  timer_end(USAF_K_TOPK, st);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

// ---------------------------------------------------------------------------
// RigL: state remap after drop / grow
// ---------------------------------------------------------------------------

// Kept entry at old position q lands at (q - dropped before q) + (grown < f).
__global__ __launch_bounds__(256) void rigl_place_kept_kernel(
    const uint32_t* __restrict__ old_idx, const float* __restrict__ old_m,
    const float* __restrict__ old_v, int64_t k, const uint32_t* __restrict__ dpos,
    const uint32_t* __restrict__ grown, int64_t r, uint32_t* __restrict__ new_idx,
    float* __restrict__ new_m, float* __restrict__ new_v) {
  const int64_t q = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= k) return;
  const int64_t nd = lower_bound_u32(dpos, r, uint64_t(q));
  if (nd < r && dpos[nd] == uint32_t(q)) return;  // dropped
  const uint32_t f = old_idx[q];
  const int64_t out = (q - nd) + lower_bound_u32(grown, r, f);
  new_idx[out] = f;
  new_m[out] = old_m[q];
  new_v[out] = old_v[q];
}

// Grown entry i lands at i + (kept entries < f); its moments start at zero.
__global__ __launch_bounds__(256) void rigl_place_grown_kernel(
    const uint32_t* __restrict__ old_idx, int64_t k, const uint32_t* __restrict__ dpos,
    const uint32_t* __restrict__ grown, int64_t r, uint32_t* __restrict__ new_idx,
    float* __restrict__ new_m, float* __restrict__ new_v) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= r) return;
  const uint32_t f = grown[i];
  const int64_t q = lower_bound_u32(old_idx, k, f);
  const int64_t kept_less = q - lower_bound_u32(dpos, r, uint64_t(q));
  const int64_t out = i + kept_less;
  new_idx[out] = f;
  new_m[out] = 0.f;
  new_v[out] = 0.f;
}

// Entries of a fresh top-k that are not in the old active set.
__global__ __launch_bounds__(256) void rigl_novelty_kernel(const uint32_t* __restrict__ fresh,
                                                           const uint32_t* __restrict__ old_idx,
                                                           int64_t k, uint32_t* __restrict__ cnt) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  bool novel = false;
  if (i < k) {
    const uint32_t f = fresh[i];
    const int64_t q = lower_bound_u32(old_idx, k, f);
    novel = !(q < k && old_idx[q] == f);
  }
  const uint64_t b = __ballot(novel);
  if ((threadIdx.x & 63) == 0 && b) atomicAdd(cnt, uint32_t(__popcll(b)));
}

__global__ void rigl_stats_init_kernel(uint32_t* cnt) { *cnt = 0; }

__global__ void rigl_stats_kernel(const uint32_t* __restrict__ cnt, int64_t r,
                                  usaf_rigl_stats* __restrict__ stats) {
  stats->n_drop = r;
  stats->n_grow = r;
  stats->topk_new_vs_old = int64_t(*cnt);
}

struct WsRigl {
  size_t topk, dpos, grown, fresh, cnt, total;
};
static WsRigl ws_rigl(int64_t N, int64_t k) {
  WsRigl L;
  L.topk = 0;
  const size_t t = topk_ws_bytes(N > k ? N : k);
  L.dpos = align256(t);
  L.grown = L.dpos + align256(size_t(k) * 4 + 4);
  L.fresh = L.grown + align256(size_t(k) * 4 + 4);
  L.cnt = L.fresh + align256(size_t(k) * 4 + 4);
  L.total = L.cnt + 256;
  return L;
}

}  // namespace usaf

using namespace usaf;

extern "C" usaf_status usaf_importance_topk(const float* grad, int64_t n, int64_t k,
                                            const uint32_t* exclude, int64_t n_exclude,
                                            uint32_t* out_idx, float* out_val, void* ws,
                                            size_t ws_bytes, hipStream_t stream) {
  if (n < 0 || k < 0 || n_exclude < 0 || n >= (int64_t(1) << 32)) return USAF_ERR_INVALID_ARG;
  if (!exclude) n_exclude = 0;
  if (n_exclude > n || k > n - n_exclude) return USAF_ERR_INVALID_ARG;
  if (k == 0) return USAF_OK;
  if (!grad || !out_idx) return USAF_ERR_INVALID_ARG;
  if (!ws || ws_bytes < topk_ws_bytes(n)) return USAF_ERR_WORKSPACE;
  return topk_run(KeyGrad{grad}, n, k, n_exclude ? exclude : nullptr, n_exclude, out_idx, out_val,
                  grad, static_cast<char*>(ws), stream);
}

extern "C" usaf_status usaf_rigl_reselect(const usaf_moe_shape* shape, const float* grad,
                                          const void* Wflat, const uint32_t* old_idx,
                                          const float* old_m, const float* old_v, int64_t k,
                                          int64_t r, uint32_t* new_idx, float* new_m, float* new_v,
                                          usaf_rigl_stats* stats, void* ws, size_t ws_bytes,
                                          hipStream_t stream) {
  USAF_TRY(check_shape(shape));
  const int64_t N = n_weights(*shape);
  if (k < 0 || r < 0 || k > N || r > k || r > N - k) return USAF_ERR_INVALID_ARG;
  if (!grad || !Wflat || !old_idx || !old_m || !old_v || !new_idx || !new_m || !new_v)
    return USAF_ERR_INVALID_ARG;
  const WsRigl L = ws_rigl(N, k);
  if (!ws || ws_bytes < L.total) return USAF_ERR_WORKSPACE;
  char* w = static_cast<char*>(ws);
  uint32_t* dpos = reinterpret_cast<uint32_t*>(w + L.dpos);
  uint32_t* grown = reinterpret_cast<uint32_t*>(w + L.grown);
  uint32_t* fresh = reinterpret_cast<uint32_t*>(w + L.fresh);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(w + L.cnt);
  char* tws = w + L.topk;
  // drop: r smallest |w| among the active entries (positions into old_idx)
  if (shape->act == USAF_BF16)
    USAF_TRY(topk_run(KeyDropBf16{static_cast<const bf16_t*>(Wflat), old_idx}, k, r, nullptr, 0,
                      dpos, nullptr, nullptr, tws, stream));
  else
    USAF_TRY(topk_run(KeyDropF32{static_cast<const float*>(Wflat), old_idx}, k, r, nullptr, 0,
                      dpos, nullptr, nullptr, tws, stream));
  // grow: r largest |g| outside the active set
  USAF_TRY(topk_run(KeyGrad{grad}, N, r, old_idx, k, grown, nullptr, nullptr, tws, stream));
  timer_begin(USAF_K_RIGL_MERGE, stream);
  if (k > 0) {
    hipLaunchKernelGGL(rigl_place_kept_kernel, dim3(unsigned(ceil_div(k, 256))), dim3(256), 0,
                       stream, old_idx, old_m, old_v, k, dpos, grown, r, new_idx, new_m, new_v);
    USAF_LAUNCH_CHECK();
  }
  if (r > 0) {
    hipLaunchKernelGGL(rigl_place_grown_kernel, dim3(unsigned(ceil_div(r, 256))), dim3(256), 0,
                       stream, old_idx, k, dpos, grown, r, new_idx, new_m, new_v);
    USAF_LAUNCH_CHECK();
  }
  timer_end(USAF_K_RIGL_MERGE, stream);
  if (stats) {
    hipLaunchKernelGGL(rigl_stats_init_kernel, dim3(1), dim3(1), 0, stream, cnt);
    USAF_LAUNCH_CHECK();
    if (k > 0) {
      USAF_TRY(topk_run(KeyGrad{grad}, N, k, nullptr, 0, fresh, nullptr, nullptr, tws, stream));
      hipLaunchKernelGGL(rigl_novelty_kernel, dim3(unsigned(ceil_div(k, 256))), dim3(256), 0,
                         stream, fresh, old_idx, k, cnt);
      USAF_LAUNCH_CHECK();
    }
    hipLaunchKernelGGL(rigl_stats_kernel, dim3(1), dim3(1), 0, stream, cnt, r, stats);
    USAF_LAUNCH_CHECK();
  }
  return USAF_OK;
}

namespace usaf {
size_t rigl_ws_bytes(int64_t N, int64_t k) { return ws_rigl(N, k).total; }
}  // namespace usaf
