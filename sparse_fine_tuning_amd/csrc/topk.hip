// Global top-k by |grad| (importance selection) and RigL drop / grow.
//
// Method: the usaf README ("tsuyu122/usaf"), "how it works": the importance
// phase keeps the ~0.5% of expert weights with the largest gradient
// magnitude; RigL reselection replaces part of the active set every 50 steps
// (RESELECT_EVERY in the env-var table).
//
// Ranking: by the 63-bit composite (key << 32) | (2^32 - 1 - index), key =
// the 31-bit magnitude (|g| as fp32 bits, or an inverted |w| for RigL's
// drop), i.e. magnitude descending, then index ascending.  Composites are
// unique, so the top-k set is unique.
//
// Selection is an exact radix select done with two full reads:
//   A  histogram of the top 11 key bits (64 privatised global copies, so the
//      few hot bins do not serialise every block's atomics) -> the bin b0
//      holding the k-th element;
//   B  per 4096-key chunk, in the chunk's own buffer regions: the indices of
//      the keys above b0 (all selected) and the indices and keys of the keys
//      in b0 (the candidates);
//   -  the remaining 52 composite bits are resolved on the stored candidate
//      keys alone (five histogram/select rounds) -> the exact k-th composite;
//   C  per chunk, the selected indices (the above list and the candidates at
//      or above the k-th composite) are merged in index order through a
//      4096-bit LDS mask and written at offsets from a scan of the per-chunk
//      counts.
// Output indices are therefore ascending.
#include "common.hpp"
#include "moe_internal.hpp"
#include "timing.hpp"

namespace usaf {

constexpr int kTopkTile = 16384;  // elements per block in the full passes
constexpr int kTopkPer = kTopkTile / 256;
constexpr int kChunk = kTopkTile / 4;  // elements per wave (4 waves per block)
constexpr int kTopkBins = 2048;
constexpr int kHistCopies = 64;

// ---------------------------------------------------------------------------
// Key sources: operator()(i, key) -> false when element i is not eligible.
// ---------------------------------------------------------------------------
struct KeyGrad {
  const float* g;
  __device__ __forceinline__ bool operator()(int64_t i, uint32_t& key) const {
    key = __float_as_uint(g[i]) & 0x7fffffffu;
    return true;
  }
};
// Smaller |w| ranks first (RigL drop).  bf16 magnitude bits are 15 wide;
// they are placed in key bits 30..16 (an order-preserving shift) so the
// first radix digit sees them.
struct KeyDropBf16 {
  const bf16_t* W;
  const uint32_t* idx;
  __device__ __forceinline__ bool operator()(int64_t i, uint32_t& key) const {
    key = (0x7fffu - (uint32_t(W[idx[i]]) & 0x7fffu)) << 16;
    return true;
  }
};
struct KeyDropF32 {
  const float* W;
  const uint32_t* idx;
  __device__ __forceinline__ bool operator()(int64_t i, uint32_t& key) const {
    key = 0x7fffffffu - (__float_as_uint(W[idx[i]]) & 0x7fffffffu);
    return true;
  }
};
// |g| at list[i], eligible where flag[i] != 0 (RigL grow among a fresh top-k).
struct KeyListGrad {
  const float* g;
  const uint32_t* list;
  const uint8_t* flag;
  __device__ __forceinline__ bool operator()(int64_t i, uint32_t& key) const {
    key = __float_as_uint(g[list[i]]) & 0x7fffffffu;
    return flag[i] != 0;
  }
};

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t i) {
  return (uint64_t(key) << 32) | uint64_t(0xffffffffu - i);
}

__device__ __forceinline__ int64_t lower_bound_u32(const uint32_t* a, int64_t n, uint64_t v) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (uint64_t(a[mid]) < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Marks, in an LDS bitmap of kTopkTile bits, the excluded indices (a sorted
// list) inside the tile starting at i0.  Ends with a barrier.
__device__ __forceinline__ void mark_excluded(uint32_t* bm, const uint32_t* ex, int64_t nex,
                                              int64_t i0) {
  __shared__ int64_t range[2];
  for (int w = threadIdx.x; w < kTopkTile / 32; w += blockDim.x) bm[w] = 0;
  if (ex && threadIdx.x < 2)
    range[threadIdx.x] = lower_bound_u32(ex, nex, uint64_t(i0) + threadIdx.x * kTopkTile);
  __syncthreads();
  if (ex) {
    for (int64_t q = range[0] + threadIdx.x; q < range[1]; q += blockDim.x) {
      const int64_t l = int64_t(ex[q]) - i0;
      if (l >= 0 && l < kTopkTile) atomicOr(&bm[l >> 5], 1u << (l & 31));
    }
  }
  __syncthreads();
}
__device__ __forceinline__ bool is_marked(const uint32_t* bm, int l) {
  return (bm[l >> 5] >> (l & 31)) & 1u;
}

// Keys of elements i..i+3 (eligibility in `ok`), with the exclusion bitmap
// of the tile (local offset l).
template <class KF>
__device__ __forceinline__ void keys4(const KF& key, int64_t i, int64_t n, const uint32_t* bm,
                                      int l, uint32_t (&kv)[4], bool (&ok)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    ok[u] = i + u < n && !is_marked(bm, l + u) && key(i + u, kv[u]);
  }
}
template <>
__device__ __forceinline__ void keys4<KeyGrad>(const KeyGrad& key, int64_t i, int64_t n,
                                               const uint32_t* bm, int l, uint32_t (&kv)[4],
                                               bool (&ok)[4]) {
  if (i + 3 < n) {
    const uint4 v = *reinterpret_cast<const uint4*>(key.g + i);
    kv[0] = v.x & 0x7fffffffu; kv[1] = v.y & 0x7fffffffu;
    kv[2] = v.z & 0x7fffffffu; kv[3] = v.w & 0x7fffffffu;
#pragma unroll
    for (int u = 0; u < 4; ++u) ok[u] = !is_marked(bm, l + u);
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) ok[u] = i + u < n && !is_marked(bm, l + u) && key(i + u, kv[u]);
  }
}

// Workspace words (u32) of one selection.
enum {
  ST_B0 = 0,        // threshold bin of the top 11 key bits
  ST_KREM = 1,      // how many of the current prefix's elements are still to take
  ST_NCAND = 2,     // candidates in bin b0
  ST_PLO = 3,       // composite prefix (low, high words)
  ST_PHI = 4,
  ST_WORDS = 64
};

struct TopkWs {
  uint32_t* hist;   // [kHistCopies][kBins]
  uint32_t* chist;  // [kBins] candidate rounds
  uint32_t* st;     // [ST_WORDS]
  uint32_t* cnt;    // [nchunks] selected per wave chunk (then exclusive offsets)
  uint32_t* ccnt;   // [nchunks] candidates per wave chunk
  uint32_t* acnt;   // [nchunks] keys above b0 per wave chunk
  uint32_t* cand;   // [n] candidate indices, chunk c's at [c*kChunk, c*kChunk + ccnt[c])
  uint32_t* ckey;   // [n] their keys, same layout
  uint32_t* above;  // [n] indices above b0, chunk c's at [c*kChunk, c*kChunk + acnt[c])
  int64_t nchunks;
};

static size_t al(size_t x) { return align256(x); }
size_t topk_ws_bytes(int64_t n) {
  const int64_t nt = ceil_div(n > 0 ? n : 1, kChunk);
  return al(size_t(kHistCopies) * kTopkBins * 4) + al(kTopkBins * 4) + al(ST_WORDS * 4) +
         3 * al(size_t(nt) * 4) + 3 * al(size_t(nt) * kChunk * 4);
}
static TopkWs topk_ws(char* w, int64_t n) {
  const int64_t nt = ceil_div(n > 0 ? n : 1, kChunk);
  TopkWs t;
  t.hist = reinterpret_cast<uint32_t*>(w);
  w += al(size_t(kHistCopies) * kTopkBins * 4);
  t.chist = reinterpret_cast<uint32_t*>(w);
  w += al(kTopkBins * 4);
  t.st = reinterpret_cast<uint32_t*>(w);
  w += al(ST_WORDS * 4);
  t.cnt = reinterpret_cast<uint32_t*>(w);
  w += al(size_t(nt) * 4);
  t.ccnt = reinterpret_cast<uint32_t*>(w);
  w += al(size_t(nt) * 4);
  t.acnt = reinterpret_cast<uint32_t*>(w);
  w += al(size_t(nt) * 4);
  t.cand = reinterpret_cast<uint32_t*>(w);
  w += al(size_t(nt) * kChunk * 4);
  t.ckey = reinterpret_cast<uint32_t*>(w);
  w += al(size_t(nt) * kChunk * 4);
  t.above = reinterpret_cast<uint32_t*>(w);
  t.nchunks = nt;
  return t;
}

// A gate lets RigL enqueue a selection that runs only when a device flag
// asks for it: with `gate` set and *gate == 0 every kernel returns at once.
__device__ __forceinline__ bool gated_off(const uint32_t* gate) { return gate && *gate == 0; }

__global__ __launch_bounds__(256) void topk_init_kernel(TopkWs w, uint32_t k, const uint32_t* gate) {
  if (gated_off(gate)) return;
  for (int b = blockIdx.x * 256 + threadIdx.x; b < kHistCopies * kTopkBins; b += gridDim.x * 256)
    w.hist[b] = 0;
  if (blockIdx.x == 0) {
    for (int b = threadIdx.x; b < kTopkBins; b += 256) w.chist[b] = 0;
    if (threadIdx.x < ST_WORDS) w.st[threadIdx.x] = 0;
    __syncthreads();
    if (threadIdx.x == 0) w.st[ST_KREM] = k;
  }
}

// Pass A: histogram of key >> 20 over eligible elements.  Each wave reads a
// contiguous chunk of kChunk keys, four consecutive per lane (16-byte loads).
template <class KF>
__global__ __launch_bounds__(256) void topk_pass_a_kernel(KF key, int64_t n, const uint32_t* ex,
                                                          int64_t nex, TopkWs w,
                                                          const uint32_t* gate) {
  if (gated_off(gate)) return;
  __shared__ uint32_t h[kTopkBins];
  __shared__ uint32_t bm[kTopkTile / 32];
  for (int b = threadIdx.x; b < kTopkBins; b += 256) h[b] = 0;
  const int64_t i0 = int64_t(blockIdx.x) * kTopkTile;
  mark_excluded(bm, ex, nex, i0);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int lbase = wid * kChunk;
  for (int r = 0; r < kChunk / 256; ++r) {
    const int l = lbase + r * 256 + lane * 4;
    uint32_t kv[4];
    bool ok[4];
    keys4(key, i0 + l, n, bm, l, kv, ok);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (ok[u]) atomicAdd(&h[kv[u] >> 20], 1u);
  }
  __syncthreads();
  uint32_t* dst = w.hist + size_t(blockIdx.x % kHistCopies) * kTopkBins;
  for (int b = threadIdx.x; b < kTopkBins; b += 256)
    if (h[b]) atomicAdd(&dst[b], h[b]);
}

// Finds, in a histogram `hist` of nb bins (summed over `copies` copies
// spaced `stride` apart), the bin holding the krem-th element from the top.
// Called by every thread of the block (threads >= 256 only join barriers);
// returns (bin, krem within the bin).
__device__ __forceinline__ void find_bin(const uint32_t* hist, int nb, int copies, int stride,
                                         uint32_t krem, int& bin_out, uint32_t& krem_out) {
  __shared__ uint32_t csum[256];
  __shared__ int sbin;
  __shared__ uint32_t skrem;
  const int per = (nb + 255) / 256;
  if (threadIdx.x < 256) {
    uint32_t s = 0;
    for (int q = 0; q < per; ++q) {
      const int b = threadIdx.x * per + q;
      if (b < nb)
        for (int c = 0; c < copies; ++c) s += hist[size_t(c) * stride + b];
    }
    csum[threadIdx.x] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t above = 0;
    int c = 255;
    for (; c > 0; --c) {
      if (above + csum[c] >= krem) break;
      above += csum[c];
    }
    int b = min(nb - 1, c * per + per - 1);
    for (; b > c * per; --b) {
      uint32_t hb = 0;
      for (int cc = 0; cc < copies; ++cc) hb += hist[size_t(cc) * stride + b];
      if (above + hb >= krem) break;
      above += hb;
    }
    sbin = b;
    skrem = krem - above;
  }
  __syncthreads();
  bin_out = sbin;
  krem_out = skrem;
}

// Sums the privatised copies into chist, then selects the bin (1024 threads).
__global__ __launch_bounds__(1024) void topk_select_a_kernel(TopkWs w, const uint32_t* gate) {
  if (gated_off(gate)) return;
  for (int b = threadIdx.x; b < kTopkBins; b += 1024) {
    uint32_t s = 0;
#pragma unroll 8
    for (int c = 0; c < kHistCopies; ++c) s += w.hist[size_t(c) * kTopkBins + b];
    w.chist[b] = s;
  }
  __syncthreads();
  int b;
  uint32_t krem;
  find_bin(w.chist, kTopkBins, 1, 0, w.st[ST_KREM], b, krem);
  __syncthreads();
  for (int q = threadIdx.x; q < kTopkBins; q += 1024) w.chist[q] = 0;
  if (threadIdx.x == 0) {
    w.st[ST_B0] = uint32_t(b);
    w.st[ST_KREM] = krem;
    w.st[ST_PHI] = uint32_t(b) << 20;  // composite bits 62..52
    w.st[ST_PLO] = 0;
  }
}

// Wave-wide exclusive prefix of a per-lane count, and the wave total.
__device__ __forceinline__ uint32_t wave_excl(uint32_t v, uint32_t& total) {
  const int lane = threadIdx.x & 63;
  uint32_t inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t u = __shfl_up(inc, d, 64);
    if (lane >= d) inc += u;
  }
  total = __shfl(inc, 63, 64);
  return inc - v;
}

// Pass B: per wave chunk, the indices of the eligible keys above b0 and the
// indices and keys of those in b0 (the candidates), each in the chunk's own
// region of its buffer, in index order -- no shared counter.
template <class KF>
__global__ __launch_bounds__(256) void topk_pass_b_kernel(KF key, int64_t n, const uint32_t* ex,
                                                          int64_t nex, TopkWs w,
                                                          const uint32_t* gate) {
  if (gated_off(gate)) return;
  __shared__ uint32_t bm[kTopkTile / 32];
  const int64_t i0 = int64_t(blockIdx.x) * kTopkTile;
  mark_excluded(bm, ex, nex, i0);
  const uint32_t b0 = w.st[ST_B0];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int lbase = wid * kChunk;
  if (i0 + lbase >= n) return;  // uniform per wave; no block barrier follows
  const int64_t chunk = int64_t(blockIdx.x) * 4 + wid;
  uint32_t* cdst = w.cand + chunk * kChunk;
  uint32_t* kdst = w.ckey + chunk * kChunk;
  uint32_t* adst = w.above + chunk * kChunk;
  uint32_t apos = 0, pos = 0;
  for (int r = 0; r < kChunk / 256; ++r) {
    const int l = lbase + r * 256 + lane * 4;
    uint32_t kv[4];
    bool ok[4];
    keys4(key, i0 + l, n, bm, l, kv, ok);
    bool c[4], a[4];
    uint32_t mine = 0, mina = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t d = kv[u] >> 20;
      a[u] = ok[u] && d > b0;
      c[u] = ok[u] && d == b0;
      mine += c[u];
      mina += a[u];
    }
    uint32_t tot, tota;
    uint32_t p = pos + wave_excl(mine, tot);
    uint32_t q = apos + wave_excl(mina, tota);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (c[u]) {
        cdst[p] = uint32_t(i0 + l + u);
        kdst[p] = kv[u];
        ++p;
      }
      if (a[u]) adst[q++] = uint32_t(i0 + l + u);
    }
    pos += tot;
    apos += tota;
  }
  if (lane == 0) {
    w.cnt[chunk] = apos;
    w.acnt[chunk] = apos;
    w.ccnt[chunk] = pos;
  }
}

// Candidate rounds: histogram of composite bits [shift, shift+width) over
// candidates matching the prefix's higher bits (one wave per chunk region).
template <class KF>
__global__ __launch_bounds__(256) void topk_cand_hist_kernel(KF key, TopkWs w, int shift,
                                                             int width, const uint32_t* gate) {
  if (gated_off(gate)) return;
  __shared__ uint32_t h[kTopkBins];
  for (int b = threadIdx.x; b < kTopkBins; b += 256) h[b] = 0;
  __syncthreads();
  const uint64_t prefix = (uint64_t(w.st[ST_PHI]) << 32) | w.st[ST_PLO];
  const int top = shift + width;  // bits >= top are fixed by the prefix
  const uint32_t dmask = (1u << width) - 1u;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  for (int64_t c = int64_t(blockIdx.x) * 4 + wid; c < w.nchunks; c += int64_t(gridDim.x) * 4) {
    const uint32_t m = w.ccnt[c];
    const uint32_t* src = w.cand + c * kChunk;
    const uint32_t* ksrc = w.ckey + c * kChunk;
    for (uint32_t j = lane; j < m; j += 64) {
      const uint64_t cp = composite(ksrc[j], src[j]);
      if ((cp >> top) == (prefix >> top)) atomicAdd(&h[uint32_t(cp >> shift) & dmask], 1u);
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b <= int(dmask); b += 256)
    if (h[b]) atomicAdd(&w.chist[b], h[b]);
}

__global__ __launch_bounds__(256) void topk_cand_select_kernel(TopkWs w, int shift, int width,
                                                               const uint32_t* gate) {
  if (gated_off(gate)) return;
  int b;
  uint32_t krem;
  find_bin(w.chist, 1 << width, 1, 0, w.st[ST_KREM], b, krem);
  __syncthreads();
  for (int q = threadIdx.x; q < (1 << width); q += 256) w.chist[q] = 0;
  if (threadIdx.x == 0) {
    const uint64_t p = ((uint64_t(w.st[ST_PHI]) << 32) | w.st[ST_PLO]) | (uint64_t(b) << shift);
    w.st[ST_PHI] = uint32_t(p >> 32);
    w.st[ST_PLO] = uint32_t(p);
    w.st[ST_KREM] = krem;
  }
}

// Adds each chunk's selected candidates (composite >= the k-th) to its count.
template <class KF>
__global__ __launch_bounds__(256) void topk_cand_count_kernel(KF key, TopkWs w, const uint32_t* gate) {
  if (gated_off(gate)) return;
  const uint64_t theta = (uint64_t(w.st[ST_PHI]) << 32) | w.st[ST_PLO];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  for (int64_t c = int64_t(blockIdx.x) * 4 + wid; c < w.nchunks; c += int64_t(gridDim.x) * 4) {
    const uint32_t m = w.ccnt[c];
    if (m == 0) continue;
    const uint32_t* src = w.cand + c * kChunk;
    const uint32_t* ksrc = w.ckey + c * kChunk;
    uint32_t nsel = 0;
    for (uint32_t j0 = 0; j0 < m; j0 += 64) {
      const uint32_t j = j0 + lane;
      bool sel = false;
      if (j < m) sel = composite(ksrc[j], src[j]) >= theta;
      nsel += __popcll(__ballot(sel));
    }
    if (lane == 0) w.cnt[c] += nsel;
  }
}

// In-place exclusive scan of n u32 values by one block of 1024 threads
// (coalesced 1024-wide segments, carried across segments).
__global__ __launch_bounds__(1024) void scan_u32_kernel(uint32_t* __restrict__ a, int64_t n,
                                                        const uint32_t* gate) {
  if (gated_off(gate)) return;
  __shared__ uint32_t wsum[16];
  __shared__ uint32_t carry_s;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();
  for (int64_t b = 0; b < n; b += 1024) {
    const int64_t i = b + threadIdx.x;
    const uint32_t v = i < n ? a[i] : 0u;
    uint32_t inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t u = __shfl_up(inc, d, 64);
      if (lane >= d) inc += u;
    }
    if (lane == 63) wsum[wid] = inc;
    __syncthreads();
    uint32_t wb = 0, tot = 0;
    for (int q = 0; q < 16; ++q) {
      if (q < wid) wb += wsum[q];
      tot += wsum[q];
    }
    const uint32_t carry = carry_s;
    if (i < n) a[i] = carry + wb + inc - v;
    __syncthreads();
    if (threadIdx.x == 0) carry_s = carry + tot;
    __syncthreads();
  }
}

// Pass C: per wave chunk, the above-b0 indices and the candidates at or
// above the k-th composite are marked in a 4096-bit LDS mask (chunk-local
// offsets) and emitted in index order at the chunk's scanned offset.
__global__ __launch_bounds__(256) void topk_pass_c_kernel(TopkWs w, uint32_t* __restrict__ out_idx,
                                                          float* __restrict__ out_val,
                                                          const float* __restrict__ valsrc,
                                                          const uint32_t* gate) {
  if (gated_off(gate)) return;
  __shared__ uint64_t mask[4][kChunk / 64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t c = int64_t(blockIdx.x) * 4 + wid;
  if (c >= w.nchunks) return;  // uniform per wave; no block barrier follows
  uint64_t* mk = mask[wid];
  mk[lane] = 0;
  const uint64_t theta = (uint64_t(w.st[ST_PHI]) << 32) | w.st[ST_PLO];
  const uint32_t base = uint32_t(c * kChunk);
  const uint32_t na = w.acnt[c], nc = w.ccnt[c];
  const uint32_t* asrc = w.above + c * kChunk;
  const uint32_t* csrc = w.cand + c * kChunk;
  const uint32_t* ksrc = w.ckey + c * kChunk;
  __builtin_amdgcn_wave_barrier();
  for (uint32_t j = lane; j < na; j += 64) {
    const uint32_t l = asrc[j] - base;
    atomicOr(reinterpret_cast<unsigned long long*>(&mk[l >> 6]), 1ull << (l & 63));
  }
  for (uint32_t j = lane; j < nc; j += 64) {
    const uint32_t i = csrc[j];
    if (composite(ksrc[j], i) >= theta) {
      const uint32_t l = i - base;
      atomicOr(reinterpret_cast<unsigned long long*>(&mk[l >> 6]), 1ull << (l & 63));
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0);
  uint64_t bits = mk[lane];
  uint32_t tot;
  uint32_t p = w.cnt[c] + wave_excl(uint32_t(__popcll(bits)), tot);
  while (bits) {
    const int b = __builtin_ctzll(bits);
    bits &= bits - 1;
    const uint32_t i = base + uint32_t(lane) * 64u + uint32_t(b);
    out_idx[p] = i;
    if (out_val) out_val[p] = valsrc[i];
    ++p;
  }
}

// Enqueue one selection: the k eligible elements ranked first by (key desc,
// index asc) among n (minus the excluded), written ascending to out_idx.
template <class KF>
usaf_status topk_run(KF key, int64_t n, int64_t k, const uint32_t* ex, int64_t nex,
                     uint32_t* out_idx, float* out_val, const float* valsrc, char* ws,
                     hipStream_t st, const uint32_t* gate = nullptr) {
  if (k == 0 || n == 0) return USAF_OK;
  const int64_t ntiles = ceil_div(n, kTopkTile);
  const TopkWs w = topk_ws(ws, n);
  const dim3 blk{256, 1, 1}, grid{unsigned(ntiles), 1, 1};
  const unsigned cgrid = 1024;
  timer_begin(USAF_K_TOPK, st);
  hipLaunchKernelGGL(topk_init_kernel, dim3(64), blk, 0, st, w, uint32_t(k), gate);
  hipLaunchKernelGGL(topk_pass_a_kernel<KF>, grid, blk, 0, st, key, n, ex, nex, w, gate);
  hipLaunchKernelGGL(topk_select_a_kernel, dim3(1), dim3(1024), 0, st, w, gate);
  hipLaunchKernelGGL(topk_pass_b_kernel<KF>, grid, blk, 0, st, key, n, ex, nex, w, gate);
  // composite bits 51..0 in rounds of 11, 11, 11, 11, 8
  const int shifts[5] = {41, 30, 19, 8, 0}, widths[5] = {11, 11, 11, 11, 8};
  for (int q = 0; q < 5; ++q) {
    hipLaunchKernelGGL(topk_cand_hist_kernel<KF>, dim3(cgrid), blk, 0, st, key, w, shifts[q],
                       widths[q], gate);
    hipLaunchKernelGGL(topk_cand_select_kernel, dim3(1), blk, 0, st, w, shifts[q], widths[q], gate);
  }
  hipLaunchKernelGGL(topk_cand_count_kernel<KF>, dim3(cgrid), blk, 0, st, key, w, gate);
  hipLaunchKernelGGL(scan_u32_kernel, dim3(1), dim3(1024), 0, st, w.cnt, w.nchunks, gate);
  hipLaunchKernelGGL(topk_pass_c_kernel, grid, blk, 0, st, w, out_idx, out_val, valsrc, gate);
  timer_end(USAF_K_TOPK, st);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

// ---------------------------------------------------------------------------
// Sorted-list membership by LDS merge: for each element of a (sorted) query
// list, whether it occurs in a sorted reference list.  Each block takes 256
// queries, stages the reference range they span in LDS, and searches there.
// ---------------------------------------------------------------------------
constexpr int kMergeCap = 4096;

__global__ __launch_bounds__(256) void member_kernel(const uint32_t* __restrict__ q, int64_t nq,
                                                     const uint32_t* __restrict__ ref, int64_t nref,
                                                     uint8_t* __restrict__ absent_flag,
                                                     uint32_t* __restrict__ n_absent) {
  __shared__ uint32_t seg[kMergeCap];
  __shared__ int64_t rng[2];
  __shared__ uint32_t wsum[4];
  const int64_t b0 = int64_t(blockIdx.x) * 256;
  const int64_t i = b0 + threadIdx.x;
  const int64_t last = min(nq, b0 + 256) - 1;
  if (threadIdx.x < 2) {
    const uint64_t v = threadIdx.x == 0 ? uint64_t(q[b0]) : uint64_t(q[last]) + 1;
    rng[threadIdx.x] = lower_bound_u32(ref, nref, v);
  }
  __syncthreads();
  const int64_t lo = rng[0], len = rng[1] - rng[0];
  const bool staged = len <= kMergeCap;
  if (staged)
    for (int64_t j = threadIdx.x; j < len; j += 256) seg[j] = ref[lo + j];
  __syncthreads();
  bool absent = false;
  if (i < nq) {
    const uint32_t v = q[i];
    bool hit;
    if (staged) {
      int a = 0, c = int(len);
      while (a < c) {
        const int mid = (a + c) >> 1;
        if (seg[mid] < v) a = mid + 1; else c = mid;
      }
      hit = a < len && seg[a] == v;
    } else {
      const int64_t p = lo + lower_bound_u32(ref + lo, len, v);
      hit = p < lo + len && ref[p] == v;
    }
    absent = !hit;
    if (absent_flag) absent_flag[i] = absent ? 1 : 0;
  }
  const uint64_t bal = __ballot(absent);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = __popcll(bal);
  __syncthreads();
  if (threadIdx.x == 0 && n_absent) {
    const uint32_t t = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (t) atomicAdd(n_absent, t);
  }
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

// grown[i] = fresh[gpos[i]]  (positions ascending -> indices ascending)
__global__ __launch_bounds__(256) void gather_u32_kernel(const uint32_t* __restrict__ src,
                                                         const uint32_t* __restrict__ pos,
                                                         int64_t n, uint32_t* __restrict__ dst,
                                                         const uint32_t* gate) {
  if (gated_off(gate)) return;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[pos[i]];
}

// gates[0] = (new entries in the fresh top-k >= r), gates[1] = !gates[0].
__global__ void rigl_gate_kernel(const uint32_t* __restrict__ novel, int64_t r,
                                 uint32_t* __restrict__ gates) {
  const bool fresh_ok = int64_t(*novel) >= r;
  gates[0] = fresh_ok ? 1u : 0u;
  gates[1] = fresh_ok ? 0u : 1u;
}

__global__ void rigl_stats_init_kernel(uint32_t* cnt) { *cnt = 0; }

__global__ void rigl_stats_kernel(const uint32_t* __restrict__ cnt, int64_t r,
                                  usaf_rigl_stats* __restrict__ stats) {
  stats->n_drop = r;
  stats->n_grow = r;
  stats->topk_new_vs_old = int64_t(*cnt);
}

struct WsRigl {
  size_t topk, dpos, grown, gpos, fresh, flag, cnt, total;
};
static WsRigl ws_rigl(int64_t N, int64_t k) {
  WsRigl L;
  L.topk = 0;
  const size_t t = topk_ws_bytes(N > k ? N : k);
  const size_t kb = align256(size_t(k) * 4 + 4);
  L.dpos = align256(t);
  L.grown = L.dpos + kb;
  L.gpos = L.grown + kb;
  L.fresh = L.gpos + kb;
  L.flag = L.fresh + kb;
  L.cnt = L.flag + align256(size_t(k) + 4);
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
  if (reinterpret_cast<uintptr_t>(grad) & 15) return USAF_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < topk_ws_bytes(n)) return USAF_ERR_WORKSPACE;
  return topk_run(KeyGrad{grad}, n, k, n_exclude ? exclude : nullptr, n_exclude, out_idx, out_val,
                  grad, static_cast<char*>(ws), stream);
}

// RigL reselection.  The grow set G (the r best outside the old set) is
// taken from the fresh top-k whenever at least r of its entries are outside
// the old set -- then every element of G is in the fresh top-k, since any
// entry outside the fresh top-k is outranked by those r -- and otherwise
// from a full selection that excludes the old set.  Which one runs is
// decided on the device (gated kernels), without a host round trip.
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
  if (reinterpret_cast<uintptr_t>(grad) & 15) return USAF_ERR_UNSUPPORTED;
  const WsRigl L = ws_rigl(N, k);
  if (!ws || ws_bytes < L.total) return USAF_ERR_WORKSPACE;
  if (k == 0) return USAF_OK;
  char* w = static_cast<char*>(ws);
  uint32_t* dpos = reinterpret_cast<uint32_t*>(w + L.dpos);
  uint32_t* grown = reinterpret_cast<uint32_t*>(w + L.grown);
  uint32_t* gpos = reinterpret_cast<uint32_t*>(w + L.gpos);
  uint32_t* fresh = reinterpret_cast<uint32_t*>(w + L.fresh);
  uint8_t* flag = reinterpret_cast<uint8_t*>(w + L.flag);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(w + L.cnt);  // [0] novel count, [1..2] gates
  char* tws = w + L.topk;
  // fresh top-k of |g| and which of its entries are new
  USAF_TRY(topk_run(KeyGrad{grad}, N, k, nullptr, 0, fresh, nullptr, nullptr, tws, stream));
  hipLaunchKernelGGL(rigl_stats_init_kernel, dim3(1), dim3(1), 0, stream, cnt);
  hipLaunchKernelGGL(member_kernel, dim3(unsigned(ceil_div(k, 256))), dim3(256), 0, stream, fresh,
                     k, old_idx, k, flag, cnt);
  USAF_LAUNCH_CHECK();
  if (r > 0) {
    hipLaunchKernelGGL(rigl_gate_kernel, dim3(1), dim3(1), 0, stream, cnt, r, cnt + 1);
    // grow from the fresh top-k (when it holds >= r new entries) ...
    USAF_TRY(topk_run(KeyListGrad{grad, fresh, flag}, k, r, nullptr, 0, gpos, nullptr, nullptr,
                      tws, stream, cnt + 1));
    hipLaunchKernelGGL(gather_u32_kernel, dim3(unsigned(ceil_div(r, 256))), dim3(256), 0, stream,
                       fresh, gpos, r, grown, cnt + 1);
    // ... or from everything outside the old set
    USAF_TRY(topk_run(KeyGrad{grad}, N, r, old_idx, k, grown, nullptr, nullptr, tws, stream,
                      cnt + 2));
    // drop: r smallest |w| among the active entries (positions into old_idx)
    if (shape->act == USAF_BF16)
      USAF_TRY(topk_run(KeyDropBf16{static_cast<const bf16_t*>(Wflat), old_idx}, k, r, nullptr, 0,
                        dpos, nullptr, nullptr, tws, stream));
    else
      USAF_TRY(topk_run(KeyDropF32{static_cast<const float*>(Wflat), old_idx}, k, r, nullptr, 0,
                        dpos, nullptr, nullptr, tws, stream));
  }
  timer_begin(USAF_K_RIGL_MERGE, stream);
  hipLaunchKernelGGL(rigl_place_kept_kernel, dim3(unsigned(ceil_div(k, 256))), dim3(256), 0,
                     stream, old_idx, old_m, old_v, k, dpos, grown, r, new_idx, new_m, new_v);
  if (r > 0)
    hipLaunchKernelGGL(rigl_place_grown_kernel, dim3(unsigned(ceil_div(r, 256))), dim3(256), 0,
                       stream, old_idx, k, dpos, grown, r, new_idx, new_m, new_v);
  timer_end(USAF_K_RIGL_MERGE, stream);
  USAF_LAUNCH_CHECK();
  if (stats) {
    hipLaunchKernelGGL(rigl_stats_kernel, dim3(1), dim3(1), 0, stream, cnt, r, stats);
    USAF_LAUNCH_CHECK();
  }
  return USAF_OK;
}

namespace usaf {
size_t rigl_ws_bytes(int64_t N, int64_t k) { return ws_rigl(N, k).total; }
}  // namespace usaf
