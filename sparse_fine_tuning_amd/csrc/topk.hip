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
//
// Over a whole gradient (no exclusion) pass A is replaced by a sample: the
// first 64 keys of every 4096 are histogrammed on 22 key bits (two levels of
// 11), and the key at which the sample holds 1.25x its share of k (plus 16)
// is taken as a threshold.  One full read (pass B1) then stores every key at
// or above it as a candidate; the candidates are made contiguous (with a
// histogram of their top key bits) and the exact k-th composite is resolved
// on them as above, then written
// out in index order.  The result is exact whatever the sample says: if
// fewer than k keys reach the threshold, pass B1 runs again with every key a
// candidate (a device-gated retry, no host round trip).
#include <algorithm>
#include <cmath>
#include <type_traits>

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
    key = (0x7fffu - (uint32_t(W[idx ? idx[i] : i]) & 0x7fffu)) << 16;
    return true;
  }
};
struct KeyDropF32 {
  const float* W;
  const uint32_t* idx;
  __device__ __forceinline__ bool operator()(int64_t i, uint32_t& key) const {
    key = 0x7fffffffu - (__float_as_uint(W[idx ? idx[i] : i]) & 0x7fffffffu);
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

// Keys gathered once into a compact array; eligible where flag (nullable)
// is non-zero.  RigL's drop and grow selections over its k-entry lists read
// these instead of gathering from W or the gradient in every pass.
struct KeyArr {
  const uint32_t* key;
  const uint8_t* flag;
  __device__ __forceinline__ bool operator()(int64_t i, uint32_t& k) const {
    k = key[i];
    return !flag || flag[i] != 0;
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

template <>
__device__ __forceinline__ void keys4<KeyArr>(const KeyArr& key, int64_t i, int64_t n,
                                              const uint32_t* bm, int l, uint32_t (&kv)[4],
                                              bool (&ok)[4]) {
  if (i + 3 < n) {  // i is a multiple of 4; the arrays are 16-byte aligned
    const uint4 v = *reinterpret_cast<const uint4*>(key.key + i);
    const uint32_t f = key.flag ? *reinterpret_cast<const uint32_t*>(key.flag + i) : 0x01010101u;
    kv[0] = v.x; kv[1] = v.y; kv[2] = v.z; kv[3] = v.w;
#pragma unroll
    for (int u = 0; u < 4; ++u) ok[u] = ((f >> (8 * u)) & 0xffu) != 0 && !is_marked(bm, l + u);
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) ok[u] = i + u < n && !is_marked(bm, l + u) && key(i + u, kv[u]);
  }
}

// Workspace words (u32) of one selection.
enum {
  ST_B0 = 0,        // threshold bin of the top 11 key bits
  ST_KREM = 1,      // how many of the current prefix's elements are still to take
  ST_NCAND = 2,     // candidates stored by the sampled pass
  ST_PLO = 3,       // composite prefix (low, high words)
  ST_PHI = 4,
  ST_BS = 5,        // sampled threshold bin (top 11 key bits)
  ST_RETRY = 6,     // 1 when the sampled threshold let fewer than k keys through
  ST_BSREM = 7,     // sampled keys still to count inside bin ST_BS
  ST_T = 8,         // sampled threshold key: keys >= it are candidates
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
  uint32_t* above;  // [n] indices above b0, chunk c's at [c*kChunk, c*kChunk + acnt[c]);
                    // the sampled pass keeps its candidates' indices here, contiguous
  uint32_t* cckey;  // [n] the sampled pass's candidate keys, contiguous
  uint32_t* bsum;   // [ceil(nchunks / kScanSeg) + 1] block sums of the count scan
  int64_t nchunks;
};

constexpr int kScanSeg = 2048;  // elements per block of the multi-block scan

static size_t al(size_t x) { return align256(x); }
size_t topk_ws_bytes(int64_t n) {
  const int64_t nt = ceil_div(n > 0 ? n : 1, kChunk);
  return al(size_t(kHistCopies) * kTopkBins * 4) + al(kTopkBins * 4) + al(ST_WORDS * 4) +
         3 * al(size_t(nt) * 4) + 4 * al(size_t(nt) * kChunk * 4) +
         al(size_t(ceil_div(nt, kScanSeg) + 1) * 4);
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
  w += al(size_t(nt) * kChunk * 4);
  t.cckey = reinterpret_cast<uint32_t*>(w);
  w += al(size_t(nt) * kChunk * 4);
  t.bsum = reinterpret_cast<uint32_t*>(w);
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
  // Scanning from the top bin down, the first bin at which the keys above it
  // plus its own reach krem; bin 0 when none does.  Group sums of `per`
  // bins first, then wave 0 finds the group and the bin within it with
  // suffix sums over lanes (no serial walk).
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
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    // suffix sums over the groups: lane l holds groups 4l..4l+3
    uint32_t g[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) g[j] = csum[4 * lane + j];
    const uint32_t s4 = (g[0] + g[1]) + (g[2] + g[3]);
    uint32_t v = s4;  // groups of lanes l.. 63
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t u = __shfl_down(v, d, 64);
      if (lane + d < 64) v += u;
    }
    // the highest group c >= 1 whose suffix (groups c..255) reaches krem
    uint32_t cum = v - s4;  // groups above this lane's
    int jc = -1;
    uint32_t above_c = 0;
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (jc < 0 && 4 * lane + j >= 1 && cum + g[j] >= krem) {
        jc = j;
        above_c = cum;
      }
      cum += g[j];
    }
    const uint64_t hit = __ballot(jc >= 0);
    int c;
    uint32_t above;
    if (hit) {
      const int lh = 63 - __clzll((long long)hit);
      c = 4 * lh + __shfl(jc, lh, 64);
      above = __shfl(above_c, lh, 64);
    } else {  // group 0, under every group above it
      c = 0;
      above = __shfl(v - (lane == 0 ? csum[0] : 0u), 0, 64);
    }
    // the bin within group c: bins c*per .. min(nb, c*per + per) - 1, the
    // lowest taken when no higher one reaches krem
    const int b0 = c * per;
    const int nbin = min(per, nb - b0);
    uint32_t hb = 0;
    if (lane < nbin)
      for (int cc = 0; cc < copies; ++cc) hb += hist[size_t(cc) * stride + b0 + lane];
    uint32_t w = hb;  // bins lane.. of the group
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t u = __shfl_down(w, d, 64);
      if (lane + d < 64) w += u;
    }
    const bool reach = lane >= 1 && lane < nbin && above + w >= krem;
    const uint64_t rb = __ballot(reach);
    const int jb = rb ? 63 - __clzll((long long)rb) : 0;
    const uint32_t wj = __shfl(w, jb, 64), hj = __shfl(hb, jb, 64);
    if (lane == 0) {
      sbin = min(b0 + jb, nb - 1);
      skrem = krem - (above + (wj - hj));
    }
  }
  __syncthreads();
  bin_out = sbin;
  krem_out = skrem;
}

// The privatised histogram copies summed into an LDS histogram by a block
// of 1024 threads: thread t sums 4 consecutive bins (one 16-byte load per
// copy) over half of the copies, all of its loads in flight together, and
// the two halves meet in LDS.  With clear, the copies are zeroed behind the
// loads.  Ends with a barrier.
__device__ __forceinline__ void sum_copies_lds(uint32_t* __restrict__ hist, uint32_t* hs, bool clear) {
  static_assert(kTopkBins == 2048 && kHistCopies % 2 == 0, "512 bin quads x 2 halves = 1024 threads");
  constexpr int kHalf = kHistCopies / 2;
  const int t = threadIdx.x, quad = t & 511, half = t >> 9;
  uint4* src = reinterpret_cast<uint4*>(hist) + size_t(half * kHalf) * (kTopkBins / 4) + quad;
  uint4 acc = make_uint4(0, 0, 0, 0);
#pragma unroll 16
  for (int c = 0; c < kHalf; ++c) {
    const uint4 v = src[size_t(c) * (kTopkBins / 4)];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  if (clear) {
#pragma unroll 16
    for (int c = 0; c < kHalf; ++c) src[size_t(c) * (kTopkBins / 4)] = make_uint4(0, 0, 0, 0);
  }
  uint4* hq = reinterpret_cast<uint4*>(hs);
  if (half == 0) hq[quad] = acc;
  __syncthreads();
  if (half == 1) {
    uint4 v = hq[quad];
    v.x += acc.x; v.y += acc.y; v.z += acc.z; v.w += acc.w;
    hq[quad] = v;
  }
  __syncthreads();
}

// Sums the privatised copies, then selects the bin (1024 threads).
__global__ __launch_bounds__(1024) void topk_select_a_kernel(TopkWs w, const uint32_t* gate) {
  if (gated_off(gate)) return;
  __shared__ __attribute__((aligned(16))) uint32_t hs[kTopkBins];
  sum_copies_lds(w.hist, hs, false);
  int b;
  uint32_t krem;
  find_bin(hs, kTopkBins, 1, 0, w.st[ST_KREM], b, krem);
  if (threadIdx.x == 0) {
    w.st[ST_B0] = uint32_t(b);
    w.st[ST_KREM] = krem;
    w.st[ST_PHI] = uint32_t(b) << 20;  // composite bits 62..52
    w.st[ST_PLO] = 0;
  }
}

// Set bits of a wave-wide mask held by the lanes below this one.
__device__ __forceinline__ uint32_t bits_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
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

// Exclusive scan of n u32 values in three launches: per-block sums of
// kScanSeg elements, a one-block scan of those sums, then each block's scan
// offset by its sum prefix.
__device__ __forceinline__ uint32_t block_excl_256(uint32_t v, uint32_t& total) {
  __shared__ uint32_t wsum[4];
  uint32_t wt;
  const uint32_t e = wave_excl(v, wt);
  const int wid = threadIdx.x >> 6;
  __syncthreads();  // wsum free (the function may run in a loop)
  if ((threadIdx.x & 63) == 0) wsum[wid] = wt;
  __syncthreads();
  uint32_t base = 0;
  for (int q = 0; q < wid; ++q) base += wsum[q];
  total = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  return base + e;
}

__global__ __launch_bounds__(256) void scan_reduce_kernel(const uint32_t* __restrict__ a, int64_t n,
                                                          uint32_t* __restrict__ bsum,
                                                          const uint32_t* gate) {
  if (gated_off(gate)) return;
  const int64_t b0 = int64_t(blockIdx.x) * kScanSeg + int64_t(threadIdx.x) * 8;
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (b0 + j < n) s += a[b0 + j];
  uint32_t total;
  block_excl_256(s, total);
  if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

__global__ __launch_bounds__(256) void scan_apply_kernel(uint32_t* __restrict__ a, int64_t n,
                                                         const uint32_t* __restrict__ bsum,
                                                         const uint32_t* gate) {
  if (gated_off(gate)) return;
  const int64_t b0 = int64_t(blockIdx.x) * kScanSeg + int64_t(threadIdx.x) * 8;
  uint32_t v[8], s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[j] = b0 + j < n ? a[b0 + j] : 0u;
    s += v[j];
  }
  uint32_t total;
  uint32_t run = bsum[blockIdx.x] + block_excl_256(s, total);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (b0 + j < n) a[b0 + j] = run;
    run += v[j];
  }
}

// In-place exclusive scan of n u32 values by one block of 1024 threads
// (coalesced 1024-wide segments, carried across segments).
__global__ __launch_bounds__(1024) void scan_u32_kernel(uint32_t* __restrict__ a, int64_t n,
                                                        const uint32_t* gate,
                                                        uint32_t* __restrict__ total_out = nullptr) {
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
  if (threadIdx.x == 0 && total_out) *total_out = carry_s;
}

// Pass C: per wave chunk, the above-b0 indices and the candidates at or
// above the k-th composite are marked in a 4096-bit LDS mask (chunk-local
// offsets) and emitted in index order at the chunk's scanned offset.
__global__ __launch_bounds__(256) void topk_pass_c_kernel(TopkWs w, uint32_t* __restrict__ out_idx,
                                                          float* __restrict__ out_val,
                                                          const float* __restrict__ valsrc,
                                                          uint32_t* __restrict__ out_key,
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
    if (out_key) out_key[p] = __float_as_uint(valsrc[i]) & 0x7fffffffu;
    ++p;
  }
}

// Exclusive scan of a[0..n) in place (three launches); *total_out (nullable,
// device) receives the sum.
static void scan_launch(uint32_t* a, int64_t n, uint32_t* bsum, const uint32_t* gate,
                        uint32_t* total_out, hipStream_t st) {
  const unsigned nb = unsigned(ceil_div(n, kScanSeg));
  hipLaunchKernelGGL(scan_reduce_kernel, dim3(nb), dim3(256), 0, st, a, n, bsum, gate);
  hipLaunchKernelGGL(scan_u32_kernel, dim3(1), dim3(1024), 0, st, bsum, int64_t(nb), gate, total_out);
  hipLaunchKernelGGL(scan_apply_kernel, dim3(nb), dim3(256), 0, st, a, n, bsum, gate);
}

// After the bin b0 of the k-th key is known: the remaining composite bits
// (51..0, in rounds of 11, 11, 11, 11, 8) on the candidates, the per-chunk
// counts, their scan and the ordered output.
template <class KF>
static void topk_finish(KF key, const TopkWs& w, uint32_t* out_idx, float* out_val,
                        const float* valsrc, uint32_t* out_key, hipStream_t st,
                        const uint32_t* gate) {
  const dim3 blk{256, 1, 1};
  const unsigned cgrid = 1024;
  const int shifts[5] = {41, 30, 19, 8, 0}, widths[5] = {11, 11, 11, 11, 8};
  for (int q = 0; q < 5; ++q) {
    hipLaunchKernelGGL(topk_cand_hist_kernel<KF>, dim3(cgrid), blk, 0, st, key, w, shifts[q],
                       widths[q], gate);
    hipLaunchKernelGGL(topk_cand_select_kernel, dim3(1), blk, 0, st, w, shifts[q], widths[q], gate);
  }
  hipLaunchKernelGGL(topk_cand_count_kernel<KF>, dim3(cgrid), blk, 0, st, key, w, gate);
  scan_launch(w.cnt, w.nchunks, w.bsum, gate, nullptr, st);
  hipLaunchKernelGGL(topk_pass_c_kernel, dim3(unsigned(ceil_div(w.nchunks, 4))), blk, 0, st, w,
                     out_idx, out_val, valsrc, out_key, gate);
}

template <class KF>
static const float* valsrc_of(const KF&) { return nullptr; }
template <>
const float* valsrc_of<KeyGrad>(const KeyGrad& key) { return key.g; }

// ---------------------------------------------------------------------------
// The sampled single pass over a whole gradient
// ---------------------------------------------------------------------------
constexpr int64_t kSampledMin = int64_t(1) << 20;  // smaller inputs take the two full reads

constexpr unsigned kSampledGrid = 2048;  // blocks of the grid-stride sampled kernels
constexpr int kSampleRun = 64;          // keys sampled at the start of every kSampleGroup
constexpr int kSampleGroup = 4096;
// The sampled pass reads the keys in wave chunks of kSuper keys (4 of the
// selection's chunks); their candidates go to [c*kSuper, ...) of cand/ckey
// (never past the chunk's own keys, so never past n).
constexpr int kSuper = 4 * kChunk;
constexpr int kStage = 256;  // candidates a wave gathers in LDS before one coalesced store

// Histogram (top 11 bits) of the first 64 keys of every 4096 (16 threads
// read them as one 256-byte run), into the privatised copies.
// Level 0 histograms key bits 30..20 of every sampled key into the
// privatised copies; level 1 histograms bits 19..9 of the sampled keys in
// bin ST_BS into chist.
template <int kLevel>
__device__ __forceinline__ void sample_add(uint32_t* h, uint32_t key, uint32_t bin) {
  key &= 0x7fffffffu;
  if (kLevel == 0) atomicAdd(&h[key >> 20], 1u);
  else if ((key >> 20) == bin) atomicAdd(&h[(key >> 9) & 0x7ffu], 1u);
}

template <int kLevel>
__global__ __launch_bounds__(256) void topk_sample_kernel(const float* __restrict__ g, int64_t n,
                                                          TopkWs w) {
  __shared__ uint32_t h[kTopkBins];
  const uint32_t bin = kLevel ? w.st[ST_BS] : 0u;
  for (int b = threadIdx.x; b < kTopkBins; b += 256) h[b] = 0;
  __syncthreads();
  const int64_t units = ceil_div(n, kSampleGroup) * (kSampleRun / 4);
  const int64_t ustride = int64_t(gridDim.x) * 256;
  for (int64_t u0 = int64_t(blockIdx.x) * 256 + threadIdx.x; u0 < units; u0 += 4 * ustride) {
    uint4 vv[4];
    int64_t pos[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {  // four loads in flight
      const int64_t u = u0 + a * ustride;
      pos[a] = u < units ? (u / (kSampleRun / 4)) * kSampleGroup + (u % (kSampleRun / 4)) * 4 : n;
      vv[a] = pos[a] + 3 < n ? *reinterpret_cast<const uint4*>(g + pos[a]) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if (pos[a] + 3 < n) {
        sample_add<kLevel>(h, vv[a].x, bin);
        sample_add<kLevel>(h, vv[a].y, bin);
        sample_add<kLevel>(h, vv[a].z, bin);
        sample_add<kLevel>(h, vv[a].w, bin);
      } else {
        for (int64_t j = pos[a]; j < n && j < pos[a] + 4; ++j)
          sample_add<kLevel>(h, __float_as_uint(g[j]), bin);
      }
    }
  }
  __syncthreads();
  uint32_t* dst = kLevel ? w.chist : w.hist + size_t(blockIdx.x % kHistCopies) * kTopkBins;
  for (int b = threadIdx.x; b < kTopkBins; b += 256)
    if (h[b]) atomicAdd(&dst[b], h[b]);
}

// Keys the sample holds: 64 per 4096 (fewer in a short last group).
static int64_t sample_count(int64_t n) {
  return (n / kSampleGroup) * kSampleRun + std::min<int64_t>(kSampleRun, n % kSampleGroup);
}

// The threshold bin from the sample: the bin holding the q-th sampled key
// from the top.  The copies are summed and cleared for pass B1.
__global__ __launch_bounds__(1024) void topk_sample_select_kernel(TopkWs w, uint32_t q) {
  __shared__ __attribute__((aligned(16))) uint32_t hs[kTopkBins];
  sum_copies_lds(w.hist, hs, true);
  int b;
  uint32_t krem;
  find_bin(hs, kTopkBins, 1, 0, q, b, krem);
  if (threadIdx.x == 0) {
    w.st[ST_BS] = uint32_t(b);
    w.st[ST_BSREM] = krem;
  }
}

// The threshold key from the second sample level: the sub-bin of bin ST_BS
// holding its ST_BSREM-th sampled key from the top; keys at or above the
// sub-bin's lowest key are the candidates.
__global__ __launch_bounds__(256) void topk_sample_select2_kernel(TopkWs w) {
  int b;
  uint32_t krem;
  find_bin(w.chist, kTopkBins, 1, 0, w.st[ST_BSREM], b, krem);
  __syncthreads();
  for (int x = threadIdx.x; x < kTopkBins; x += 256) w.chist[x] = 0;
  if (threadIdx.x == 0) w.st[ST_T] = (w.st[ST_BS] << 20) | (uint32_t(b) << 9);
}

// Wait for this wave's LDS accesses only (vm and export counters at their
// maximum), so that lanes read what other lanes of the wave wrote.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
}

// Pass B1: per wave chunk of kSuper keys, the indices and keys of every key
// at or above the sampled threshold key (the candidates), in index order in the chunk's own regions
// (gathered in LDS and stored kStage at a time), their count (in ccnt and
// cnt), and a histogram of their top 11 bits in the privatised copies.
__global__ __launch_bounds__(256) void topk_pass_b1_kernel(const float* __restrict__ g, int64_t n,
                                                           TopkWs w, const uint32_t* gate) {
  if (gated_off(gate)) return;
  __shared__ uint32_t sidx[4][kStage], skey[4][kStage];
  const uint32_t thr = w.st[ST_T];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t chunk = int64_t(blockIdx.x) * 4 + wid;
  const int64_t nsup = ceil_div(n, kSuper);
  if (chunk < nsup) {  // uniform per wave
    const int64_t i0 = chunk * kSuper;
    uint32_t* cdst = w.cand + i0;
    uint32_t* kdst = w.ckey + i0;
    uint32_t* si = sidx[wid];
    uint32_t* sk = skey[wid];
    uint32_t stored = 0, staged = 0;
    auto flush = [&]() {
      wave_lds_sync();
      for (uint32_t j = lane; j < staged; j += 64) {
        cdst[stored + j] = si[j];
        kdst[stored + j] = sk[j];
      }
      stored += staged;
      staged = 0;
      wave_lds_sync();  // the staging buffer is free again
    };
    // one row of 256 keys: the lane's 4 keys at i (c: at or above thr).  A
    // candidate's place in the row (index order: lane, then u) is the count
    // of the candidates of the lanes below it, from one ballot per u
    auto row = [&](int64_t i, const uint32_t (&kv)[4], const bool (&c)[4]) {
      const uint64_t b0 = __ballot(c[0]), b1 = __ballot(c[1]), b2 = __ballot(c[2]),
                     b3 = __ballot(c[3]);
      if (b0 | b1 | b2 | b3) {  // uniform: many rows of 256 keys hold no candidate
        const uint32_t tot = uint32_t(__popcll(b0) + __popcll(b1) + __popcll(b2) + __popcll(b3));
        if (staged + tot > kStage) flush();  // uniform; a row holds at most kStage
        uint32_t p = staged + ((bits_below(b0) + bits_below(b1)) + (bits_below(b2) + bits_below(b3)));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (c[u]) {
            si[p] = uint32_t(i + u);
            sk[p] = kv[u];
            ++p;
          }
        }
        staged += tot;
      }
    };
    if (i0 + kSuper <= n) {  // uniform: a full chunk
      // rows in batches of kAhead 16-byte loads per lane, two batches in
      // flight: batch b + 1 is loaded before batch b is processed
      constexpr int kAhead = 4, kRows = kSuper / 256;
      static_assert(kRows % (2 * kAhead) == 0, "whole pairs of batches");
      auto load = [&](int r0, uint4 (&vv)[kAhead]) {
#pragma unroll
        for (int a = 0; a < kAhead; ++a)
          vv[a] = *reinterpret_cast<const uint4*>(g + i0 + (r0 + a) * 256 + lane * 4);
      };
      auto process = [&](int r0, const uint4 (&vv)[kAhead]) {
#pragma unroll
        for (int a = 0; a < kAhead; ++a) {
          const uint32_t kv[4] = {vv[a].x & 0x7fffffffu, vv[a].y & 0x7fffffffu,
                                  vv[a].z & 0x7fffffffu, vv[a].w & 0x7fffffffu};
          const bool c[4] = {kv[0] >= thr, kv[1] >= thr, kv[2] >= thr, kv[3] >= thr};
          row(i0 + (r0 + a) * 256 + lane * 4, kv, c);
        }
      };
      uint4 va[kAhead], vb[kAhead];
      load(0, va);
      for (int r0 = 0; r0 < kRows; r0 += 2 * kAhead) {
        load(r0 + kAhead, vb);
        process(r0, va);
        if (r0 + 2 * kAhead < kRows) load(r0 + 2 * kAhead, va);  // uniform
        process(r0 + kAhead, vb);
      }
    } else {  // the last, partial chunk
      for (int r = 0; r < kSuper / 256; ++r) {
        const int64_t i = i0 + r * 256 + lane * 4;
        uint32_t kv[4] = {0, 0, 0, 0};
        bool c[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          c[u] = i + u < n;
          if (c[u]) {
            kv[u] = __float_as_uint(g[i + u]) & 0x7fffffffu;
            c[u] = kv[u] >= thr;
          }
        }
        row(i, kv, c);
      }
    }
    flush();
    if (lane == 0) {
      w.ccnt[chunk] = stored;
      w.cnt[chunk] = stored;
    }
  }
}

// Fewer than k candidates (their total is st[NCAND], from the count scan):
// clear the histogram and let every key be a candidate on the gated second
// run of pass B1 and its scan.
__global__ __launch_bounds__(1024) void topk_retry_kernel(TopkWs w, uint32_t k) {
  const bool retry = w.st[ST_NCAND] < k;
  __syncthreads();  // every thread has read the count
  if (threadIdx.x == 0) {
    w.st[ST_RETRY] = retry ? 1u : 0u;
    if (retry) w.st[ST_T] = 0;
  }
  if (!retry) return;  // uniform
  for (int b = threadIdx.x; b < kHistCopies * kTopkBins; b += 1024) w.hist[b] = 0;
}

// The candidates made contiguous, in index order: wave chunk c's ccnt[c]
// entries go to [cnt[c], cnt[c] + ccnt[c]) of above (indices) and cckey
// (keys).  One wave per chunk.
__global__ __launch_bounds__(256) void topk_compact_kernel(TopkWs w, int64_t nsup) {
  __shared__ uint32_t h[kTopkBins];
  for (int b = threadIdx.x; b < kTopkBins; b += 256) h[b] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  for (int64_t c = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6); c < nsup;
       c += int64_t(gridDim.x) * 4) {
    const uint32_t m = w.ccnt[c], o = w.cnt[c];
    const uint32_t* src = w.cand + c * kSuper;
    const uint32_t* ksrc = w.ckey + c * kSuper;
    for (uint32_t j = lane; j < m; j += 64) {
      const uint32_t key = ksrc[j];
      w.above[o + j] = src[j];
      w.cckey[o + j] = key;
      atomicAdd(&h[key >> 20], 1u);  // the candidates' top 11 key bits
    }
  }
  __syncthreads();
  uint32_t* dst = w.hist + size_t(blockIdx.x % kHistCopies) * kTopkBins;
  for (int b = threadIdx.x; b < kTopkBins; b += 256)
    if (h[b]) atomicAdd(&dst[b], h[b]);
}

// Candidate rounds on the contiguous candidates (st[NCAND] of them):
// histogram of composite bits [shift, shift + width) over those matching the
// prefix's higher bits.
__global__ __launch_bounds__(256) void topk_cc_hist_kernel(TopkWs w, int shift, int width) {
  __shared__ uint32_t h[kTopkBins];
  for (int b = threadIdx.x; b < kTopkBins; b += 256) h[b] = 0;
  __syncthreads();
  const uint64_t prefix = (uint64_t(w.st[ST_PHI]) << 32) | w.st[ST_PLO];
  const int top = shift + width;
  const uint32_t dmask = (1u << width) - 1u;
  const int64_t m = w.st[ST_NCAND];
  for (int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x; j < m; j += int64_t(gridDim.x) * 256) {
    const uint64_t cp = composite(w.cckey[j], w.above[j]);
    if ((cp >> top) == (prefix >> top)) atomicAdd(&h[uint32_t(cp >> shift) & dmask], 1u);
  }
  __syncthreads();
  for (int b = threadIdx.x; b <= int(dmask); b += 256)
    if (h[b]) atomicAdd(&w.chist[b], h[b]);
}

constexpr int kEmitSeg = 4096;  // candidates per segment of the output (256 threads x 16)

// Selected candidates (composite >= the k-th) per segment of kEmitSeg
// contiguous candidates, into cnt[s] for every s < nchunks (0 past the end).
__global__ __launch_bounds__(256) void topk_cc_count_kernel(TopkWs w) {
  const uint64_t theta = (uint64_t(w.st[ST_PHI]) << 32) | w.st[ST_PLO];
  const int64_t m = w.st[ST_NCAND];
  for (int64_t sg = blockIdx.x; sg < w.nchunks; sg += gridDim.x) {
    const int64_t j0 = sg * kEmitSeg;
    if (j0 >= m) {  // uniform: past the candidates
      if (threadIdx.x == 0) w.cnt[sg] = 0;
      continue;
    }
    uint32_t c = 0;
#pragma unroll
    for (int u = 0; u < kEmitSeg / 256; ++u) {
      const int64_t j = j0 + u * 256 + threadIdx.x;
      c += (j < m && composite(w.cckey[j], w.above[j]) >= theta) ? 1u : 0u;
    }
    uint32_t total;
    block_excl_256(c, total);
    if (threadIdx.x == 0) w.cnt[sg] = total;
  }
}

// The selected candidates of each segment at its scanned offset, in index
// order (16 consecutive candidates per thread).
__global__ __launch_bounds__(256) void topk_cc_emit_kernel(TopkWs w, uint32_t* __restrict__ out_idx,
                                                           float* __restrict__ out_val,
                                                           const float* __restrict__ valsrc,
                                                           uint32_t* __restrict__ out_key) {
  const uint64_t theta = (uint64_t(w.st[ST_PHI]) << 32) | w.st[ST_PLO];
  const int64_t m = w.st[ST_NCAND];
  __shared__ uint32_t wcnt[kEmitSeg / 256][4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint64_t below = (uint64_t(1) << lane) - 1;
  for (int64_t sg = blockIdx.x; sg * kEmitSeg < m; sg += gridDim.x) {
    // row u holds candidates j0 + 256 u + thread; rows, then threads, are in
    // index order, so ballot ranks within a row give the output order
    const int64_t j0 = sg * kEmitSeg;
    bool sel[kEmitSeg / 256];
    uint32_t idx[kEmitSeg / 256], ck[kEmitSeg / 256], lp[kEmitSeg / 256];
#pragma unroll
    for (int u = 0; u < kEmitSeg / 256; ++u) {
      const int64_t j = j0 + u * 256 + threadIdx.x;
      idx[u] = j < m ? w.above[j] : 0u;
      ck[u] = j < m ? w.cckey[j] : 0u;
      sel[u] = j < m && composite(ck[u], idx[u]) >= theta;
      const uint64_t b = __ballot(sel[u]);
      lp[u] = uint32_t(__popcll(b & below));
      if (lane == 0) wcnt[u][wid] = uint32_t(__popcll(b));
    }
    __syncthreads();
    uint32_t run = w.cnt[sg];
#pragma unroll
    for (int u = 0; u < kEmitSeg / 256; ++u) {
      uint32_t before = 0;
      for (int q = 0; q < 4; ++q) before += q < wid ? wcnt[u][q] : 0u;
      if (sel[u]) {
        const uint32_t p = run + before + lp[u];
        out_idx[p] = idx[u];
        if (out_val) out_val[p] = valsrc[idx[u]];
        if (out_key) out_key[p] = ck[u];
      }
      run += (wcnt[u][0] + wcnt[u][1]) + (wcnt[u][2] + wcnt[u][3]);
    }
    __syncthreads();  // wcnt is reused by the next segment
  }
}

static usaf_status topk_run_sampled(const float* g, int64_t n, int64_t k, uint32_t* out_idx,
                                    float* out_val, uint32_t* out_key, char* ws, hipStream_t st);

// Enqueue one selection: the k eligible elements ranked first by (key desc,
// index asc) among n (minus the excluded), written ascending to out_idx.
// out_key (nullable; gradient keys only) receives each selected entry's key,
// |g| as bits, aligned with out_idx.
template <class KF>
usaf_status topk_run(KF key, int64_t n, int64_t k, const uint32_t* ex, int64_t nex,
                     uint32_t* out_idx, float* out_val, const float* valsrc, char* ws,
                     hipStream_t st, const uint32_t* gate = nullptr, uint32_t* out_key = nullptr) {
  if (k == 0 || n == 0) return USAF_OK;
  if (out_key && !std::is_same<KF, KeyGrad>::value) return USAF_ERR_UNSUPPORTED;
  if (out_key && !valsrc) valsrc = valsrc_of(key);
  if (!ex && !gate && n >= kSampledMin && std::is_same<KF, KeyGrad>::value)
    return topk_run_sampled(valsrc_of(key), n, k, out_idx, out_val, out_key, ws, st);
  const int64_t ntiles = ceil_div(n, kTopkTile);
  const TopkWs w = topk_ws(ws, n);
  const dim3 blk{256, 1, 1}, grid{unsigned(ntiles), 1, 1};
  timer_begin(USAF_K_TOPK, st);
  hipLaunchKernelGGL(topk_init_kernel, dim3(64), blk, 0, st, w, uint32_t(k), gate);
  hipLaunchKernelGGL(topk_pass_a_kernel<KF>, grid, blk, 0, st, key, n, ex, nex, w, gate);
  hipLaunchKernelGGL(topk_select_a_kernel, dim3(1), dim3(1024), 0, st, w, gate);
  hipLaunchKernelGGL(topk_pass_b_kernel<KF>, grid, blk, 0, st, key, n, ex, nex, w, gate);
  topk_finish<KF>(key, w, out_idx, out_val, valsrc, out_key, st, gate);
  timer_end(USAF_K_TOPK, st);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

// The sampled single pass (see the file comment) over a whole gradient.
static usaf_status topk_run_sampled(const float* g, int64_t n, int64_t k, uint32_t* out_idx,
                                    float* out_val, uint32_t* out_key, char* ws, hipStream_t st) {
  const TopkWs w = topk_ws(ws, n);
  const dim3 blk{256, 1, 1};
  const int64_t S = sample_count(n);
  const double share = double(k) * double(S) / double(n);
  const int64_t q = std::min<int64_t>(S, int64_t(std::ceil(1.25 * share)) + 16);
  const int64_t units = ceil_div(n, kSampleGroup) * (kSampleRun / 4);
  const unsigned sgrid = unsigned(std::min<int64_t>(ceil_div(units, 256), kSampledGrid));
  const int64_t nsup = ceil_div(n, kSuper);
  const unsigned bgrid = unsigned(ceil_div(nsup, 4));  // every chunk its own wave
  const unsigned cgrid = 1024;
  uint32_t* ncand = w.st + ST_NCAND;
  timer_begin(USAF_K_TOPK, st);
  hipLaunchKernelGGL(topk_init_kernel, dim3(64), blk, 0, st, w, uint32_t(k), nullptr);
  hipLaunchKernelGGL(topk_sample_kernel<0>, dim3(sgrid), blk, 0, st, g, n, w);
  hipLaunchKernelGGL(topk_sample_select_kernel, dim3(1), dim3(1024), 0, st, w, uint32_t(q));
  hipLaunchKernelGGL(topk_sample_kernel<1>, dim3(sgrid), blk, 0, st, g, n, w);
  hipLaunchKernelGGL(topk_sample_select2_kernel, dim3(1), blk, 0, st, w);
  hipLaunchKernelGGL(topk_pass_b1_kernel, dim3(bgrid), blk, 0, st, g, n, w, nullptr);
  scan_launch(w.cnt, nsup, w.bsum, nullptr, ncand, st);
  hipLaunchKernelGGL(topk_retry_kernel, dim3(1), dim3(1024), 0, st, w, uint32_t(k));
  hipLaunchKernelGGL(topk_pass_b1_kernel, dim3(bgrid), blk, 0, st, g, n, w, w.st + ST_RETRY);
  scan_launch(w.cnt, nsup, w.bsum, w.st + ST_RETRY, ncand, st);
  hipLaunchKernelGGL(topk_compact_kernel, dim3(bgrid), blk, 0, st, w, nsup);
  // the candidates' histogram -> the bin b0 of the k-th key; then the
  // remaining composite bits on the contiguous candidates
  hipLaunchKernelGGL(topk_select_a_kernel, dim3(1), dim3(1024), 0, st, w, nullptr);
  const int shifts[5] = {41, 30, 19, 8, 0}, widths[5] = {11, 11, 11, 11, 8};
  for (int r = 0; r < 5; ++r) {
    hipLaunchKernelGGL(topk_cc_hist_kernel, dim3(cgrid), blk, 0, st, w, shifts[r], widths[r]);
    hipLaunchKernelGGL(topk_cand_select_kernel, dim3(1), blk, 0, st, w, shifts[r], widths[r], nullptr);
  }
  hipLaunchKernelGGL(topk_cc_count_kernel, dim3(cgrid), blk, 0, st, w);
  scan_launch(w.cnt, w.nchunks, w.bsum, nullptr, nullptr, st);
  hipLaunchKernelGGL(topk_cc_emit_kernel, dim3(cgrid), blk, 0, st, w, out_idx, out_val, g, out_key);
  timer_end(USAF_K_TOPK, st);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

// ---------------------------------------------------------------------------
// Merges of sorted u32 lists (RigL's membership test and state remap).
// A list is cut into blocks of kPB entries; where each block's values fall
// in the other list is found first (one wave per block boundary), then each
// block works on its own slices in LDS.
// ---------------------------------------------------------------------------
constexpr int kPB = 2048;    // list entries per block (256 threads x 8)
constexpr int kPCap = 4096;  // entries of the other list a block stages in LDS

// lower_bound over a sorted u32 array by one whole wave (every lane returns
// the same result): each step probes 64 evenly spaced entries of the range
// [lo, hi) holding the answer and keeps the part between the last probe
// below v and the first at or above it, 64-fold narrower.
__device__ __forceinline__ int64_t wave_lower_bound(const uint32_t* __restrict__ a, int64_t n,
                                                    uint64_t v) {
  const int lane = threadIdx.x & 63;
  int64_t lo = 0, hi = n;
  while (hi - lo > 64) {
    const int64_t step = (hi - lo + 63) / 64;
    const int64_t p = lo + (int64_t(lane) + 1) * step - 1;
    const bool less = p < hi && uint64_t(a[p]) < v;
    const int c = __popcll(__ballot(less));  // probes below v: a prefix of the lanes
    const int64_t pc = lo + (int64_t(c) + 1) * step - 1;
    if (c < 64 && pc < hi) hi = pc;
    lo += int64_t(c) * step;
  }
  const int64_t p = lo + lane;
  const bool less = p < hi && uint64_t(a[p]) < v;
  return lo + __popcll(__ballot(less));
}

// bounds[b], b = 0..nb: 0, then lower_bound(ref, v_b) for 0 < b < nb, then
// nref; v_b = q[b * kPB] (the first entry of block b of list q), or b * kPB
// itself when q is null.  One wave per bound.
__global__ __launch_bounds__(256) void part_bounds_kernel(const uint32_t* __restrict__ q, int64_t nb,
                                                          const uint32_t* __restrict__ ref,
                                                          int64_t nref, uint32_t* __restrict__ bounds,
                                                          const uint32_t* gate) {
  if (gated_off(gate)) return;
  const int64_t b = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (b > nb) return;  // uniform per wave
  uint32_t out;
  if (b == 0) {
    out = 0;
  } else if (b == nb) {
    out = uint32_t(nref);
  } else {
    const uint64_t v = q ? uint64_t(q[b * kPB]) : uint64_t(b * kPB);
    out = uint32_t(wave_lower_bound(ref, nref, v));
  }
  if ((threadIdx.x & 63) == 0) bounds[b] = out;
}

__device__ __forceinline__ int lds_lower_bound(const uint32_t* a, int n, uint32_t v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// For each entry of the sorted list q, whether it is absent from the sorted
// list ref (flag 1) and how many are.  Block b holds q's entries from b*kPB;
// every ref value they could equal lies in ref[bounds[b], bounds[b+1]).
__global__ __launch_bounds__(256) void member_merge_kernel(const uint32_t* __restrict__ q, int64_t nq,
                                                           const uint32_t* __restrict__ ref,
                                                           const uint32_t* __restrict__ bounds,
                                                           uint8_t* __restrict__ absent_flag,
                                                           uint32_t* __restrict__ n_absent) {
  __shared__ uint32_t seg[kPCap];
  const int64_t q0 = int64_t(blockIdx.x) * kPB;
  const int64_t lo = bounds[blockIdx.x];
  const int64_t len = int64_t(bounds[blockIdx.x + 1]) - lo;
  const bool staged = len <= kPCap;
  if (staged)
    for (int64_t j = threadIdx.x; j < len; j += 256) seg[j] = ref[lo + j];
  __syncthreads();
  uint32_t nabs = 0;
  for (int j = 0; j < kPB / 256; ++j) {
    const int64_t i = q0 + j * 256 + threadIdx.x;
    if (i >= nq) break;
    const uint32_t v = q[i];
    bool hit;
    if (staged) {
      const int a = lds_lower_bound(seg, int(len), v);
      hit = a < len && seg[a] == v;
    } else {
      const int64_t a = lo + lower_bound_u32(ref + lo, len, v);
      hit = a < lo + len && ref[a] == v;
    }
    absent_flag[i] = hit ? 0 : 1;
    nabs += hit ? 0u : 1u;
  }
  uint32_t total;
  block_excl_256(nabs, total);
  if (threadIdx.x == 0 && total) atomicAdd(n_absent, total);
}

// RigL's new list and moments.  Block b holds the old entries q0 = b*kPB ..
// q0 + nq; D[b] counts the dropped positions below q0 and G[b] the grown
// entries below old_idx[q0] (0 for the first block).  A kept entry at old
// position q lands at (q - dropped before q) + (grown below it) with its
// moments; a grown entry j whose value falls in this block's old range lands
// at j + (kept entries below it) with zero moments.  With new_w, the compact
// weight list follows: a kept entry's weight from old_w, a grown entry's
// from the flat weights.
template <class W>
__global__ __launch_bounds__(256) void rigl_place_kernel(
    const uint32_t* __restrict__ old_idx, const float* __restrict__ old_m,
    const float* __restrict__ old_v, int64_t k, const uint32_t* __restrict__ dpos,
    const uint32_t* __restrict__ D, const uint32_t* __restrict__ grown,
    const uint32_t* __restrict__ G, uint32_t* __restrict__ new_idx, float* __restrict__ new_m,
    float* __restrict__ new_v, const W* __restrict__ old_w, const W* __restrict__ Wf,
    W* __restrict__ new_w) {
  __shared__ uint32_t os[kPB];       // old entries of the block
  __shared__ uint32_t pre[kPB + 1];  // dropped flags, then dropped before each position
  __shared__ uint32_t gs[kPCap];     // grown entries in the block's range
  const int tid = threadIdx.x;
  const int64_t q0 = int64_t(blockIdx.x) * kPB;
  const int nq = int(min(int64_t(kPB), k - q0));
  for (int j = tid; j < kPB; j += 256) {
    if (j < nq) os[j] = old_idx[q0 + j];
    pre[j] = 0;
  }
  __syncthreads();
  const uint32_t d0 = D[blockIdx.x], d1 = D[blockIdx.x + 1];
  for (uint32_t x = d0 + tid; x < d1; x += 256) pre[dpos[x] - q0] = 1;
  const uint32_t g0 = G[blockIdx.x], g1 = G[blockIdx.x + 1];
  const int glen = int(g1 - g0);
  const bool staged = glen <= kPCap;
  if (staged)
    for (int j = tid; j < glen; j += 256) gs[j] = grown[g0 + j];
  __syncthreads();
  {  // exclusive scan of the flags, 8 per thread
    uint32_t f[8], sum = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f[j] = pre[tid * 8 + j];
      sum += f[j];
    }
    uint32_t total;
    uint32_t run = block_excl_256(sum, total);  // its barriers order the reads above
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pre[tid * 8 + j] = run;
      run += f[j];
    }
    if (tid == 0) pre[kPB] = total;
  }
  __syncthreads();
  for (int j = tid; j < nq; j += 256) {
    if (pre[j + 1] != pre[j]) continue;  // dropped
    const uint32_t f = os[j];
    const int64_t below = staged ? lds_lower_bound(gs, glen, f) : lower_bound_u32(grown + g0, glen, f);
    const int64_t out = (q0 + j - (int64_t(d0) + pre[j])) + int64_t(g0) + below;
    new_idx[out] = f;
    new_m[out] = old_m[q0 + j];
    new_v[out] = old_v[q0 + j];
    if (new_w) new_w[out] = old_w[q0 + j];
  }
  for (int x = tid; x < glen; x += 256) {
    const uint32_t f = staged ? gs[x] : grown[g0 + x];
    const int p = lds_lower_bound(os, nq, f);
    const int64_t kept_below = (q0 + p) - (int64_t(d0) + pre[p]);
    const int64_t out = int64_t(g0) + x + kept_below;
    new_idx[out] = f;
    new_m[out] = 0.f;
    new_v[out] = 0.f;
    if (new_w) new_w[out] = Wf[f];
  }
}

// Sorted union of two strictly ascending lists a and b.  Block q holds a's
// entries from q*kPB and the b entries whose values fall in its range
// (b[bounds[q], bounds[q+1])); b entries equal to an a entry are dropped.
// Pass 0 writes each block's output count; pass 1 (after their scan) writes
// the block's entries at its offset, in ascending order.
template <int kPass>
__global__ __launch_bounds__(256) void union_merge_kernel(const uint32_t* __restrict__ a, int64_t na,
                                                          const uint32_t* __restrict__ b,
                                                          const uint32_t* __restrict__ bounds,
                                                          uint32_t* __restrict__ cnt,
                                                          uint32_t* __restrict__ out) {
  __shared__ uint32_t as[kPB];
  __shared__ uint32_t adup[kPB + 1];  // a entry present in b, then the count of those before
  __shared__ uint32_t bs[kPCap];
  const int tid = threadIdx.x;
  const int64_t q0 = int64_t(blockIdx.x) * kPB;
  const int nq = int(min(int64_t(kPB), na - q0));
  for (int j = tid; j < kPB; j += 256) {
    as[j] = j < nq ? a[q0 + j] : 0xffffffffu;
    adup[j] = 0;
  }
  const uint32_t b0 = bounds[blockIdx.x], b1 = bounds[blockIdx.x + 1];
  const int blen = int(b1 - b0);
  const bool staged = blen <= kPCap;
  if (staged)
    for (int j = tid; j < blen; j += 256) bs[j] = b[b0 + j];
  __syncthreads();
  // mark the a entries that b also holds (each b value lands on at most one)
  uint32_t nnew = 0;  // b entries of this thread that a lacks
  for (int j = tid; j < blen; j += 256) {
    const uint32_t v = staged ? bs[j] : b[b0 + j];
    const int p = lds_lower_bound(as, nq, v);
    if (p < nq && as[p] == v) adup[p] = 1;
    else ++nnew;
  }
  __syncthreads();
  if (kPass == 0) {
    uint32_t total;
    block_excl_256(nnew, total);
    if (tid == 0) cnt[blockIdx.x] = uint32_t(nq) + total;
    return;
  }
  {  // exclusive scan of the duplicate flags, 8 per thread
    uint32_t f[8], sum = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f[j] = adup[tid * 8 + j];
      sum += f[j];
    }
    uint32_t total;
    uint32_t run = block_excl_256(sum, total);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      adup[tid * 8 + j] = run;
      run += f[j];
    }
    if (tid == 0) adup[kPB] = total;
  }
  __syncthreads();
  const uint32_t base = cnt[blockIdx.x];
  // an a entry lands after the block's a entries and new b entries below it
  for (int j = tid; j < nq; j += 256) {
    const uint32_t v = as[j];
    const int below = staged ? lds_lower_bound(bs, blen, v) : int(lower_bound_u32(b + b0, blen, v));
    // b entries below v: the new ones, plus the duplicates of a entries below v
    out[base + j + (below - adup[j])] = v;
  }
  // a new b entry lands after the a entries below it and the new b entries before it
  for (int j = tid; j < blen; j += 256) {
    const uint32_t v = staged ? bs[j] : b[b0 + j];
    const int p = lds_lower_bound(as, nq, v);
    if (p < nq && as[p] == v) continue;  // already in a
    // b entries before j: j of them, adup[p] of which are duplicates (of a entries below v)
    out[base + p + (j - adup[p])] = v;
  }
}

// The drop keys of RigL's list-sized drop selection: the key of W at each
// old entry, from the flat weights (KD with the old list) or from a compact
// copy of them (KD without a list).
template <class KD>
__global__ __launch_bounds__(256) void rigl_drop_keys_kernel(KD drop, int64_t k,
                                                             uint32_t* __restrict__ kdrop) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < k; i += stride) {
    uint32_t key;
    drop(i, key);
    kdrop[i] = key;
  }
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
  size_t topk, dpos, grown, gpos, fresh, flag, kdrop, kgrow, bounds, cnt, total;
};
static WsRigl ws_rigl(int64_t N, int64_t k) {
  WsRigl L;
  L.topk = 0;
  const size_t t = topk_ws_bytes(N > k ? N : k);
  const size_t kb = align256(size_t(k) * 4 + 4);
  const size_t nb = size_t(ceil_div(k > 0 ? k : 1, kPB)) + 1;
  L.dpos = align256(t);
  L.grown = L.dpos + kb;
  L.gpos = L.grown + kb;
  L.fresh = L.gpos + kb;
  L.flag = L.fresh + kb;
  L.kdrop = L.flag + align256(size_t(k) + 4);
  L.kgrow = L.kdrop + kb;
  L.bounds = L.kgrow + kb;           // three bound arrays of nb words
  L.cnt = L.bounds + 3 * align256(nb * 4);
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
  if (reinterpret_cast<uintptr_t>(ws) & 15) return USAF_ERR_UNSUPPORTED;  // 16-byte histogram reads
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
                                          const void* Wflat, const void* old_w,
                                          const uint32_t* old_idx,
                                          const float* old_m, const float* old_v, int64_t k,
                                          int64_t r, uint32_t* new_idx, float* new_m, float* new_v,
                                          void* new_w, usaf_rigl_stats* stats, void* ws,
                                          size_t ws_bytes, hipStream_t stream) {
  USAF_TRY(check_shape(shape));
  const int64_t N = n_weights(*shape);
  if (k < 0 || r < 0 || k > N || r > k || r > N - k) return USAF_ERR_INVALID_ARG;
  if (!grad || !Wflat || !old_idx || !old_m || !old_v || !new_idx || !new_m || !new_v)
    return USAF_ERR_INVALID_ARG;
  if (new_w && !old_w) return USAF_ERR_INVALID_ARG;  // kept weights come from old_w
  if (reinterpret_cast<uintptr_t>(grad) & 15) return USAF_ERR_UNSUPPORTED;
  const WsRigl L = ws_rigl(N, k);
  if (!ws || ws_bytes < L.total) return USAF_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & 15) return USAF_ERR_UNSUPPORTED;  // 16-byte histogram reads
  if (k == 0) return USAF_OK;
  char* w = static_cast<char*>(ws);
  uint32_t* dpos = reinterpret_cast<uint32_t*>(w + L.dpos);
  uint32_t* grown = reinterpret_cast<uint32_t*>(w + L.grown);
  uint32_t* gpos = reinterpret_cast<uint32_t*>(w + L.gpos);
  uint32_t* fresh = reinterpret_cast<uint32_t*>(w + L.fresh);
  uint8_t* flag = reinterpret_cast<uint8_t*>(w + L.flag);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(w + L.cnt);  // [0] novel count, [1..2] gates
  char* tws = w + L.topk;
  uint32_t* kdrop = reinterpret_cast<uint32_t*>(w + L.kdrop);
  uint32_t* kgrow = reinterpret_cast<uint32_t*>(w + L.kgrow);
  const int64_t nb = ceil_div(k, kPB);
  const size_t bstride = align256(size_t(nb + 1) * 4) / 4;
  uint32_t* B_fresh = reinterpret_cast<uint32_t*>(w + L.bounds);  // old_idx bounds of fresh's blocks
  uint32_t* B_drop = B_fresh + bstride;                              // dpos bounds of old's blocks
  uint32_t* B_grow = B_drop + bstride;                               // grown bounds of old's blocks
  const unsigned bgrid = unsigned(ceil_div(nb + 1, 4));
  // fresh top-k of |g| (with its keys, the grow selection's keys) and which
  // of its entries are new
  USAF_TRY(topk_run(KeyGrad{grad}, N, k, nullptr, 0, fresh, nullptr, nullptr, tws, stream, nullptr,
                    kgrow));
  hipLaunchKernelGGL(rigl_stats_init_kernel, dim3(1), dim3(1), 0, stream, cnt);
  hipLaunchKernelGGL(part_bounds_kernel, dim3(bgrid), dim3(256), 0, stream, fresh, nb, old_idx, k,
                     B_fresh, nullptr);
  hipLaunchKernelGGL(member_merge_kernel, dim3(unsigned(nb)), dim3(256), 0, stream, fresh, k,
                     old_idx, B_fresh, flag, cnt);
  USAF_LAUNCH_CHECK();
  if (r > 0) {
    hipLaunchKernelGGL(rigl_gate_kernel, dim3(1), dim3(1), 0, stream, cnt, r, cnt + 1);
    const unsigned kgrid = unsigned(std::min<int64_t>(ceil_div(k, 256), 8192));
    const uint32_t* kidx = old_w ? nullptr : old_idx;  // the compact list is read in order
    const void* wsrc = old_w ? old_w : Wflat;
    if (shape->act == USAF_BF16)
      hipLaunchKernelGGL(rigl_drop_keys_kernel<KeyDropBf16>, dim3(kgrid), dim3(256), 0, stream,
                         KeyDropBf16{static_cast<const bf16_t*>(wsrc), kidx}, k, kdrop);
    else
      hipLaunchKernelGGL(rigl_drop_keys_kernel<KeyDropF32>, dim3(kgrid), dim3(256), 0, stream,
                         KeyDropF32{static_cast<const float*>(wsrc), kidx}, k, kdrop);
    USAF_LAUNCH_CHECK();
    // grow from the fresh top-k (when it holds >= r new entries) ...
    USAF_TRY(topk_run(KeyArr{kgrow, flag}, k, r, nullptr, 0, gpos, nullptr, nullptr, tws, stream,
                      cnt + 1));
    hipLaunchKernelGGL(gather_u32_kernel, dim3(unsigned(ceil_div(r, 256))), dim3(256), 0, stream,
                       fresh, gpos, r, grown, cnt + 1);
    // ... or from everything outside the old set
    USAF_TRY(topk_run(KeyGrad{grad}, N, r, old_idx, k, grown, nullptr, nullptr, tws, stream,
                      cnt + 2));
    // drop: r smallest |w| among the active entries (positions into old_idx)
    USAF_TRY(topk_run(KeyArr{kdrop, nullptr}, k, r, nullptr, 0, dpos, nullptr, nullptr, tws, stream));
  }
  timer_begin(USAF_K_RIGL_MERGE, stream);
  hipLaunchKernelGGL(part_bounds_kernel, dim3(bgrid), dim3(256), 0, stream, nullptr, nb, dpos, r,
                     B_drop, nullptr);
  hipLaunchKernelGGL(part_bounds_kernel, dim3(bgrid), dim3(256), 0, stream, old_idx, nb, grown, r,
                     B_grow, nullptr);
  if (shape->act == USAF_BF16)
    hipLaunchKernelGGL(rigl_place_kernel<bf16_t>, dim3(unsigned(nb)), dim3(256), 0, stream, old_idx,
                       old_m, old_v, k, dpos, B_drop, grown, B_grow, new_idx, new_m, new_v,
                       static_cast<const bf16_t*>(old_w), static_cast<const bf16_t*>(Wflat),
                       static_cast<bf16_t*>(new_w));
  else
    hipLaunchKernelGGL(rigl_place_kernel<float>, dim3(unsigned(nb)), dim3(256), 0, stream, old_idx,
                       old_m, old_v, k, dpos, B_drop, grown, B_grow, new_idx, new_m, new_v,
                       static_cast<const float*>(old_w), static_cast<const float*>(Wflat),
                       static_cast<float*>(new_w));
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
size_t union_ws_bytes(int64_t na) {
  const int64_t nblk = na > 0 ? ceil_div(na, kPB) : 0;
  return 2 * align256(size_t(nblk + 1) * 4) + align256(size_t(ceil_div(nblk + 1, kScanSeg) + 1) * 4) +
         256;
}
__global__ void union_count_kernel(const uint32_t* total, int64_t* n_out) { *n_out = int64_t(*total); }
}  // namespace usaf

extern "C" usaf_status usaf_sorted_union(const uint32_t* a, int64_t na, const uint32_t* b, int64_t nb,
                                         uint32_t* out, int64_t* n_out, void* ws, size_t ws_bytes,
                                         hipStream_t stream) {
  if (na < 0 || nb < 0 || na + nb >= (int64_t(1) << 32)) return USAF_ERR_INVALID_ARG;
  if ((na && !a) || (nb && !b) || (na + nb && !out) || !n_out) return USAF_ERR_INVALID_ARG;
  if (!ws || ws_bytes < usaf::union_ws_bytes(na + nb)) return USAF_ERR_WORKSPACE;
  if (na == 0) {  // the union is b (a copy) -- as a merge of b with an empty list
    std::swap(a, b);
    std::swap(na, nb);
  }
  const int64_t nblk = na ? ceil_div(na, kPB) : 0;
  uint32_t* w = static_cast<uint32_t*>(ws);
  uint32_t* bounds = w;                                   // [nblk + 1]
  uint32_t* cnt = w + align256(size_t(nblk + 1) * 4) / 4;  // [nblk] counts, then offsets
  uint32_t* bsum = cnt + align256(size_t(nblk + 1) * 4) / 4;
  uint32_t* total = bsum + align256(size_t(ceil_div(nblk + 1, kScanSeg) + 1) * 4) / 4;
  hipLaunchKernelGGL(rigl_stats_init_kernel, dim3(1), dim3(1), 0, stream, total);
  if (nblk > 0) {
    hipLaunchKernelGGL(part_bounds_kernel, dim3(unsigned(ceil_div(nblk + 1, 4))), dim3(256), 0, stream,
                       a, nblk, b, nb, bounds, nullptr);
    hipLaunchKernelGGL(union_merge_kernel<0>, dim3(unsigned(nblk)), dim3(256), 0, stream, a, na, b,
                       bounds, cnt, out);
    scan_launch(cnt, nblk, bsum, nullptr, total, stream);
    hipLaunchKernelGGL(union_merge_kernel<1>, dim3(unsigned(nblk)), dim3(256), 0, stream, a, na, b,
                       bounds, cnt, out);
  }
  hipLaunchKernelGGL(union_count_kernel, dim3(1), dim3(1), 0, stream, total, n_out);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}
