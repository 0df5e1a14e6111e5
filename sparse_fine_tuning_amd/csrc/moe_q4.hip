// Expert GEMMs of the forward that read the pages' own 4-bit storage
// directly (README "how it works": caching bullet, the trade between a
// resident dequantised copy and dequantising as the weights are used;
// quantisation recipe: affine codes in groups along the input dimension).
//
// The weight operand is staged through registers: each thread loads one
// 32-bit word of codes (8 weights) and the group's fp16 scale and zero,
// forms w = bf16(fp32(fp32(q - z) * s)) exactly as the resident dequant
// does, and writes the 8 bf16 values into the k-contiguous LDS row the
// register-staged MFMA kernel multiplies from.  A layer so computed equals,
// bit for bit, the same layer run on the resident copy of the same codes:
// the weights are the same bf16 values and each output element accumulates
// the same 16-wide MFMA chunks in the same k order from zero.
//
// gate_up: [g | u] = x W_gu^T, a = bf16(silu(g) u); down: y = a W_d^T per
// slot (bf16), combined per token by the routing weights afterwards.  Used
// for layers that only run forward (the frozen lower layers of a stack).
#include "gemm_v2.hpp"
#include "moe_internal.hpp"
#include "timing.hpp"

namespace usaf {
namespace q4 {

constexpr int kTileM = 128, kTileN = 128;

// Rows of affine 4-bit codes, k-contiguous: row r of the tile is code row
// map(r); element 2i of a row is the low nibble of byte i.
struct CodeRows {
  const uint8_t* q;   // [rows, K/2]
  const uint16_t* s;  // [rows, K/G] fp16
  const uint16_t* z;  // [rows, K/G] fp16
  int64_t qpitch;     // K/2 bytes per row
  int64_t gpitch;     // K/G groups per row
  int gshift;         // log2(G)
};

// The dequantising loader: 4 rows x 8 k per thread, like KcLoader<bf16_t>.
struct KcLoaderQ4 {
  const uint32_t* qp[4];
  const uint16_t* sp[4];
  const uint16_t* zp[4];
  uint32_t ok;
  int c, kend, gshift;
  uint32_t word[4];
  uint16_t sc[4], zr[4];
  int klive;
  template <class Src>
  __device__ __forceinline__ void init(const Src& src, int tid) {
    c = tid & 7;
    kend = src.kend;
    gshift = src.codes.gshift;
    ok = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      const bool live = src.valid(r);
      const int64_t row = src.code_row(live ? r : 0);
      ok |= live ? (1u << i) : 0u;
      qp[i] = reinterpret_cast<const uint32_t*>(src.codes.q + row * src.codes.qpitch);
      sp[i] = src.codes.s + row * src.codes.gpitch;
      zp[i] = src.codes.z + row * src.codes.gpitch;
    }
  }
  __device__ __forceinline__ void load(int k0) {
    const int k = k0 + 8 * c;
    const int kk = min(k, kend - 8);
    klive = k < kend;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      word[i] = qp[i][kk >> 3];
      sc[i] = sp[i][kk >> gshift];
      zr[i] = zp[i][kk >> gshift];
    }
  }
  __device__ __forceinline__ void store(bf16_t* S, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool live = ((ok >> i) & 1u) && klive;
      const float s = float(__builtin_bit_cast(_Float16, sc[i]));
      const float z = float(__builtin_bit_cast(_Float16, zr[i]));
      uint32_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float d0 = float((word[i] >> (8 * j)) & 0xfu) - z;
        const float d1 = float((word[i] >> (8 * j + 4)) & 0xfu) - z;
        o[j] = live ? f2bf2(d0 * s, d1 * s) : 0u;
      }
      *reinterpret_cast<uint4*>(&S[((tid >> 3) + 32 * i) * kLdsRow + 8 * c]) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
};

// bf16 activation rows for the register-staged loader.
struct ActRows {
  const bf16_t* act; const int32_t* perm; int K; int base; int rows; int64_t ld; int kend;
  bool gather;  // rows of tokens through perm (gate_up), else consecutive rows (down)
  __device__ __forceinline__ const bf16_t* row(int r) const {
    const int rr = min(r, rows - 1);
    return gather ? act + int64_t(perm[base + rr] / K) * ld : act + int64_t(base + rr) * ld;
  }
};

// gate_up weight rows of a 128-column tile holding 64 features: wave column
// wn takes features F0 + 32 wn .. + 31, its first 32 columns the gate rows
// and its next 32 the up rows of those features (so one lane holds g and u
// of one feature).
struct GateUpCodes {
  CodeRows codes; int64_t row0; int F0; int I; int kend;
  __device__ __forceinline__ int feature(int col) const { return F0 + 32 * (col >> 6) + (col & 31); }
  __device__ __forceinline__ bool valid(int col) const { return feature(col) < I; }
  __device__ __forceinline__ int64_t code_row(int col) const {
    const int f = feature(col);
    return row0 + (((col >> 5) & 1) ? I + f : f);
  }
};
struct DownCodes {
  CodeRows codes; int64_t row0; int n0; int H; int kend;
  __device__ __forceinline__ bool valid(int col) const { return n0 + col < H; }
  __device__ __forceinline__ int64_t code_row(int col) const { return row0 + n0 + col; }
};

struct QGateUp {
  using ALoader = KcLoader<bf16_t>;
  using BLoader = KcLoaderQ4;
  const bf16_t* X; CodeRows w; const int32_t* offsets; const int32_t* perm;
  bf16_t* gu; bf16_t* a;
  int H, E, K, I, NT;
  __device__ __forceinline__ bool tile(int L, MTile& t) const {
    if (!g2::grouped_tile<kTileM>(offsets, E, NT, L, t)) return false;
    t.kb = 0; t.ke = H; t.n0 = t.nt * (kTileN / 2);
    return true;
  }
  __device__ __forceinline__ ActRows a_src(const MTile& t) const {
    return ActRows{X, perm, K, t.off + t.m0, t.mc, H, H, true};
  }
  __device__ __forceinline__ GateUpCodes b_src(const MTile& t) const {
    return GateUpCodes{w, int64_t(t.e) * 2 * I, t.n0, I, H};
  }
  __device__ __forceinline__ void epilogue(const MTile& t, f32x16_t (&acc)[2][2], int wm, int wn,
                                           int lane) const {
    const int f = t.n0 + 32 * wn + (lane & 31);
    if (f >= I) return;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row(wm, i, r, lane);
        if (row >= t.mc) continue;
        // g, u rounded once; a = bf16(silu(g) u) from the rounded values
        const uint32_t gp = f2bf2(acc[i][0][r], 0.f), up = f2bf2(acc[i][1][r], 0.f);
        const float g = __uint_as_float(gp << 16), u = __uint_as_float(up << 16);
        const int64_t p = t.off + t.m0 + row;
        gu[p * 2 * I + f] = bf16_t(gp & 0xffffu);
        gu[p * 2 * I + I + f] = bf16_t(up & 0xffffu);
        a[p * I + f] = bf16_t(f2bf2(silu_f(g) * u, 0.f) & 0xffffu);
      }
  }
};

struct QDown {
  using ALoader = KcLoader<bf16_t>;
  using BLoader = KcLoaderQ4;
  const bf16_t* a; CodeRows w; const int32_t* offsets; bf16_t* ybuf;
  int H, E, I, NT;
  __device__ __forceinline__ bool tile(int L, MTile& t) const {
    if (!g2::grouped_tile<kTileM>(offsets, E, NT, L, t)) return false;
    t.kb = 0; t.ke = I; t.n0 = t.nt * kTileN; t.nc = min(kTileN, H - t.n0);
    return true;
  }
  __device__ __forceinline__ ActRows a_src(const MTile& t) const {
    return ActRows{a, nullptr, 1, t.off + t.m0, t.mc, I, I, false};
  }
  __device__ __forceinline__ DownCodes b_src(const MTile& t) const {
    return DownCodes{w, int64_t(t.e) * H, t.n0, H, I};
  }
  __device__ __forceinline__ void epilogue(const MTile& t, f32x16_t (&acc)[2][2], int wm, int wn,
                                           int lane) const {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = acc_col(wn, j, lane);
        if (col >= t.nc) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = acc_row(wm, i, r, lane);
          if (row >= t.mc) continue;
          ybuf[(t.off + t.m0 + row) * int64_t(H) + t.n0 + col] = bf16_t(f2bf2(acc[i][j][r], 0.f) & 0xffffu);
        }
      }
  }
};

template <class P>
static usaf_status launch(const P& p, int64_t tiles, hipStream_t st, int kclass) {
  if (tiles <= 0) return USAF_OK;
  const int64_t blocks = (tiles + 7) / 8 * 8;
  if (blocks >= (int64_t(1) << 31)) return USAF_ERR_UNSUPPORTED;
  timer_begin(kclass, st);
  hipLaunchKernelGGL(gemm_mfma_kernel<P>, dim3(unsigned(blocks)), dim3(256), 0, st, p);
  timer_end(kclass, st);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

static int log2_exact(int g) {
  int s = 0;
  while ((1 << s) < g) ++s;
  return s;
}

}  // namespace q4

usaf_status q4_gate_up(const usaf_moe_shape& s, const bf16_t* X, const usaf_q4_experts& w,
                       const int32_t* offsets, const int32_t* perm, bf16_t* gu, bf16_t* a,
                       hipStream_t st) {
  const int NT = int(ceil_div(s.I, q4::kTileN / 2));
  const int64_t S = int64_t(s.T) * s.K;
  const q4::CodeRows cr{w.q_gu, w.s_gu, w.z_gu, s.H / 2, s.H / w.group, q4::log2_exact(w.group)};
  q4::QGateUp p{X, cr, offsets, perm, gu, a, s.H, s.E, s.K, s.I, NT};
  return q4::launch(p, (ceil_div(S, q4::kTileM) + s.E) * NT, st, USAF_K_GATE_UP);
}

usaf_status q4_down(const usaf_moe_shape& s, const bf16_t* a, const usaf_q4_experts& w,
                    const int32_t* offsets, bf16_t* ybuf, hipStream_t st) {
  const int NT = int(ceil_div(s.H, q4::kTileN));
  const int64_t S = int64_t(s.T) * s.K;
  const q4::CodeRows cr{w.q_d, w.s_d, w.z_d, s.I / 2, s.I / w.group, q4::log2_exact(w.group)};
  q4::QDown p{a, cr, offsets, ybuf, s.H, s.E, s.I, NT};
  return q4::launch(p, (ceil_div(S, q4::kTileM) + s.E) * NT, st, USAF_K_DOWN);
}

}  // namespace usaf
