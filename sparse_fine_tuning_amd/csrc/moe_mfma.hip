// bf16 MFMA grouped GEMMs of the MoE layer (gfx950).
//
// The expert projections of the usaf README's fused tensors (gate_up
// [E, 2I, H], down [E, H, I]) as grouped GEMMs over the expert-major token
// grouping, with the SwiGLU forward and backward fused into the epilogues;
// the dense router GEMM; and the dense per-expert weight-gradient GEMMs of
// the importance / RigL scan.
#include "common.hpp"
#include "gemm_mfma.hpp"
#include "gemm_v2.hpp"
#include "moe_internal.hpp"
#include "timing.hpp"

namespace usaf {

// ---------------------------------------------------------------------------
// Operand sources
// ---------------------------------------------------------------------------
// Plain rows: row r at base + r*ld.
struct PlainRows {
  typedef bf16_t elem_t;
  const bf16_t* base; int64_t ld; int rows; int kend;
  __device__ __forceinline__ const bf16_t* row(int r) const { return base + int64_t(r) * ld; }
};
// fp32 router rows, rounded to bf16 while staging.
struct RouterRows {
  typedef float elem_t;
  const float* base; int64_t ld; int rows; int kend;
  __device__ __forceinline__ const float* row(int r) const { return base + int64_t(r) * ld; }
};
// ---------------------------------------------------------------------------
// Problems
// ---------------------------------------------------------------------------
// Router logits[T, E] = X bf16(Wr)^T, split over K into KS partial sums
// parts[ks][T][E] (k-range ks*Kc .. (ks+1)*Kc), summed later in fixed order.
struct MRouter {
  const bf16_t* X; const float* Wr; float* parts;
  int T, H, E, MT, NT, KS, Kc;
  using ALoader = KcLoader<bf16_t>;
  using BLoader = KcLoader<float>;
  __device__ bool tile(int L, MTile& t) const {
    if (L >= MT * NT * KS) return false;
    const int ks = L / (MT * NT);
    const int rem = L - ks * MT * NT;
    t.nt = rem / MT;
    t.m0 = (rem - t.nt * MT) * kMB;
    t.n0 = t.nt * kNB;
    t.mc = min(kMB, T - t.m0);
    t.nc = min(kNB, E - t.n0);
    t.kb = ks * Kc; t.ke = min(H, t.kb + Kc); t.e = ks; t.off = 0;
    return true;
  }
  __device__ PlainRows a_src(const MTile& t) const { return PlainRows{X + int64_t(t.m0) * H, H, t.mc, t.ke}; }
  __device__ RouterRows b_src(const MTile& t) const { return RouterRows{Wr + int64_t(t.n0) * H, H, t.nc, t.ke}; }
  __device__ void epilogue(const MTile& t, f32x16_t (&acc)[2][2], int wm, int wn, int lane) const {
    float* logits = parts + int64_t(t.e) * T * E;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = acc_col(wn, j, lane);
        if (col >= t.nc) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = acc_row(wm, i, r, lane);
          if (row < t.mc) logits[int64_t(t.m0 + row) * E + t.n0 + col] = acc[i][j][r];
        }
      }
  }
};

// ---------------------------------------------------------------------------
// Problems on the direct-to-LDS kernel (gemm_v2.hpp).  Row sources clamp to a
// valid row so every copy reads mapped memory; the epilogues store only rows
// and columns inside the tile.
// ---------------------------------------------------------------------------
namespace g2 {

// k-major rows gathered by token: row r -> act[tok(perm[base + min(r, n-1)])]
struct TokRowsC {
  const bf16_t* act; const int32_t* perm; int K; int base; int n; int64_t ld;
  __device__ __forceinline__ const bf16_t* row(int r) const {
    return act + int64_t(perm[base + min(r, n - 1)] / K) * ld;
  }
};
// k-major plain rows: row r -> base + min(r, n-1) * ld
struct PlainRowsC {
  const bf16_t* base; int64_t ld; int n;
  __device__ __forceinline__ const bf16_t* row(int r) const { return base + int64_t(min(r, n - 1)) * ld; }
};
// mn-major: element (col, k) at base + k*ld + col, ncols valid columns
struct StridedKC {
  const bf16_t* base; int64_t ld; int ncols;
  __device__ __forceinline__ const bf16_t* kptr(int k) const { return base + int64_t(k) * ld; }
};
// gate_up weight rows for a tile holding half as many features as columns:
// wave column wn (CW columns) holds features F0 + (CW/2) wn + [0, CW/2); its
// 32-column blocks alternate gate, up, gate, up over 32-feature groups.
template <int CW>
struct GateUpRowsC {
  const bf16_t* We; int F0; int I; int64_t H;
  __device__ __forceinline__ const bf16_t* row(int c) const {
    const int wn = c / CW, j = (c % CW) >> 5;
    const int f = min(F0 + (CW / 2) * wn + 32 * (j >> 1) + (c & 31), I - 1);
    return We + int64_t((j & 1) ? I + f : f) * H;
  }
};

template <int BM_, int BN_, int NS_, int WM_ = 2, int WN_ = 2, int BK_ = 64>
struct MGateUp {
  static constexpr int BM = BM_, BN = BN_, NS = NS_, WM = WM_, WN = WN_, NTHR = 64 * WM_ * WN_;
  static constexpr int kBlocksPerCU = Occupancy<BM_, BN_, BK_, NS_, WM_ * WN_>::kBlocksPerCU;
  static constexpr int kWavesPerEU = Occupancy<BM_, BN_, BK_, NS_, WM_ * WN_>::kWavesPerEU;
  static constexpr int RW = (BM / WM + 31) / 32 * 32, CW = BN / WN, IM = RW / 32, NJ = CW / 32;
  // two wave-rows share an odd number of row blocks evenly at run time
  static constexpr bool kSplit = WM_ == 2 && (BM_ / 32) % 2 == 1;
  using AOp = KMajor<BM, WM_ * WN_, BK_>;
  using BOp = KMajor<BN, WM_ * WN_, BK_>;
  const bf16_t* X; const bf16_t* Wgu; const int32_t* offsets; const int32_t* perm;
  bf16_t* gu; bf16_t* a;
  int H, E, K, I, NT;
  SplitWs sk;  // tail split partials (none: no split)
  static constexpr bool kTailSplit = true;
  __device__ __forceinline__ TailSplit split() const {
    return grouped_split_plan<BM, BK_>(offsets, E, NT, H, sk);
  }
  __device__ __forceinline__ bool tile(int L, MTile& t, const TailSplit& plan) const {
    if (!grouped_split_tile<BM, BK_>(offsets, E, NT, L, H, plan, t)) return false;
    t.n0 = t.nt * (BN / 2); t.nc = 0;
    return true;
  }
  // a contraction part [kb, ke): both operands' rows start at column kb
  __device__ __forceinline__ TokRowsC a_src(const MTile& t) const {
    return TokRowsC{X + t.kb, perm, K, t.off + t.m0, t.mc, H};
  }
  __device__ __forceinline__ GateUpRowsC<CW> b_src(const MTile& t) const {
    return GateUpRowsC<CW>{Wgu + int64_t(t.e) * 2 * I * H + t.kb, t.n0, I, H};
  }
  // persistent epilogue staging: one tensor's 32-row block (CW/2 features)
  static constexpr int kPStage =
      WaveRows<CW / 2>::kBytes * WM_ * WN_ <= (BM_ + BN_) * BK_ * 2 ? WaveRows<CW / 2>::kBytes : 0;
  static constexpr int kStageBytes = kPStage;
  __device__ __forceinline__ void epilogue(const MTile& t, f32x16_t (&acc)[IM][NJ], int wm, int wn, int lane,
                                           unsigned char* stage) const {
    static_assert(NJ % 2 == 0, "gate / up blocks of 32 features alternate");
    const int F = t.n0 + (CW / 2) * wn;  // first feature of this wave
    int r0, vb;
    wave_rows<kSplit, RW, IM>(t.mc, wm, r0, vb);
    static_for<IM>([&](auto I_) {
      constexpr int i = decltype(I_)::value;
      const int rb = r0 + 32 * i;
      if (kSplit ? i >= vb : rb >= t.mc) return;
      const int r = lane & 31, h = lane >> 5;
      // g, u (rounded once) and a = bf16(silu(g) u), as packed word pairs
      uint32_t gw[NJ / 2][4][2], uw[NJ / 2][4][2], aw[NJ / 2][4][2];
#pragma unroll
      for (int jp = 0; jp < NJ / 2; ++jp)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const uint32_t gp = pack_bf16x2(acc[i][2 * jp][4 * g + e], acc[i][2 * jp][4 * g + e + 1]);
            const uint32_t up = pack_bf16x2(acc[i][2 * jp + 1][4 * g + e], acc[i][2 * jp + 1][4 * g + e + 1]);
            const float g0 = __uint_as_float(gp << 16), g1 = __uint_as_float(gp & 0xffff0000u);
            const float u0 = __uint_as_float(up << 16), u1 = __uint_as_float(up & 0xffff0000u);
            gw[jp][g][e / 2] = gp;
            uw[jp][g][e / 2] = up;
            aw[jp][g][e / 2] = pack_bf16x2(silu_f(g0) * u0, silu_f(g1) * u1);
          }
      const int64_t p0 = t.off + t.m0 + rb;
      auto emit = [&](const uint32_t (&wv)[NJ / 2][4][2], bf16_t* base, int64_t ld, int coff) {
        if (stage) {
#pragma unroll
          for (int jp = 0; jp < NJ / 2; ++jp)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              WaveRows<CW / 2>::put2(stage, r, 32 * jp + 8 * g + 4 * h, wv[jp][g][0], wv[jp][g][1]);
          WaveRows<CW / 2>::drain(stage, lane, [&](int row, int c8, uint4 v) {
            if (rb + row < t.mc && F + c8 < I)
              *reinterpret_cast<uint4*>(base + (p0 + row) * ld + coff + F + c8) = v;
          });
        } else {
#pragma unroll
          for (int jp = 0; jp < NJ / 2; ++jp)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int c = 32 * jp + 8 * g + 4 * h;
              if (rb + r < t.mc && F + c < I)
                *reinterpret_cast<uint2*>(base + (p0 + r) * ld + coff + F + c) = make_uint2(wv[jp][g][0], wv[jp][g][1]);
            }
        }
      };
      emit(gw, gu, 2 * I, 0);
      emit(uw, gu, 2 * I, I);
      emit(aw, a, I, 0);
    });
  }
};

// bf16 [32 rows x CW] blocks of a wave's accumulators to rows base + row*ld:
// staged through the wave's LDS region (CW = 32 or 64), else 8-byte stores.
template <int IM, int NJ, int CW>
__device__ __forceinline__ void store_rows_bf16(const f32x16_t (&acc)[IM][NJ], unsigned char* stage, int r0,
                                                int vb, int lane, int mc, int ncw, bf16_t* base0,
                                                int64_t ld) {
  static_for<IM>([&](auto I_) {
    constexpr int i = decltype(I_)::value;
    const int rb = r0 + 32 * i;
    if (i >= vb) return;
    bf16_t* base = base0 + int64_t(rb) * ld;
    const int r = lane & 31, h = lane >> 5;
    if constexpr (CW == 32 || CW == 64) {
      if (stage) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            WaveRows<CW>::put2(stage, r, 32 * j + 8 * g + 4 * h,
                               pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                               pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]));
        WaveRows<CW>::drain(stage, lane, [&](int row, int c8, uint4 v) {
          if (rb + row < mc && c8 < ncw) *reinterpret_cast<uint4*>(base + row * ld + c8) = v;
        });
        return;
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 32 * j + 8 * g + 4 * h;
        if (rb + r < mc && c < ncw)
          *reinterpret_cast<uint2*>(base + r * ld + c) =
              make_uint2(pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                         pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]));
      }
  });
}

template <int BM_, int BN_, int NS_, int WM_ = 2, int WN_ = 2, int BK_ = 64>
struct MDown {
  static constexpr int BM = BM_, BN = BN_, NS = NS_, WM = WM_, WN = WN_, NTHR = 64 * WM_ * WN_;
  static constexpr int kBlocksPerCU = Occupancy<BM_, BN_, BK_, NS_, WM_ * WN_>::kBlocksPerCU;
  static constexpr int kWavesPerEU = Occupancy<BM_, BN_, BK_, NS_, WM_ * WN_>::kWavesPerEU;
  static constexpr int RW = (BM / WM + 31) / 32 * 32, CW = BN / WN, IM = RW / 32, NJ = CW / 32;
  // two wave-rows share an odd number of row blocks evenly at run time
  static constexpr bool kSplit = WM_ == 2 && (BM_ / 32) % 2 == 1;
  using AOp = KMajor<BM, WM_ * WN_, BK_>;
  using BOp = KMajor<BN, WM_ * WN_, BK_>;
  const bf16_t* a; const bf16_t* Wd; const int32_t* offsets; bf16_t* ybuf;
  int H, E, I, NT;
  SplitWs sk;  // tail split partials (none: no split)
  static constexpr bool kTailSplit = true;
  __device__ __forceinline__ TailSplit split() const {
    return grouped_split_plan<BM, BK_>(offsets, E, NT, I, sk);
  }
  __device__ __forceinline__ bool tile(int L, MTile& t, const TailSplit& plan) const {
    if (!grouped_split_tile<BM, BK_>(offsets, E, NT, L, I, plan, t)) return false;
    t.n0 = t.nt * BN; t.nc = min(BN, H - t.n0);
    return true;
  }
  __device__ __forceinline__ PlainRowsC a_src(const MTile& t) const {
    return PlainRowsC{a + int64_t(t.off + t.m0) * I + t.kb, I, t.mc};
  }
  __device__ __forceinline__ PlainRowsC b_src(const MTile& t) const {
    return PlainRowsC{Wd + (int64_t(t.e) * H + t.n0) * I + t.kb, I, t.nc};
  }
  // staging through one ring stage, where the wave's block fits there
  static constexpr int kPStage = ((CW == 32 || CW == 64) &&
                                  WaveRows<(CW == 32 ? 32 : 64)>::kBytes * WM_ * WN_ <= (BM_ + BN_) * BK_ * 2)
                                     ? WaveRows<(CW == 32 ? 32 : 64)>::kBytes : 0;
  static constexpr int kStageBytes = kPStage;
  __device__ __forceinline__ void epilogue(const MTile& t, f32x16_t (&acc)[IM][NJ], int wm, int wn, int lane,
                                           unsigned char* stage) const {
    int r0, vb;
    wave_rows<kSplit, RW, IM>(t.mc, wm, r0, vb);
    store_rows_bf16<IM, NJ, CW>(acc, stage, r0, vb, lane, t.mc, t.nc - wn * CW,
                                ybuf + int64_t(t.off + t.m0) * H + t.n0 + wn * CW, H);
  }
};

// The forward GEMMs on the pages' affine 4-bit storage (README "how it
// works": caching bullet, the trade between a resident dequantised copy and
// dequantising as the weights are used; quantisation recipe: codes in groups
// along the input dimension): the same problems with the weight operand read
// as codes and dequantised in LDS, a stage at a time (KMajorQ4).  A layer so
// computed equals, bit for bit, the same layer on the resident copy of the
// same codes: the weights are the same bf16 values, and every output
// accumulates the same MFMA chunks in the same order.
struct Q4Codes {
  const uint8_t* q; const uint16_t* s; const uint16_t* z;
  int64_t qpitch;  // bytes per code row (K / 2)
  int kg;          // groups per row (K / G)
  int gshift;      // log2(G)
  int kst0 = 0;    // first 64-wide stage of the tile's contraction
};
// gate_up code rows in the feature order of GateUpRowsC
template <int CW>
struct GateUpCodesC : Q4Codes {
  int64_t row0; int F0; int I;
  __device__ __forceinline__ int64_t code_row(int c) const {
    const int wn = c / CW, j = (c % CW) >> 5;
    const int f = min(F0 + (CW / 2) * wn + 32 * (j >> 1) + (c & 31), I - 1);
    return row0 + ((j & 1) ? I + f : f);
  }
};
// consecutive code rows: row r -> row0 + min(r, n - 1)
struct RowCodesC : Q4Codes {
  int64_t row0; int n;
  __device__ __forceinline__ int64_t code_row(int r) const { return row0 + min(r, n - 1); }
};

template <int BM_, int BN_, int NS_, int WM_, int WN_>
struct MGateUpQ4 : MGateUp<BM_, BN_, NS_, WM_, WN_, 64> {
  using Base = MGateUp<BM_, BN_, NS_, WM_, WN_, 64>;
  using BOp = KMajorQ4<BN_, WM_ * WN_>;
  static constexpr int kPStage =
      Base::kPStage * WM_ * WN_ <= Base::AOp::kBytes + BOp::kBytes ? Base::kPStage : 0;
  static constexpr int kStageBytes = kPStage;
  Q4Codes c;
  __device__ __forceinline__ GateUpCodesC<Base::CW> b_src(const MTile& t) const {
    GateUpCodesC<Base::CW> r{c, int64_t(t.e) * 2 * this->I, t.n0, this->I};
    r.kst0 = t.kb / 64;
    return r;
  }
};

template <int BM_, int BN_, int NS_, int WM_, int WN_>
struct MDownQ4 : MDown<BM_, BN_, NS_, WM_, WN_, 64> {
  using Base = MDown<BM_, BN_, NS_, WM_, WN_, 64>;
  using BOp = KMajorQ4<BN_, WM_ * WN_>;
  static constexpr int kPStage =
      Base::kPStage * WM_ * WN_ <= Base::AOp::kBytes + BOp::kBytes ? Base::kPStage : 0;
  static constexpr int kStageBytes = kPStage;
  Q4Codes c;
  __device__ __forceinline__ RowCodesC b_src(const MTile& t) const {
    RowCodesC r{c, int64_t(t.e) * this->H + t.n0, t.nc};
    r.kst0 = t.kb / 64;
    return r;
  }
};

template <int BM_, int BN_, int NS_, int WM_ = 2, int WN_ = 2, int BK_ = 64>
struct MDa {
  static constexpr int BM = BM_, BN = BN_, NS = NS_, WM = WM_, WN = WN_, NTHR = 64 * WM_ * WN_;
  static constexpr int kBlocksPerCU = Occupancy<BM_, BN_, BK_, NS_, WM_ * WN_>::kBlocksPerCU;
  static constexpr int kWavesPerEU = Occupancy<BM_, BN_, BK_, NS_, WM_ * WN_>::kWavesPerEU;
  static constexpr int RW = (BM / WM + 31) / 32 * 32, CW = BN / WN, IM = RW / 32, NJ = CW / 32;
  // two wave-rows share an odd number of row blocks evenly at run time
  static constexpr bool kSplit = WM_ == 2 && (BM_ / 32) % 2 == 1;
  using AOp = KMajor<BM, WM_ * WN_, BK_>;
  using BOp = MNMajor<BN, WM_ * WN_, BK_>;
  const bf16_t* dY; const bf16_t* Wd; const int32_t* offsets; const int32_t* perm;
  const float* topk_w; const bf16_t* gu; const bf16_t* a; bf16_t* dgu; float* dwpart;
  int H, E, K, I, NT, NTP;
  SplitWs sk;  // tail split partials (none: no split)
  static constexpr bool kTailSplit = true;
  __device__ __forceinline__ TailSplit split() const {
    return grouped_split_plan<BM, BK_>(offsets, E, NT, H, sk);
  }
  __device__ __forceinline__ bool tile(int L, MTile& t, const TailSplit& plan) const {
    if (!grouped_split_tile<BM, BK_>(offsets, E, NT, L, H, plan, t)) return false;
    t.n0 = t.nt * BN; t.nc = min(BN, I - t.n0);
    return true;
  }
  // a contraction part [kb, ke): dY's rows from column kb, W_d from row kb
  __device__ __forceinline__ TokRowsC a_src(const MTile& t) const {
    return TokRowsC{dY + t.kb, perm, K, t.off + t.m0, t.mc, H};
  }
  __device__ __forceinline__ StridedKC b_src(const MTile& t) const {
    return StridedKC{Wd + (int64_t(t.e) * H + t.kb) * I + t.n0, I, t.nc};
  }
  // staging through one ring stage, where the wave's block fits there
  static constexpr int kPStage = ((CW == 32 || CW == 64) &&
                                  WaveRows<(CW == 32 ? 32 : 64)>::kBytes * WM_ * WN_ <= (BM_ + BN_) * BK_ * 2)
                                     ? WaveRows<(CW == 32 ? 32 : 64)>::kBytes : 0;
  static constexpr int kStageBytes = kPStage;
  __device__ __forceinline__ void epilogue(const MTile& t, f32x16_t (&acc)[IM][NJ], int wm, int wn, int lane,
                                           unsigned char* stage) const {
    int r0, vb;
    wave_rows<kSplit, RW, IM>(t.mc, wm, r0, vb);
    static_for<IM>([&](auto I_) {
      constexpr int i = decltype(I_)::value;
      if (i >= vb) return;
      const int row = r0 + 32 * i + (lane & 31);
      const bool vrow = row < t.mc;
      const int64_t p = t.off + t.m0 + (vrow ? row : 0);
      const float wt = topk_w[perm[p]];
      float part = 0.f;
      uint32_t dgw[NJ][4][2], duw[NJ][4][2];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) dgw[j][g][0] = dgw[j][g][1] = duw[j][g][0] = duw[j][g][1] = 0u;
      // With 8 waves (two per SIMD) every saved g|u word of this row block
      // is loaded before the first dGU store, which could otherwise alias
      // them and serialise the loads (measured: 17% faster there, 4% slower
      // with one wave per SIMD, where they are loaded next to their use).
      // With a staging region the block's g and u rows come in as 16-byte
      // row pieces (8 rows per load) and are read back from LDS in the
      // output layout.
      constexpr bool kBatch = WM_ * WN_ >= 8;
      const bool staged = kPStage > 0 && stage != nullptr;
      uint2 gvs[NJ][4], uvs[NJ][4];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = out_col(CW, wn, j, g, lane);
          gvs[j][g] = uvs[j][g] = make_uint2(0u, 0u);
          if (staged || !kBatch || !vrow || col >= t.nc) continue;
          const int f = t.n0 + col;
          gvs[j][g] = *reinterpret_cast<const uint2*>(gu + p * 2 * I + f);
          uvs[j][g] = *reinterpret_cast<const uint2*>(gu + p * 2 * I + I + f);
        }
      if constexpr (kPStage > 0) {
        if (staged) {
          constexpr int NC = CW == 32 ? 32 : 64;
          using WR = WaveRows<NC>;
          const int rb0 = r0 + 32 * i, ncw0 = t.nc - wn * CW;
          const int lr = lane / WR::kLanesPerRow, lc = lane % WR::kLanesPerRow;
          const bf16_t* gbase = gu + int64_t(t.off + t.m0 + rb0) * 2 * I + t.n0 + wn * CW;
          uint4 gq[32 / WR::kRowsPerStore], uq[32 / WR::kRowsPerStore];
#pragma unroll
          for (int q = 0; q < 32 / WR::kRowsPerStore; ++q) {
            const int row = WR::kRowsPerStore * q + lr;
            gq[q] = uq[q] = make_uint4(0u, 0u, 0u, 0u);
            if (rb0 + row < t.mc && 8 * lc < ncw0) {
              gq[q] = *reinterpret_cast<const uint4*>(gbase + int64_t(row) * 2 * I + 8 * lc);
              uq[q] = *reinterpret_cast<const uint4*>(gbase + int64_t(row) * 2 * I + I + 8 * lc);
            }
          }
          auto back = [&](const uint4 (&rows)[32 / WR::kRowsPerStore], uint2 (&out)[NJ][4]) {
#pragma unroll
            for (int q = 0; q < 32 / WR::kRowsPerStore; ++q)
              *reinterpret_cast<uint4*>(stage + (WR::kRowsPerStore * q + lr) * WR::kPitch + 16 * lc) = rows[q];
            wave_lds_sync();
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
              for (int g = 0; g < 4; ++g)
                out[j][g] = *reinterpret_cast<const uint2*>(stage + (lane & 31) * WR::kPitch +
                                                            2 * (32 * j + 8 * g + 4 * (lane >> 5)));
            wave_lds_sync();
          };
          back(gq, gvs);
          back(uq, uvs);
        }
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = out_col(CW, wn, j, g, lane);
          if (!vrow || col >= t.nc) continue;
          const int f = t.n0 + col;
          // a = bf16(silu(g) u) is recomputed from the saved g|u exactly as the
          // forward epilogue rounded it, instead of being read back
          const uint2 gv = (kBatch || staged) ? gvs[j][g] : *reinterpret_cast<const uint2*>(gu + p * 2 * I + f);
          const uint2 uv = (kBatch || staged) ? uvs[j][g] : *reinterpret_cast<const uint2*>(gu + p * 2 * I + I + f);
          const uint32_t gw[2] = {gv.x, gv.y}, uw[2] = {uv.x, uv.y};
          uint32_t dg[2], du[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float dgs[2], dus[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const float U = acc[i][j][4 * g + 2 * h + q];
              const float g1 = q ? bf2f(bf16_t(gw[h] >> 16)) : bf2f(bf16_t(gw[h] & 0xffffu));
              const float u1 = q ? bf2f(bf16_t(uw[h] >> 16)) : bf2f(bf16_t(uw[h] & 0xffffu));
              const float sg = sigmoid_f(g1);
              const float av1 = bf2f(f2bf(g1 * sg * u1));
              part = fmaf(U, av1, part);
              const float da = wt * U;
              dgs[q] = da * u1 * sg * (1.f + g1 * (1.f - sg));
              dus[q] = da * g1 * sg;
            }
            dg[h] = pack_bf16x2(dgs[0], dgs[1]);
            du[h] = pack_bf16x2(dus[0], dus[1]);
          }
          dgw[j][g][0] = dg[0]; dgw[j][g][1] = dg[1];
          duw[j][g][0] = du[0]; duw[j][g][1] = du[1];
        }
      // dGU: the wave's 32 rows x CW columns of dg, then of du
      const int rb = r0 + 32 * i;
      const int ncw = t.nc - wn * CW;
      const int64_t p0 = t.off + t.m0 + rb;
      auto emit = [&](const uint32_t (&wv)[NJ][4][2], int coff) {
        bf16_t* base = dgu + p0 * 2 * I + coff + t.n0 + wn * CW;
        if constexpr (kPStage > 0) {
          if (stage) {
            constexpr int NC = CW == 32 ? 32 : 64;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
              for (int g = 0; g < 4; ++g)
                WaveRows<NC>::put2(stage, lane & 31, 32 * j + 8 * g + 4 * (lane >> 5), wv[j][g][0], wv[j][g][1]);
            WaveRows<NC>::drain(stage, lane, [&](int row, int c8, uint4 v) {
              if (rb + row < t.mc && c8 < ncw) *reinterpret_cast<uint4*>(base + row * 2 * I + c8) = v;
            });
            return;
          }
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = 32 * j + 8 * g + 4 * (lane >> 5);
            if (vrow && c < ncw)
              *reinterpret_cast<uint2*>(base + (lane & 31) * 2 * I + c) = make_uint2(wv[j][g][0], wv[j][g][1]);
          }
      };
      emit(dgw, 0);
      emit(duw, I);
      // lanes l and l + 32 hold the same row
      part += __shfl_xor(part, 32, 64);
      if (lane < 32 && vrow) dwpart[p * NTP + WN * t.nt + wn] = part;
    });
  }
};

template <int BM_, int BN_, int NS_, int WM_ = 2, int WN_ = 2, int BK_ = 64>
struct MDx {
  static constexpr int BM = BM_, BN = BN_, NS = NS_, WM = WM_, WN = WN_, NTHR = 64 * WM_ * WN_;
  static constexpr int kBlocksPerCU = Occupancy<BM_, BN_, BK_, NS_, WM_ * WN_>::kBlocksPerCU;
  static constexpr int kWavesPerEU = Occupancy<BM_, BN_, BK_, NS_, WM_ * WN_>::kWavesPerEU;
  static constexpr int RW = (BM / WM + 31) / 32 * 32, CW = BN / WN, IM = RW / 32, NJ = CW / 32;
  // two wave-rows share an odd number of row blocks evenly at run time
  static constexpr bool kSplit = WM_ == 2 && (BM_ / 32) % 2 == 1;
  using AOp = KMajor<BM, WM_ * WN_, BK_>;
  using BOp = MNMajor<BN, WM_ * WN_, BK_>;
  const bf16_t* dgu; const bf16_t* Wgu; const int32_t* offsets; bf16_t* vbuf;
  int H, E, I, NT;
  SplitWs sk;  // tail split partials (none: no split)
  static constexpr bool kTailSplit = true;
  __device__ __forceinline__ TailSplit split() const {
    return grouped_split_plan<BM, BK_>(offsets, E, NT, 2 * I, sk);
  }
  __device__ __forceinline__ bool tile(int L, MTile& t, const TailSplit& plan) const {
    if (!grouped_split_tile<BM, BK_>(offsets, E, NT, L, 2 * I, plan, t)) return false;
    t.n0 = t.nt * BN; t.nc = min(BN, H - t.n0);
    return true;
  }
  __device__ __forceinline__ PlainRowsC a_src(const MTile& t) const {
    return PlainRowsC{dgu + int64_t(t.off + t.m0) * 2 * I + t.kb, 2 * I, t.mc};
  }
  __device__ __forceinline__ StridedKC b_src(const MTile& t) const {
    return StridedKC{Wgu + (int64_t(t.e) * 2 * I + t.kb) * H + t.n0, H, t.nc};
  }
  // staging through one ring stage, where the wave's block fits there
  static constexpr int kPStage = ((CW == 32 || CW == 64) &&
                                  WaveRows<(CW == 32 ? 32 : 64)>::kBytes * WM_ * WN_ <= (BM_ + BN_) * BK_ * 2)
                                     ? WaveRows<(CW == 32 ? 32 : 64)>::kBytes : 0;
  static constexpr int kStageBytes = kPStage;
  __device__ __forceinline__ void epilogue(const MTile& t, f32x16_t (&acc)[IM][NJ], int wm, int wn, int lane,
                                           unsigned char* stage) const {
    int r0, vb;
    wave_rows<kSplit, RW, IM>(t.mc, wm, r0, vb);
    store_rows_bf16<IM, NJ, CW>(acc, stage, r0, vb, lane, t.mc, t.nc - wn * CW,
                                vbuf + int64_t(t.off + t.m0) * H + t.n0 + wn * CW, H);
  }
};

// Dense weight gradients of one expert, contraction over its slots p, with
// both operands expert-major slot rows (mn-major):
//   gate_up: dW[r, c] = sum_p dGU[p, r] Xg[p, c]    (rows 2I, cols H)
//   down:    dW[r, c] = sum_p wdYg[p, r] a[p, c]    (rows H,  cols I)
// Xg = X gathered by token and wdYg = bf16(w_p dY[tok(p)]) are staged first.
template <bool kDown, int BM_, int BN_, int NS_, int WM_ = 2, int WN_ = 2, int BK_ = 64>
struct MDenseDw {
  static constexpr int BM = BM_, BN = BN_, NS = NS_, WM = WM_, WN = WN_, NTHR = 64 * WM_ * WN_;
  static constexpr int kBlocksPerCU = Occupancy<BM_, BN_, BK_, NS_, WM_ * WN_>::kBlocksPerCU;
  static constexpr int kWavesPerEU = Occupancy<BM_, BN_, BK_, NS_, WM_ * WN_>::kWavesPerEU;
  static constexpr int RW = BM / WM, CW = BN / WN, IM = RW / 32, NJ = CW / 32;
  using AOp = MNMajor<BM, WM_ * WN_, BK_>;
  using BOp = MNMajor<BN, WM_ * WN_, BK_>;
  const bf16_t* L; const bf16_t* R; const int32_t* offsets; float* dW;
  int H, E, I, MT, NT;
  int64_t ngu;
  __device__ __forceinline__ int rows_total() const { return kDown ? H : 2 * I; }
  __device__ __forceinline__ int cols_total() const { return kDown ? I : H; }
  __device__ __forceinline__ bool tile(int Lt, MTile& t) const {
    const int per = MT * NT;
    t.e = Lt / per;
    if (t.e >= E) return false;
    const int rem = Lt - t.e * per;
    t.nt = rem / MT;
    t.m0 = (rem - t.nt * MT) * BM;
    t.n0 = t.nt * BN;
    t.mc = min(BM, rows_total() - t.m0);
    t.nc = min(BN, cols_total() - t.n0);
    t.off = offsets[t.e];
    t.kb = 0;
    t.ke = offsets[t.e + 1] - t.off;
    return true;
  }
  __device__ __forceinline__ StridedKC a_src(const MTile& t) const {
    const int ld = rows_total();
    return StridedKC{L + int64_t(t.off) * ld + t.m0, ld, t.mc};
  }
  __device__ __forceinline__ StridedKC b_src(const MTile& t) const {
    const int ld = cols_total();
    return StridedKC{R + int64_t(t.off) * ld + t.n0, ld, t.nc};
  }
  static constexpr int kStageBytes = 32 * (32 * NJ * 4 + 16);
  __device__ __forceinline__ void epilogue(const MTile& t, f32x16_t (&acc)[IM][NJ], int wm, int wn, int lane,
                                           unsigned char* stage) const {
    const int64_t obase = kDown ? ngu + int64_t(t.e) * H * I : int64_t(t.e) * 2 * I * H;
    const int ldo = cols_total();
    static_for<IM>([&](auto I_) {
      constexpr int i = decltype(I_)::value;
      const int rb = wm * RW + 32 * i;
      if (rb >= t.mc) return;
      const int ncw = t.nc - wn * CW;
      float* base = dW + obase + int64_t(t.m0 + rb) * ldo + t.n0 + wn * CW;
      const int64_t ld = ldo;
      stage_f32<NJ>(stage, acc[i], lane, [&](int row, int col, float4 v) {
        if (rb + row < t.mc && col < ncw) *reinterpret_cast<float4*>(base + row * ld + col) = v;
      });
    });
  }
};

// Expert-major operands of the dense gradient: Xg[p] = X[tok(p)],
// wdYg[p] = bf16(w_p dY[tok(p)]); 8 elements per thread.
__global__ __launch_bounds__(256) void stage_dense_kernel(const bf16_t* __restrict__ X,
                                                          const bf16_t* __restrict__ dY,
                                                          const int32_t* __restrict__ perm,
                                                          const float* __restrict__ topk_w,
                                                          int S, int H, int K,
                                                          bf16_t* __restrict__ Xg,
                                                          bf16_t* __restrict__ wdYg) {
  const int per_row = H / 8;
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= int64_t(S) * per_row) return;
  const int p = int(i / per_row), c = int(i - int64_t(p) * per_row) * 8;
  const int slot = perm[p];
  const int64_t src = int64_t(slot / K) * H + c;
  const float w = topk_w[slot];
  *reinterpret_cast<uint4*>(Xg + int64_t(p) * H + c) = *reinterpret_cast<const uint4*>(X + src);
  const uint4 v = *reinterpret_cast<const uint4*>(dY + src);
  const uint32_t in[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float lo = w * bf2f(bf16_t(in[q] & 0xffffu)), hi = w * bf2f(bf16_t(in[q] >> 16));
    o[q] = pack_bf16x2(lo, hi);
  }
  *reinterpret_cast<uint4*>(wdYg + int64_t(p) * H + c) = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace g2

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <class P>
static usaf_status launch_mfma(const P& p, int64_t tiles, hipStream_t st, int kclass) {
  if (tiles <= 0) return USAF_OK;
  const int64_t blocks = (tiles + 7) / 8 * 8;
  if (blocks >= (int64_t(1) << 31)) return USAF_ERR_UNSUPPORTED;
  timer_begin(kclass, st);
  hipLaunchKernelGGL(gemm_mfma_kernel<P>, dim3(unsigned(blocks)), dim3(256), 0, st, p);
  timer_end(kclass, st);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

template <class P>
static usaf_status launch_v2(const P& p, int64_t tiles, hipStream_t st, int kclass) {
  if (tiles <= 0) return USAF_OK;
  const int64_t blocks = (tiles + 7) / 8 * 8;
  if (blocks >= (int64_t(1) << 31)) return USAF_ERR_UNSUPPORTED;
  timer_begin(kclass, st);
  hipLaunchKernelGGL(g2::gemm2_kernel<P>, dim3(unsigned(blocks)), dim3(P::NTHR), 0, st, p);
  timer_end(kclass, st);
  USAF_LAUNCH_CHECK();
  return USAF_OK;
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// Persistent launch: about P::kBlocksPerCU blocks per CU (a multiple of 8
// for the XCD remap), never more blocks than tiles; with split_bytes of
// partial buffer at split_ws, the tail split (grouped_split_plan) and the
// reduction of the split tiles after the launch.
template <class P>
static usaf_status launch_persistent_split(P p, int64_t tiles, float* split_ws, size_t split_bytes,
                                           hipStream_t st, int kclass) {
  if (tiles <= 0) return USAF_OK;
  // the buffer's last 256 bytes hold the plan the launch records
  const size_t unit = size_t(P::NTHR) * P::IM * P::NJ * 16 * 4;  // a tile's accumulators
  const size_t cap = split_ws && split_bytes > 256 ? (split_bytes - 256) / unit : 0;
  int64_t blocks = int64_t(P::kBlocksPerCU) * device_cus();
  if (blocks > tiles) blocks = tiles;
  blocks = (blocks + 7) / 8 * 8;
  int* hdr = cap >= 2 ? reinterpret_cast<int*>(reinterpret_cast<char*>(split_ws) + split_bytes - 256) : nullptr;
  p.sk = g2::SplitWs{split_ws, int(cap < size_t(1 << 20) ? cap : size_t(1 << 20)), int(blocks), hdr};
  timer_begin(kclass, st);
  hipLaunchKernelGGL(g2::gemm2_persistent<P>, dim3(unsigned(blocks)), dim3(P::NTHR), 0, st, p);
  USAF_LAUNCH_CHECK();
  if (p.sk.cap >= 2) {  // the tail is at most half the grid: (G / 2) NW one-wave blocks
    const int64_t rblocks = (blocks / 2) * (P::NTHR / 64);
    hipLaunchKernelGGL(g2::gemm2_split_reduce<P>, dim3(unsigned(rblocks)), dim3(64), 0, st, p);
    USAF_LAUNCH_CHECK();
  }
  timer_end(kclass, st);
  return USAF_OK;
}

static int64_t grouped_tiles_bound(const usaf_moe_shape& s, int NT, int BM = kMB) {
  return (ceil_div(int64_t(s.T) * s.K, BM) + s.E) * NT;
}

usaf_status mfma_router(const usaf_moe_shape& s, const bf16_t* X, const float* Wr, float* parts,
                        int nparts, hipStream_t st) {
  const int MT = int(ceil_div(s.T, kMB)), NT = int(ceil_div(s.E, kNB));
  const int Kc = int(ceil_div(ceil_div(s.H, nparts), kKB) * kKB);
  return launch_mfma(MRouter{X, Wr, parts, s.T, s.H, s.E, MT, NT, nparts, Kc},
                     int64_t(MT) * NT * nparts, st, USAF_K_ROUTER_GEMM);
}

// Tile shapes and LDS ring depths of the direct-to-LDS GEMMs.
constexpr int kFwdBM = 160, kFwdBN = 256, kFwdNS = 3;  // gate_up, down, dA, dX: 156 KiB LDS
constexpr int kFwdWM = 2, kFwdWN = 4;                  // 8 waves: 2 per SIMD
constexpr int kFwdBK = 64;                             // contraction depth of a stage
constexpr int kDaWN = 4;                               // dA: 8 waves of 64 columns
constexpr int kDwBM = 256, kDwBN = 256, kDwNS = 3;     // dense dW: 3 stages of depth 32, 96 KiB LDS
constexpr int kDwBK = 32;

// Groups of at least kBigRows rows on average (few large experts) take
// 256-row tiles: twice the MFMA work per staged byte, and little ragged waste.
constexpr int kBigRows = 512;
constexpr int kBigBM = 256, kBigNS = 2, kBigBK = 64;  // 2 x 64 KiB LDS stages
constexpr int kBigWM = 2, kBigWN = 4;    // 8 waves of 128 x 64
static bool big_groups(const usaf_moe_shape& s) {
  return int64_t(s.T) * s.K >= int64_t(kBigRows) * s.E;
}

usaf_status mfma_gate_up(const usaf_moe_shape& s, const bf16_t* X, const bf16_t* Wgu,
                         const int32_t* offsets, const int32_t* perm, bf16_t* gu, bf16_t* a,
                         float* split_ws, size_t split_bytes, hipStream_t st) {
  const int NT = int(ceil_div(s.I, kFwdBN / 2));
  if (big_groups(s))
    return launch_persistent_split(
        g2::MGateUp<kBigBM, kFwdBN, kBigNS, kBigWM, kBigWN, kBigBK>{X, Wgu, offsets, perm, gu, a, s.H, s.E,
                                                                    s.K, s.I, NT},
        grouped_tiles_bound(s, NT, kBigBM), split_ws, split_bytes, st, USAF_K_GATE_UP);
  return launch_persistent_split(
      g2::MGateUp<kFwdBM, kFwdBN, kFwdNS, kFwdWM, kFwdWN, kFwdBK>{X, Wgu, offsets, perm, gu, a, s.H, s.E,
                                                                  s.K, s.I, NT},
      grouped_tiles_bound(s, NT, kFwdBM), split_ws, split_bytes, st, USAF_K_GATE_UP);
}

usaf_status mfma_down(const usaf_moe_shape& s, const bf16_t* a, const bf16_t* Wd,
                      const int32_t* offsets, bf16_t* ybuf, float* split_ws, size_t split_bytes,
                      hipStream_t st) {
  const int NT = int(ceil_div(s.H, kFwdBN));
  if (big_groups(s))
    return launch_persistent_split(
        g2::MDown<kBigBM, kFwdBN, kBigNS, kBigWM, kBigWN, kBigBK>{a, Wd, offsets, ybuf, s.H, s.E, s.I, NT},
        grouped_tiles_bound(s, NT, kBigBM), split_ws, split_bytes, st, USAF_K_DOWN);
  return launch_persistent_split(
      g2::MDown<kFwdBM, kFwdBN, kFwdNS, kFwdWM, kFwdWN, kFwdBK>{a, Wd, offsets, ybuf, s.H, s.E, s.I, NT},
      grouped_tiles_bound(s, NT, kFwdBM), split_ws, split_bytes, st, USAF_K_DOWN);
}

int mfma_dw_partials(const usaf_moe_shape& s) { return kDaWN * int(ceil_div(s.I, kFwdBN)); }

usaf_status mfma_da(const usaf_moe_shape& s, const bf16_t* dY, const bf16_t* Wd,
                    const int32_t* offsets, const int32_t* perm, const float* topk_w,
                    const bf16_t* gu, const bf16_t* a, bf16_t* dgu, float* dwpart,
                    float* split_ws, size_t split_bytes, hipStream_t st) {
  // dA keeps the 160-row tiles for large groups too: its epilogue's g|u
  // loads spill on 256-row tiles (measured 13% slower at the Mixtral shape)
  const int NT = int(ceil_div(s.I, kFwdBN));
  return launch_persistent_split(
      g2::MDa<kFwdBM, kFwdBN, kFwdNS, 2, kDaWN, kFwdBK>{dY, Wd, offsets, perm, topk_w, gu, a, dgu, dwpart,
                                                        s.H, s.E, s.K, s.I, NT, kDaWN * NT},
      grouped_tiles_bound(s, NT, kFwdBM), split_ws, split_bytes, st, USAF_K_DA);
}

usaf_status mfma_dx(const usaf_moe_shape& s, const bf16_t* dgu, const bf16_t* Wgu,
                    const int32_t* offsets, bf16_t* vbuf, float* split_ws, size_t split_bytes,
                    hipStream_t st) {
  const int NT = int(ceil_div(s.H, kFwdBN));
  if (big_groups(s))
    return launch_persistent_split(
        g2::MDx<kBigBM, kFwdBN, kBigNS, kBigWM, kBigWN, kBigBK>{dgu, Wgu, offsets, vbuf, s.H, s.E, s.I, NT},
        grouped_tiles_bound(s, NT, kBigBM), split_ws, split_bytes, st, USAF_K_DX);
  return launch_persistent_split(
      g2::MDx<kFwdBM, kFwdBN, kFwdNS, kFwdWM, kFwdWN, kFwdBK>{dgu, Wgu, offsets, vbuf, s.H, s.E, s.I, NT},
      grouped_tiles_bound(s, NT, kFwdBM), split_ws, split_bytes, st, USAF_K_DX);
}

usaf_status mfma_dense_dw(const usaf_moe_shape& s, const bf16_t* X, const bf16_t* dY,
                          const bf16_t* dgu, const bf16_t* a, const int32_t* offsets,
                          const int32_t* perm, const float* topk_w, bf16_t* stage, float* dW,
                          hipStream_t st) {
  const int64_t ngu = int64_t(s.E) * 2 * s.I * s.H;
  const int64_t S = int64_t(s.T) * s.K;
  bf16_t* Xg = stage;
  bf16_t* wdYg = stage + S * s.H;
  timer_begin(USAF_K_DENSE_DW, st);
  {
    const int64_t n = S * (s.H / 8);
    hipLaunchKernelGGL(g2::stage_dense_kernel, dim3(unsigned(ceil_div(n, 256))), dim3(256), 0, st,
                       X, dY, perm, topk_w, int(S), s.H, s.K, Xg, wdYg);
    USAF_LAUNCH_CHECK();
  }
  {
    const int MT = int(ceil_div(2 * s.I, kDwBM)), NT = int(ceil_div(s.H, kDwBN));
    g2::MDenseDw<false, kDwBM, kDwBN, kDwNS, 2, 2, kDwBK> p{dgu, Xg, offsets, dW, s.H, s.E, s.I, MT, NT, ngu};
    USAF_TRY(launch_v2(p, int64_t(MT) * NT * s.E, st, -1));
  }
  {
    const int MT = int(ceil_div(s.H, kDwBM)), NT = int(ceil_div(s.I, kDwBN));
    g2::MDenseDw<true, kDwBM, kDwBN, kDwNS, 2, 2, kDwBK> p{wdYg, a, offsets, dW, s.H, s.E, s.I, MT, NT, ngu};
    USAF_TRY(launch_v2(p, int64_t(MT) * NT * s.E, st, -1));
  }
  timer_end(USAF_K_DENSE_DW, st);
  return USAF_OK;
}

// The 4-bit forward GEMMs: the ring holds the activations only (3 stages,
// 60 KiB, for 160-row tiles; 2 stages, 64 KiB, for 256-row ones), beside
// three code buffers (3 x 8 KiB for 256 weight rows), three scale buffers
// (3 x 2 KiB) and two converted bf16 stages (2 x 32 KiB).
constexpr int kQ4NS = 3, kQ4BigNS = 2;

static int log2_exact(int g) {
  int s = 0;
  while ((1 << s) < g) ++s;
  return s;
}

usaf_status q4_gate_up(const usaf_moe_shape& s, const bf16_t* X, const usaf_q4_experts& w,
                       const int32_t* offsets, const int32_t* perm, bf16_t* gu, bf16_t* a,
                       float* split_ws, size_t split_bytes, hipStream_t st) {
  // the same tiles, grid and tail split as mfma_gate_up
  const int NT = int(ceil_div(s.I, kFwdBN / 2));
  const g2::Q4Codes c{w.q_gu, w.s_gu, w.z_gu, s.H / 2, s.H / w.group, log2_exact(w.group)};
  if (big_groups(s)) {
    using P = g2::MGateUpQ4<kBigBM, kFwdBN, kQ4BigNS, kBigWM, kBigWN>;
    static_assert(P::kBlocksPerCU == g2::MGateUp<kBigBM, kFwdBN, kBigNS, kBigWM, kBigWN, kBigBK>::kBlocksPerCU,
                  "the 4-bit and bf16 gate_up launches share their grid");
    const P p{{X, nullptr, offsets, perm, gu, a, s.H, s.E, s.K, s.I, NT}, c};
    return launch_persistent_split(p, grouped_tiles_bound(s, NT, kBigBM), split_ws, split_bytes, st,
                                   USAF_K_GATE_UP);
  }
  using P = g2::MGateUpQ4<kFwdBM, kFwdBN, kQ4NS, kFwdWM, kFwdWN>;
  static_assert(P::kBlocksPerCU == g2::MGateUp<kFwdBM, kFwdBN, kFwdNS, kFwdWM, kFwdWN, kFwdBK>::kBlocksPerCU,
                "the 4-bit and bf16 gate_up launches share their grid");
  const P p{{X, nullptr, offsets, perm, gu, a, s.H, s.E, s.K, s.I, NT}, c};
  return launch_persistent_split(p, grouped_tiles_bound(s, NT, kFwdBM), split_ws, split_bytes, st,
                                 USAF_K_GATE_UP);
}

usaf_status q4_down(const usaf_moe_shape& s, const bf16_t* a, const usaf_q4_experts& w,
                    const int32_t* offsets, bf16_t* ybuf, float* split_ws, size_t split_bytes,
                    hipStream_t st) {
  // the same tiles, grid and tail split as mfma_down: the same sums in the
  // same order
  const int NT = int(ceil_div(s.H, kFwdBN));
  const g2::Q4Codes c{w.q_d, w.s_d, w.z_d, s.I / 2, s.I / w.group, log2_exact(w.group)};
  if (big_groups(s)) {
    using P = g2::MDownQ4<kBigBM, kFwdBN, kQ4BigNS, kBigWM, kBigWN>;
    static_assert(P::kBlocksPerCU == g2::MDown<kBigBM, kFwdBN, kBigNS, kBigWM, kBigWN, kBigBK>::kBlocksPerCU,
                  "the 4-bit and bf16 down launches share their grid");
    const P p{{a, nullptr, offsets, ybuf, s.H, s.E, s.I, NT}, c};
    return launch_persistent_split(p, grouped_tiles_bound(s, NT, kBigBM), split_ws, split_bytes, st,
                                   USAF_K_DOWN);
  }
  using P = g2::MDownQ4<kFwdBM, kFwdBN, kQ4NS, kFwdWM, kFwdWN>;
  static_assert(P::kBlocksPerCU == g2::MDown<kFwdBM, kFwdBN, kFwdNS, kFwdWM, kFwdWN, kFwdBK>::kBlocksPerCU,
                "the 4-bit and bf16 down launches share their grid");
  const P p{{a, nullptr, offsets, ybuf, s.H, s.E, s.I, NT}, c};
  return launch_persistent_split(p, grouped_tiles_bound(s, NT, kFwdBM), split_ws, split_bytes, st,
                                 USAF_K_DOWN);
}

}  // namespace usaf
