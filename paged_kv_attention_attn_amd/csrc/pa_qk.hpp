// Score / softmax / P.V machinery shared by the decode kernels (fixed-partition grid and
// balanced persistent workers): the two ways to form q.k on gfx950 (vector ALUs or matrix cores)
// and the per-row-group online softmax with fp32 P.V on the vector ALUs.
//
// Each policy holds the q operand and a wave's online-softmax state, and provides
//   init(p, b, h0, lane, qflip, c2)   load q for query heads [h0, h0+G) of sequence b, reset state
//   issue(tile, kb, vb, lane)         start the loads of one 16-token tile of K and V
//   consume<MASKED>(tile, ...)        fold the tile into the state (MASKED: select tokens in
//                                     [lo, hi), NaN-safe)
//   merge_rows(M, l)                  merge the 4 row groups; row-0 lanes end with the wave's
//                                     (max, sum, acc) of every head
// Online softmax reaching the plain softmax in another order: vllm.cpp PR #564
// "spec(BACKEND-ROCM): the ROCm head_dim=128 decode arm", "It is a mirror of merged work, not new
// design"; a separate matrix-core arm for d=128: same page, "One deviation from the original
// commit"; wave64 reductions crossing all four 16-lane rows: vllm.cpp PR #506 review, finding 2.
#pragma once

#include <type_traits>

#include "pa_device.hpp"
#include "pa_kernels.hpp"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Rescale threshold of the online softmax, in log2 units.  A row group's running max m is only
// raised when a tile's max exceeds it by more than this, so between raises
// p = 2^(s - m) <= 2^kRescaleSlack (no overflow risk in fp32) and most tiles skip the rescale
// multiplies.  The result does not depend on when rescales happen: every (m, l, acc) triple
// stays consistent and the merges use the exact log-sum-exp rule.
constexpr float kRescaleSlack = 8.0f;

// value of x in lane H of this lane's 16-lane row (DPP row_newbcast)
template <int H>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), 0x150 + H, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_bcast_dyn(float x, int h) {
  switch (h) {   // h is a compile-time constant after unrolling
    case 0: return row_bcast<0>(x);
    case 1: return row_bcast<1>(x);
    case 2: return row_bcast<2>(x);
    case 3: return row_bcast<3>(x);
    case 4: return row_bcast<4>(x);
    case 5: return row_bcast<5>(x);
    case 6: return row_bcast<6>(x);
    default: return row_bcast<7>(x);
  }
}

// V rows of a tile in the P.V layout: row group r (lane / 16) holds tokens 4j + r, lane c of the
// row holds slice c of the head dim.
template <int D, bool NT = true>
__device__ __forceinline__ void load_v_rows(uint32_t (&v)[kTileSteps][RowGeom<D>::kWords],
                                            const char* vb, int lane, int rs) {
  const int r = lane >> 4, c = lane & 15;
#pragma unroll
  for (int j = 0; j < kTileSteps; ++j)
    load_row<D, NT>(vb + (kRows * j + r) * rs, c, v[j]);
}

template <int NWORDS>
__device__ __forceinline__ void mask_v_words(uint32_t (&v)[kTileSteps][NWORDS], int tok0, int lo,
                                             int hi, int lane) {
#pragma unroll
  for (int j = 0; j < kTileSteps; ++j) {
    const int tk = tok0 + kRows * j + (lane >> 4);
    const bool ok = tk >= lo && tk < hi;
#pragma unroll
    for (int w = 0; w < NWORDS; ++w) v[j][w] = ok ? v[j][w] : 0u;
  }
}

template <int D>
__device__ __forceinline__ void mask_v_rows(uint32_t (&v)[kTileSteps][RowGeom<D>::kWords],
                                            int tok0, int lo, int hi, int lane) {
  mask_v_words<RowGeom<D>::kWords>(v, tok0, lo, hi, lane);
}

// ---------------------------------------------------------------------------------------------
// QK^T on the vector ALUs.  State per lane: (m, l) for each of the G heads of its row group,
// acc[G][E] for its head-dim slice.
// ---------------------------------------------------------------------------------------------
template <int D, int G>
struct QkValu {
  static constexpr int W = RowGeom<D>::kWords;
  static constexpr int E = RowGeom<D>::kElems;
  static constexpr int kRowBytes = RowGeom<D>::kRowBytes;
  static constexpr int kMinWavesPerEu = 1;
  static constexpr bool kColumns = false;   // one query token, flush by heads (out)
  static constexpr bool kQueryTokens = false;
  struct Tile {
    uint32_t k[kTileSteps][W];
    uint32_t v[kTileSteps][W];
  };
  uint32_t qw[G][W];
  float c2;
  float m[G], l[G], acc[G][E];

  __device__ __forceinline__ void load_q(const DecodeParams& p, int b, int h0, int lane,
                                         uint32_t qflip) {
    const int c = lane & 15;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      load_row_cached<D>(
          reinterpret_cast<const char*>(p.q + ((size_t)b * p.num_q_heads + h0 + h) * D), c,
          qw[h]);
#pragma unroll
      for (int w = 0; w < W; ++w) qw[h][w] ^= qflip;
    }
  }
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
    }
  }
  int rs;   // bytes between a block's consecutive K/V rows (the pool layout's row stride)
  __device__ __forceinline__ void load_q(const DecodeParams& p, const QShape&, int b, int h0,
                                         int lane, uint32_t qflip) {
    load_q(p, b, h0, lane, qflip);
  }
  __device__ __forceinline__ void init(const DecodeParams& p, const QShape&, int b, int h0,
                                       int lane, uint32_t qflip, float c2_) {
    c2 = c2_;
    rs = (int)p.kv_row_stride;
    load_q(p, b, h0, lane, qflip);
    reset();
  }

  __device__ __forceinline__ void issue(Tile& t, const char* kb, const char* vb, int lane) const {
    const int r = lane >> 4, c = lane & 15;
#pragma unroll
    for (int j = 0; j < kTileSteps; ++j)
      load_row<D>(kb + (kRows * j + r) * rs, c, t.k[j]);
    load_v_rows<D>(t.v, vb, lane, rs);
  }

  template <bool MASKED>
  __device__ __forceinline__ void consume(Tile& t, int tok0, int lo, int hi, int lane) {
    constexpr int J = kTileSteps;
    const int r = lane >> 4;
    float s[J][G];
#pragma unroll
    for (int j = 0; j < J; ++j) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) a = dot2_bf16(qw[h][w], t.k[j][w], a);
        s[j][h] = row_sum16(a);
      }
    }
    if constexpr (MASKED) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int tk = tok0 + kRows * j + r;
        const bool ok = tk >= lo && tk < hi;
#pragma unroll
        for (int h = 0; h < G; ++h) s[j][h] = ok ? s[j][h] * c2 : -INFINITY;
      }
      mask_v_rows<D>(t.v, tok0, lo, hi, lane);
    }
    float mx[G];
    bool need = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mx[h] = fmaxf(fmaxf(s[0][h], s[1][h]), fmaxf(s[2][h], s[3][h]));
      if constexpr (!MASKED) mx[h] *= c2;    // c2 >= 0 commutes with max
      need |= mx[h] > m[h] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], mx[h]);
        const float mu = mn == -INFINITY ? 0.f : mn;
        const float alpha = fast_exp2(m[h] - mu);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
        m[h] = mn;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mu = m[h] == -INFINITY ? 0.f : m[h];
#pragma unroll
      for (int j = 0; j < J; ++j)
        s[j][h] = MASKED ? fast_exp2(s[j][h] - mu) : fast_exp2(fmaf(s[j][h], c2, -mu));
      l[h] += (s[0][h] + s[1][h]) + (s[2][h] + s[3][h]);
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      float vf[E];
#pragma unroll
      for (int w = 0; w < W; ++w) {
        vf[2 * w] = bf16_lo(t.v[j][w]);
        vf[2 * w + 1] = bf16_hi(t.v[j][w]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = fmaf(s[j][h], vf[e], acc[h][e]);
      }
    }
  }

  // Merge the 4 row groups; lanes of row 0 end with the wave's (M, l, acc) of every head.
  __device__ __forceinline__ void merge_rows(float (&Mh)[G], float (&lh)[G]) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float M = rows_max(m[h]);
      const float f = fast_exp2(m[h] - (M == -INFINITY ? 0.f : M));
      lh[h] = rows_sum(l[h] * f);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = rows_sum(acc[h][e] * f);
      Mh[h] = M;
    }
  }
  // After merge_rows, on the row-0 lanes: the accumulated P.V of head h at dim(lane, e).
  __device__ __forceinline__ float out(int h, int e) const { return acc[h][e]; }
};

// ---------------------------------------------------------------------------------------------
// QK^T on the matrix cores.  For the 16x16x32 bf16 MFMA, lane l holds A[l%16][8(l/16)+i],
// B[8(l/16)+i][l%16] and C[4(l/16)+i][l%16] (checked on gfx950).  MFMA row m of a tile is token
// 4(m%4) + m/4, so the four scores a lane gets back (C rows 4g+i, g = l/16) are tokens 4i+g: the
// tokens its row group handles in the P.V layout.  The k order inside the contraction is free
// (A and B share it): chunk 4kk + l/16 of the head dim for MFMA kk, so each lane reads whole
// 16-byte pieces of K rows and q.  State per lane: (m, l) of head l%16 for row group l/16, and
// acc[G][E] in the P.V layout; probabilities reach the P.V layout by row_newbcast.
// ---------------------------------------------------------------------------------------------
template <int D, int G>
struct QkMfma {
  static constexpr int KK = D / 32;
  static constexpr int W = RowGeom<D>::kWords;
  static constexpr int E = RowGeom<D>::kElems;
  static constexpr int kRowBytes = RowGeom<D>::kRowBytes;
  static constexpr int kMinWavesPerEu = 1;
  static constexpr bool kColumns = false;   // one query token, flush by heads (out)
  static constexpr bool kQueryTokens = false;
  struct Tile {
    u32x4_t k[KK];
    uint32_t v[kTileSteps][W];
  };
  u32x4_t qb[KK];
  float c2;
  bool head_lane;
  float m, l, acc[G][E];

  __device__ __forceinline__ void load_q(const DecodeParams& p, int b, int h0, int lane,
                                         uint32_t qflip) {
    const int n = lane & 15;
    head_lane = n < G;
    const char* qrow = reinterpret_cast<const char*>(
        p.q + ((size_t)b * p.num_q_heads + h0 + (head_lane ? n : 0)) * D);
    const uint32_t keep = head_lane ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(qrow + 64 * kk + 16 * (lane >> 4));
      x.x = (x.x ^ qflip) & keep;
      x.y = (x.y ^ qflip) & keep;
      x.z = (x.z ^ qflip) & keep;
      x.w = (x.w ^ qflip) & keep;
      qb[kk] = x;
    }
  }
  __device__ __forceinline__ void reset() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
    }
  }
  int rs;   // bytes between a block's consecutive K/V rows (the pool layout's row stride)
  __device__ __forceinline__ void load_q(const DecodeParams& p, const QShape&, int b, int h0,
                                         int lane, uint32_t qflip) {
    load_q(p, b, h0, lane, qflip);
  }
  __device__ __forceinline__ void init(const DecodeParams& p, const QShape&, int b, int h0,
                                       int lane, uint32_t qflip, float c2_) {
    c2 = c2_;
    rs = (int)p.kv_row_stride;
    load_q(p, b, h0, lane, qflip);
    reset();
  }

  __device__ __forceinline__ void issue(Tile& t, const char* kb, const char* vb, int lane) const {
    const int mrow = lane & 15;
    const int tok = 4 * (mrow & 3) + (mrow >> 2);
    const char* krow = kb + tok * rs + 16 * (lane >> 4);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      t.k[kk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(krow + 64 * kk));
    load_v_rows<D>(t.v, vb, lane, rs);
  }

  template <bool MASKED>
  __device__ __forceinline__ void consume(Tile& t, int tok0, int lo, int hi, int lane) {
    const int g = lane >> 4;
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, t.k[kk]),
                                                   __builtin_bit_cast(bf16x8_t, qb[kk]), sc, 0,
                                                   0, 0);
    if constexpr (MASKED) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tk = tok0 + 4 * i + g;
        sc[i] = (tk >= lo && tk < hi) ? sc[i] * c2 : -INFINITY;
      }
      mask_v_rows<D>(t.v, tok0, lo, hi, lane);
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if constexpr (!MASKED) mx *= c2;
    const bool need = head_lane && mx > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float mn = fmaxf(m, mx);
      const float alpha = fast_exp2(m - (mn == -INFINITY ? 0.f : mn));
      l *= alpha;
      m = mn;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float a_h = row_bcast_dyn(alpha, h);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] *= a_h;
      }
    }
    const float mu = m == -INFINITY ? 0.f : m;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pr[i] = MASKED ? fast_exp2(sc[i] - mu) : fast_exp2(fmaf(sc[i], c2, -mu));
    l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
#pragma unroll
    for (int j = 0; j < kTileSteps; ++j) {
      float vf[E];
#pragma unroll
      for (int w = 0; w < W; ++w) {
        vf[2 * w] = bf16_lo(t.v[j][w]);
        vf[2 * w + 1] = bf16_hi(t.v[j][w]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pb = row_bcast_dyn(pr[j], h);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = fmaf(pb, vf[e], acc[h][e]);
      }
    }
  }

  // Merge the 4 row groups; lanes of row 0 end with the wave's (M, l, acc) of every head.
  __device__ __forceinline__ void merge_rows(float (&Mh)[G], float (&lh)[G]) {
    const float M = rows_max(m);
    const float f = fast_exp2(m - (M == -INFINITY ? 0.f : M));
    const float lt = rows_sum(l * f);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float f_h = row_bcast_dyn(f, h);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = rows_sum(acc[h][e] * f_h);
      Mh[h] = row_bcast_dyn(M, h);
      lh[h] = row_bcast_dyn(lt, h);
    }
  }
  // After merge_rows, on the row-0 lanes: the accumulated P.V of head h at dim(lane, e).
  __device__ __forceinline__ float out(int h, int e) const { return acc[h][e]; }
};

// ---------------------------------------------------------------------------------------------
// q.k and P.V both on the matrix cores.  q.k as in QkMfma.  P.V uses the 16x16x16 bf16 MFMA
// (lane l holds A[l%16][4(l/16)+j], B[4(l/16)+j][l%16], C[4(l/16)+i][l%16]; checked on gfx950)
// with the probabilities as A (row = query head l%16, k = 4(l/16)+j = token 4j+l/16: exactly the
// scores the lane holds after q.k) and V as B (column c of MFMA e = head-dim index dim(c, e);
// k = 4g+j is token 4j+g, the rows row group g loads).  P is split into two bf16 terms,
// p = hi + lo, each multiplied exactly and accumulated in fp32, so the product keeps about
// 16 bits of p (relative error below 2^-16) instead of bf16's 8.  All row groups feed the same
// accumulator, so they share one running max per head (raised, lazily, from the wave-wide tile
// max); each keeps its own partial sum of p.  State per lane: m and l of head l%16, and
// cacc[e] = C rows 4(l/16)+i (heads), column l%16 (dim(l%16, e)).
// ---------------------------------------------------------------------------------------------
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two OCP FP8 E4M3 codes (the low or the high half of a word) -> a bf16 pair, exactly: an E4M3
// value has at most four significant bits and an exponent inside bf16's range, and with a
// scale of 1 gfx950's scaled conversion (v_cvt_scalef32_pk_bf16_fp8) is the plain decoding (a
// NaN code gives a NaN).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// Eight codes (two words) -> eight bf16 (four words), in order.
__device__ __forceinline__ u32x4_t fp8x8_to_bf16x8(u32x2_t x) {
  u32x4_t r;
  r.x = fp8x2_to_bf16x2<false>(x.x);
  r.y = fp8x2_to_bf16x2<true>(x.x);
  r.z = fp8x2_to_bf16x2<false>(x.y);
  r.w = fp8x2_to_bf16x2<true>(x.y);
  return r;
}

// FP8 = true: the KV cache holds OCP FP8 E4M3 codes (one byte per value, rows of D bytes) with
// one fp32 scale per tensor.  K and V are converted to bf16 in registers (exactly) and go
// through the same MFMAs; the K scale is folded into the score scale by the host and the V
// scale multiplies the output.  NT: K/V loads carry the non-temporal hint (rows read once).
// HP = 2 (one query token): a unit is a pair of adjacent KV heads, G = 2 * group columns
// (the query heads of both, in order), and a tile holds both heads' 16-token K and V rows.  Each
// head's K runs its own score MFMAs and each lane keeps the scores of its column's head; each
// head's V runs its own P.V MFMAs into its own accumulators, whose rows of the other head's
// columns are never read.  (Masking the operands instead would let 0 x NaN from one head's
// rows reach the other's.)  A step then streams two heads' rows, the bytes of one head_dim-256
// tile at head_dim 128, for the same per-byte work.
template <int D, int G, bool FP8, bool NT = true, int HP = 1>
struct QkMfmaPvT {
  static constexpr int KK = D / 32;
  static constexpr int W = RowGeom<D>::kWords;
  static constexpr int E = RowGeom<D>::kElems;
  static constexpr int kRowBytes = FP8 ? D : 2 * D;
  // Occupancy floor handed to the compiler.  A floor of two caps a wave at 256 registers,
  // which also makes it keep the MFMA accumulators in ordinary VGPRs instead of copying them
  // to and from AGPRs around every branch of the tile loop.  For FP8 tiles (half the bytes per
  // tile, so the per-tile instruction stream weighs twice as much) that pays; a floor of three
  // (168 registers at D = 128, with two spilled) measured no better.
  static constexpr int kMinWavesPerEu = FP8 && D <= 128 ? 2 : 1;
  static_assert(HP == 1 || (HP == 2 && G <= 8), "head pairs: head-wise columns");
  static constexpr int VW = FP8 ? E / 4 : W;   // words a lane holds of one V row
  static_assert(!FP8 || E == 4 * VW, "an FP8 lane slice is whole words");
  // K: bf16, one 16-byte piece per score MFMA; FP8, one 16-byte piece per two (halves)
  static constexpr int KL = FP8 ? KK / 2 : KK;
  struct TileHead {
    u32x4_t k[KL];
    uint32_t v[kTileSteps][VW];
  };
  struct Tile {
    TileHead x[HP];
  };
  // Columns: the N side of both contractions is (query token, head) pairs, n = i * group + h,
  // G of them at most (q_len * group <= G <= 16); with one query token a column is a head.
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "columns");
  // Sixteen columns live in all four row groups: flush them column-wise (merge_cols, col_m,
  // acc).  Up to eight, the head-wise flush (merge_rows, out) keeps the finishing values in
  // scalar registers and costs about 28 fewer VGPRs.
  static constexpr bool kColumns = G == 16;
  static constexpr bool kQueryTokens = true;   // columns may be several query tokens
  static constexpr int kHalves = 1;
  static constexpr int kHeads = HP;
  u32x4_t qb[KK];
  bool half1;                        // head pairs: this lane's column belongs to the second head
  int64_t pair_off;                  // head pairs: bytes from a pair's first head to its second
  float c2;
  float vs;   // FP8: V scale
  bool head_lane;
  int col_q;  // query token of this lane's column
  float m, l;
  float lsum;  // after merge_cols: the column's sum over the row groups
  f32x4_t cacc[E];
  f32x4_t cacc1[HP == 2 ? E : 1];   // head pairs: P.V of the second head's V
  float up[(G > 4 && G <= 8) ? 4 : 1][E];   // G = 8: heads 4..7 brought up by merge_rows

  // q rows of the unit whose first head is h0 (= KV head * group): lane column n (col_base +
  // lane % 16; col_base = 16 for the second half of a 32-column pair) reads query token
  // n / group, head h0 + n % group.  Columns past q_len * group are padding (zero q).
  __device__ __forceinline__ void load_q(const DecodeParams& p, const QShape& qs, int b, int h0,
                                         int lane, uint32_t qflip, int col_base = 0) {
    const int n = col_base + (lane & 15);
    const int sh = __builtin_ctz((unsigned)qs.group);   // group is a power of two
    col_q = n >> sh;
    head_lane = col_q < qs.q_len;
    const int hh = n & (qs.group - 1);
    const char* qrow = reinterpret_cast<const char*>(
        p.q + (((size_t)b * qs.q_total + qs.q_first + (head_lane ? col_q : 0)) * p.num_q_heads +
               h0 + (head_lane ? hh : 0)) * D);
    half1 = HP == 2 && n >= G / 2;
    const uint32_t keep = head_lane ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      // score MFMA kk, lane group g: dims 32kk + 8g .. +8 (bf16), or, matching the FP8 K
      // pieces, 64(kk/2) + 16g + 8(kk%2) .. +8 (a permutation of the dot product's terms)
      const int off = FP8 ? 128 * (kk >> 1) + 32 * (lane >> 4) + 16 * (kk & 1)
                          : 64 * kk + 16 * (lane >> 4);
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(qrow + off);
      x.x = (x.x ^ qflip) & keep;
      x.y = (x.y ^ qflip) & keep;
      x.z = (x.z ^ qflip) & keep;
      x.w = (x.w ^ qflip) & keep;
      qb[kk] = x;
    }
  }
  __device__ __forceinline__ void reset() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) cacc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (HP == 2) {
#pragma unroll
      for (int e = 0; e < E; ++e) cacc1[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
  int rs;   // bytes between a block's consecutive K/V rows (the pool layout's row stride)
  __device__ __forceinline__ void init(const DecodeParams& p, const QShape& qs, int b, int h0,
                                       int lane, uint32_t qflip, float c2_, int col_base = 0) {
    c2 = c2_;
    rs = (int)p.kv_row_stride;
    vs = p.v_scale;
    pair_off = p.kv_pair_off;
    load_q(p, qs, b, h0, lane, qflip, col_base);
    reset();
  }

  __device__ __forceinline__ void issue(Tile& t, const char* kb, const char* vb, int lane) const {
    issue_head(t.x[0], kb, vb, lane);
    if constexpr (HP == 2) issue_head(t.x[1], kb + pair_off, vb + pair_off, lane);
  }
  __device__ __forceinline__ void issue_head(TileHead& t, const char* kb, const char* vb,
                                             int lane) const {
    const int mrow = lane & 15;
    const int tok = 4 * (mrow & 3) + (mrow >> 2);
    if constexpr (FP8) {
      // K: bytes 64i + 16(lane/16) .. +16 of the token's row, i < KK/2 (16-byte pieces: 8-byte
      // ones, one per score MFMA, halve the streaming rate); its halves feed MFMAs 2i, 2i+1.
      // V: the lane's slice of each of its four rows, E bytes (two 8-byte pieces at D = 256)
      const char* krow = kb + tok * rs + 16 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < KL; ++i)
        t.k[i] = kv_load<NT>(reinterpret_cast<const u32x4_t*>(krow + 64 * i));
      const int r = lane >> 4, c = lane & 15;
#pragma unroll
      for (int j = 0; j < kTileSteps; ++j) {
        const char* row = vb + (kRows * j + r) * rs;
        if constexpr (D == 64) {
          t.v[j][0] = kv_load<NT>(reinterpret_cast<const uint32_t*>(row + 4 * c));
        } else {
          const u32x2_t x =
              kv_load<NT>(reinterpret_cast<const u32x2_t*>(row + 8 * c));
          t.v[j][0] = x.x;
          t.v[j][1] = x.y;
          if constexpr (D == 256) {
            const u32x2_t y =
                kv_load<NT>(reinterpret_cast<const u32x2_t*>(row + 128 + 8 * c));
            t.v[j][2] = y.x;
            t.v[j][3] = y.y;
          }
        }
      }
    } else {
      const char* krow = kb + tok * rs + 16 * (lane >> 4);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        t.k[kk] = kv_load<NT>(reinterpret_cast<const u32x4_t*>(krow + 64 * kk));
      load_v_rows<D, NT>(t.v, vb, lane, rs);
    }
  }

  // A tile copied to LDS: K rows then V rows, kRowBytes each; within a row the 16-byte piece p
  // sits at piece p ^ (row & kLdsSwizzle), which spreads a column of pieces over the rows'
  // banks.  Byte `off` of row `row` of half h (0 = K, 1 = V):
  static constexpr int kLdsSwizzle = kRowBytes / 16 < 16 ? kRowBytes / 16 - 1 : 15;
  __device__ __forceinline__ static const char* lds_at(const char* tile, int h, int row,
                                                       int off) {
    return tile + (h * kTileTokens + row) * kRowBytes +
           ((((off >> 4) ^ (row & kLdsSwizzle))) << 4) + (off & 15);
  }
  // Fill t from such a copy: the same pieces issue() reads from the pool.
  // A head pair's copy holds the second head's tile (K rows, then V rows) after the first's.
  static constexpr int kHeadTileBytes = 2 * kTileTokens * kRowBytes;
  __device__ __forceinline__ void fill_from_lds(Tile& tt, const char* tile, int lane) const {
    fill_head_from_lds(tt.x[0], tile, lane);
    if constexpr (HP == 2) fill_head_from_lds(tt.x[1], tile + kHeadTileBytes, lane);
  }
  __device__ __forceinline__ void fill_head_from_lds(TileHead& t, const char* tile,
                                                     int lane) const {
    const int mrow = lane & 15;
    const int tok = 4 * (mrow & 3) + (mrow >> 2);
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int i = 0; i < KL; ++i)
      t.k[i] = *reinterpret_cast<const u32x4_t*>(lds_at(tile, 0, tok, 64 * i + 16 * g));
#pragma unroll
    for (int j = 0; j < kTileSteps; ++j) {
      const int row = kRows * j + g;
      if constexpr (FP8) {
        if constexpr (D == 64) {
          t.v[j][0] = *reinterpret_cast<const uint32_t*>(lds_at(tile, 1, row, 4 * c));
        } else {
          const u32x2_t x = *reinterpret_cast<const u32x2_t*>(lds_at(tile, 1, row, 8 * c));
          t.v[j][0] = x.x;
          t.v[j][1] = x.y;
          if constexpr (D == 256) {
            const u32x2_t y =
                *reinterpret_cast<const u32x2_t*>(lds_at(tile, 1, row, 128 + 8 * c));
            t.v[j][2] = y.x;
            t.v[j][3] = y.y;
          }
        }
      } else if constexpr (D == 64) {
        const u32x2_t x = *reinterpret_cast<const u32x2_t*>(lds_at(tile, 1, row, 8 * c));
        t.v[j][0] = x.x;
        t.v[j][1] = x.y;
      } else {
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(lds_at(tile, 1, row, 16 * c));
        t.v[j][0] = x.x; t.v[j][1] = x.y; t.v[j][2] = x.z; t.v[j][3] = x.w;
        if constexpr (D == 256) {
          const u32x4_t y = *reinterpret_cast<const u32x4_t*>(lds_at(tile, 1, row, 256 + 16 * c));
          t.v[j][4] = y.x; t.v[j][5] = y.y; t.v[j][6] = y.z; t.v[j][7] = y.w;
        }
      }
    }
  }

  template <bool MASKED>
  __device__ __forceinline__ void consume(Tile& t, int tok0, int lo, int hi, int lane) {
    consume<MASKED>(t, tok0, lo, hi, lo, hi, lane);
  }
  // Masked tile with query tokens: this lane's column sees keys [max(hi - window, 0), hi) with
  // hi = hi_base + its query token (hi_base: the first token's position + 1).
  __device__ __forceinline__ void consume_cols(Tile& t, int tok0, int hi_base, int window,
                                               int vlo, int vhi, int lane) {
    const int hi = hi_base + col_q;
    const int lo = window > 0 ? max(hi - window, 0) : 0;
    consume<true>(t, tok0, lo, hi, vlo, vhi, lane);
  }
  // Masked form: scores of column (lane) keys outside [lo, hi) drop out (lo, hi may differ by
  // lane: the column's query token); V rows outside [vlo, vhi), the union, are zeroed so that a
  // stray NaN there cannot meet a zero probability.
  template <bool MASKED>
  __device__ __forceinline__ void consume(Tile& t, int tok0, int lo, int hi, int vlo, int vhi,
                                          int lane) {
    consume_impl<MASKED ? 1 : 0>(t, false, tok0, lo, hi, vlo, vhi, lane);
  }
  // One code path for every tile of a loop, masked unless `full` (wave-uniform: every key of
  // the tile attended by every column).  Separate masked and unmasked paths through the
  // matrix instructions leave the compiler two versions of the accumulators to merge after
  // them, which it does by copying all of them, twice per tile; here only the masking step is
  // conditional.
  __device__ __forceinline__ void consume_flex(Tile& t, bool full, int tok0, int lo, int hi,
                                               int vlo, int vhi, int lane) {
    consume_impl<2>(t, full, tok0, lo, hi, vlo, vhi, lane);
  }
  // consume_flex with the column's own key range (as consume_cols)
  __device__ __forceinline__ void consume_cols_flex(Tile& t, bool full, int tok0, int hi_base,
                                                    int window, int vlo, int vhi, int lane) {
    const int hi = hi_base + col_q;
    const int lo = window > 0 ? max(hi - window, 0) : 0;
    consume_impl<2>(t, full, tok0, lo, hi, vlo, vhi, lane);
  }
  // MODE 0: every key attended (the score scale folded into the exponent); 1: masked; 2:
  // masked unless `full`.
  template <int MODE>
  __device__ __forceinline__ void consume_impl(Tile& t, bool full, int tok0, int lo, int hi,
                                               int vlo, int vhi, int lane) {
    constexpr bool MASKED = MODE != 0;
    const int g = lane >> 4;
    f32x4_t sc = scores(t.x[0]);
    if constexpr (HP == 2) {
      const f32x4_t sc1 = scores(t.x[1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = half1 ? sc1[i] : sc[i];
    }
    if constexpr (MODE == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tk = tok0 + 4 * i + g;
        sc[i] = (tk >= lo && tk < hi) ? sc[i] * c2 : -INFINITY;
      }
#pragma unroll
      for (int hp = 0; hp < HP; ++hp) mask_v_words<VW>(t.x[hp].v, tok0, vlo, vhi, lane);
    } else if constexpr (MODE == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] *= c2;
      if (!full) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tk = tok0 + 4 * i + g;
          sc[i] = (tk >= lo && tk < hi) ? sc[i] : -INFINITY;
        }
#pragma unroll
        for (int hp = 0; hp < HP; ++hp) mask_v_words<VW>(t.x[hp].v, tok0, vlo, vhi, lane);
      }
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if constexpr (!MASKED) mx *= c2;
    const bool need = head_lane && mx > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      // one running max per head for the whole wave: raise it to the wave's tile max
      const float mn = fmaxf(m, rows_max(mx));
      const float alpha = fast_exp2(m - (mn == -INFINITY ? 0.f : mn));
      l *= alpha;
      m = mn;
      // C row 4g+i is head 4g+i, whose factor sits in lane 4g+i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a_i = __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute((4 * g + i) << 2, __builtin_bit_cast(int, alpha)));
#pragma unroll
        for (int e = 0; e < E; ++e) cacc[e][i] *= a_i;
        if constexpr (HP == 2) {
#pragma unroll
          for (int e = 0; e < E; ++e) cacc1[e][i] *= a_i;
        }
      }
    }
    const float mu = m == -INFINITY ? 0.f : m;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = MASKED ? fast_exp2(sc[i] - mu) : fast_exp2(fmaf(sc[i], c2, -mu));
      pr[i] = head_lane ? pr[i] : 0.f;
    }
    l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    // p = hi + lo in bf16
    const bf16x2_t h01 = {(__bf16)pr[0], (__bf16)pr[1]};
    const bf16x2_t h23 = {(__bf16)pr[2], (__bf16)pr[3]};
    const uint32_t uh01 = __builtin_bit_cast(uint32_t, h01);
    const uint32_t uh23 = __builtin_bit_cast(uint32_t, h23);
    const bf16x2_t l01 = {(__bf16)(pr[0] - __builtin_bit_cast(float, uh01 << 16)),
                          (__bf16)(pr[1] - __builtin_bit_cast(float, uh01 & 0xFFFF0000u))};
    const bf16x2_t l23 = {(__bf16)(pr[2] - __builtin_bit_cast(float, uh23 << 16)),
                          (__bf16)(pr[3] - __builtin_bit_cast(float, uh23 & 0xFFFF0000u))};
    const s16x4_t a_hi = __builtin_bit_cast(s16x4_t, u32x2_t{uh01, uh23});
    const s16x4_t a_lo = __builtin_bit_cast(
        s16x4_t, u32x2_t{__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)});
    pv_head(t.x[0], a_hi, a_lo, cacc);
    if constexpr (HP == 2) pv_head(t.x[1], a_hi, a_lo, cacc1);
  }

  // q.k of one head's tile: the scores of this lane's column for the four tokens of its row
  // group (unscaled)
  __device__ __forceinline__ f32x4_t scores(const TileHead& th) const {
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4_t kw;
      if constexpr (FP8) {
        const u32x4_t x = th.k[kk >> 1];
        kw = fp8x8_to_bf16x8((kk & 1) ? u32x2_t{x.z, x.w} : u32x2_t{x.x, x.y});
      } else {
        kw = th.k[kk];
      }
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kw),
                                                   __builtin_bit_cast(bf16x8_t, qb[kk]), sc, 0,
                                                   0, 0);
    }
    return sc;
  }

  // P.V of one head's tile into acc: P as the two bf16 terms a_hi + a_lo
  __device__ __forceinline__ static void pv_head(const TileHead& th, s16x4_t a_hi, s16x4_t a_lo,
                                                 f32x4_t (&acc)[E]) {
    // B: element e of the slice of tokens 4j+g, j = 0..3, as bf16 pairs {token 4j+g of rows
    // j = 0, 1} and {j = 2, 3}
    const auto pv = [&](int e, uint32_t b01, uint32_t b23) {
      const s16x4_t bv = __builtin_bit_cast(s16x4_t, u32x2_t{b01, b23});
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_hi, bv, acc[e], 0, 0, 0);
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_lo, bv, acc[e], 0, 0, 0);
    };
    const auto& v = th.v;
    if constexpr (FP8) {
      // word w holds elements 4w..4w+3 of a row: interleave the bytes of rows (0, 1) and (2, 3)
      // (x: elements 4w, 4w+1; y: 4w+2, 4w+3), then each half converts to one bf16 pair
#pragma unroll
      for (int w = 0; w < VW; ++w) {
        const uint32_t x01 = __builtin_amdgcn_perm(v[1][w], v[0][w], 0x05010400u);
        const uint32_t y01 = __builtin_amdgcn_perm(v[1][w], v[0][w], 0x07030602u);
        const uint32_t x23 = __builtin_amdgcn_perm(v[3][w], v[2][w], 0x05010400u);
        const uint32_t y23 = __builtin_amdgcn_perm(v[3][w], v[2][w], 0x07030602u);
        pv(4 * w + 0, fp8x2_to_bf16x2<false>(x01), fp8x2_to_bf16x2<false>(x23));
        pv(4 * w + 1, fp8x2_to_bf16x2<true>(x01), fp8x2_to_bf16x2<true>(x23));
        pv(4 * w + 2, fp8x2_to_bf16x2<false>(y01), fp8x2_to_bf16x2<false>(y23));
        pv(4 * w + 3, fp8x2_to_bf16x2<true>(y01), fp8x2_to_bf16x2<true>(y23));
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        // bf16 halves gathered by v_perm
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        pv(e, __builtin_amdgcn_perm(v[1][e / 2], v[0][e / 2], sel),
           __builtin_amdgcn_perm(v[3][e / 2], v[2][e / 2], sel));
      }
    }
  }

  // Sum the row groups' partial sums: every lane ends with the wave's (M, l) of every head.
  // With G = 8, heads 4..7 live in row 1 and are brought up here, where every lane is active
  // (a lane permute reads nothing from inactive lanes).
  __device__ __forceinline__ void merge_rows(float (&Mh)[G], float (&lh)[G]) {
    const float lt = rows_sum(l);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      Mh[h] = row_bcast_dyn(m, h);
      lh[h] = row_bcast_dyn(lt, h);
    }
    if constexpr (G > 4 && G <= 8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < E; ++e)
          up[i][e] = xor_lane<16>(HP == 2 ? cacc1[e][i] : cacc[e][i]);
      }
    }
  }
  // After merge_rows, on the row-0 lanes: the accumulated P.V of head h at dim(lane, e)
  // (times the V scale for an FP8 cache).
  __device__ __forceinline__ float out(int h, int e) const {
    static_assert(G <= 8, "out() covers eight columns");
    // head pairs: heads h < G / 2 are the first KV head's, in cacc; the rest the second's (in
    // cacc1, or for G = 8 brought up from row group 1 by merge_rows)
    const float x = HP == 2 && G <= 4 ? (h < G / 2 ? cacc[e][h & 3] : cacc1[e][h & 3])
                    : h < 4           ? cacc[e][h & 3]
                                      : up[(h - 4) & 3][e];
    return FP8 ? x * vs : x;
  }

  // Column-wise finish, for any G: after merge_cols every lane can read column n's running max
  // and sum (col_m / col_l, read from lane n; call them on every lane), and lane (r, c) holds
  // the accumulated P.V of column 4r + i at dim(c, e) as acc(i, e).
  __device__ __forceinline__ void merge_cols() { lsum = rows_sum(l); }
  __device__ __forceinline__ float col_m(int n) const {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_ds_bpermute(n << 2, __builtin_bit_cast(int, m)));
  }
  __device__ __forceinline__ float col_l(int n) const {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_ds_bpermute(n << 2, __builtin_bit_cast(int, lsum)));
  }
  __device__ __forceinline__ float acc(int i, int e) const {
    return FP8 ? cacc[e][i] * vs : cacc[e][i];
  }
};

template <int D, int G>
using QkMfmaPv = QkMfmaPvT<D, G, false>;
template <int D, int G>
using QkMfmaPvFp8 = QkMfmaPvT<D, G, true>;

// Thirty-two columns (query tokens x heads) as two 16-column halves that share every K/V tile:
// the tile is loaded once and each half runs its own q.k, softmax and P.V on it.  Finished
// column-wise, half by half (col_base 0 and 16).
template <int D, bool FP8, bool NT = true>
struct QkMfmaPvPair {
  using Half = QkMfmaPvT<D, 16, FP8, NT>;
  using Tile = typename Half::Tile;
  static constexpr int kRowBytes = Half::kRowBytes;
  static constexpr int kMinWavesPerEu = 1;
  static constexpr bool kColumns = true;
  static constexpr bool kQueryTokens = true;
  static constexpr int kHalves = 2;
  static constexpr int kHeads = 1;
  Half h[2];

  __device__ __forceinline__ void init(const DecodeParams& p, const QShape& qs, int b, int h0,
                                       int lane, uint32_t qflip, float c2) {
    h[0].init(p, qs, b, h0, lane, qflip, c2, 0);
    h[1].init(p, qs, b, h0, lane, qflip, c2, 16);
  }
  __device__ __forceinline__ void load_q(const DecodeParams& p, const QShape& qs, int b, int h0,
                                         int lane, uint32_t qflip) {
    h[0].load_q(p, qs, b, h0, lane, qflip, 0);
    h[1].load_q(p, qs, b, h0, lane, qflip, 16);
  }
  __device__ __forceinline__ void reset() {
    h[0].reset();
    h[1].reset();
  }
  __device__ __forceinline__ void issue(Tile& t, const char* kb, const char* vb,
                                        int lane) const {
    h[0].issue(t, kb, vb, lane);
  }
  static constexpr int kLdsSwizzle = Half::kLdsSwizzle;
  __device__ __forceinline__ void fill_from_lds(Tile& t, const char* tile, int lane) const {
    h[0].fill_from_lds(t, tile, lane);
  }
  template <bool MASKED>
  __device__ __forceinline__ void consume(Tile& t, int tok0, int lo, int hi, int lane) {
    h[0].template consume<MASKED>(t, tok0, lo, hi, lane);
    h[1].template consume<MASKED>(t, tok0, lo, hi, lane);
  }
  __device__ __forceinline__ void consume_cols(Tile& t, int tok0, int hi_base, int window,
                                               int vlo, int vhi, int lane) {
    h[0].consume_cols(t, tok0, hi_base, window, vlo, vhi, lane);
    h[1].consume_cols(t, tok0, hi_base, window, vlo, vhi, lane);
  }
  __device__ __forceinline__ void consume_cols_flex(Tile& t, bool full, int tok0, int hi_base,
                                                    int window, int vlo, int vhi, int lane) {
    h[0].consume_cols_flex(t, full, tok0, hi_base, window, vlo, vhi, lane);
    h[1].consume_cols_flex(t, full, tok0, hi_base, window, vlo, vhi, lane);
  }
};

// The policy of a path (32 columns: the matrix-core P.V pair).
template <int D, int G, QkPath PATH>
using QkPolicy = typename std::conditional<
    G == 32, QkMfmaPvPair<D, PATH == QkPath::kMfmaPvFp8>,
    typename std::conditional<
        PATH == QkPath::kValu, QkValu<D, G>,
        typename std::conditional<
            PATH == QkPath::kMfma, QkMfma<D, G>,
            typename std::conditional<
                PATH == QkPath::kMfmaPv, QkMfmaPv<D, G>,
                typename std::conditional<
                    PATH == QkPath::kMfmaPvHeads2, QkMfmaPvT<D, G, false, true, 2>,
                    typename std::conditional<PATH == QkPath::kMfmaPvFp8Heads2,
                                              QkMfmaPvT<D, G, true, true, 2>,
                                              QkMfmaPvFp8<D, G>>::type>::type>::type>::type>::
        type>::type;

}  // namespace pa
