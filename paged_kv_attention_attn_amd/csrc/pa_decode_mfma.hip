// Single-token paged-attention decode for gfx950 with QK^T on the matrix cores.
//
// Same work decomposition, softmax and epilogue as the VALU kernel (one workgroup per
// (partition, KV head, sequence); 16-token tiles; per-row-group online softmax merged with the
// log-sum-exp rule).  What changes is the score computation: for a tile, the G query heads that
// share the KV head form a dense [16 tokens x D] . [D x G] contraction, done as D/32
// v_mfma_f32_16x16x32_bf16 (bf16 products, fp32 accumulation; heads padded to 16 columns).
// P.V stays on the vector ALUs in fp32: the probabilities never round to bf16.
//
// Lane layouts (verified on gfx950): for the 16x16x32 bf16 MFMA, lane l holds A[l%16][8(l/16)+i],
// B[8(l/16)+i][l%16] and C[4(l/16)+i][l%16].  MFMA row m of a tile is token 4(m%4) + m/4, so the
// four scores a lane gets back (C rows 4g+i, g = l/16) are tokens 4i+g: the same tokens that
// lane's DPP row handles in the P.V layout (row group r = l/16 holds rows 4j+r).  The k order
// inside the contraction is a free choice (A and B use the same one): chunk 4kk + l/16 of the
// head dim for MFMA kk, so each lane reads contiguous 16-byte pieces of K rows and q.
//
// Probabilities reach the P.V layout with DPP row_newbcast (lane h of each 16-lane row to the
// whole row): lane (h, row r) holds p of head h for tokens 4j + r.
//
// Sources: the decode step, GQA grouping and online softmax as in the VALU kernel
// (ROCm/rocm-libraries PR #13700 "prepare saved paged decode bindings once", Summary; vllm.cpp
// PR #564 "spec(BACKEND-ROCM): the ROCm head_dim=128 decode arm", "It is a mirror of merged
// work, not new design" and "What is deliberately not here"); a matrix-core arm for a wide
// grouped-query tile: the same page, "One deviation from the original commit" (the separate
// WMMA d=128 arm).
#include <cstdio>

#include "pa_device.hpp"
#include "pa_kernels.hpp"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kSlack = 8.0f;   // lazy-rescale threshold, log2 units (see the VALU kernel)

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// value of x in lane h of this lane's 16-lane row
template <int H>
__device__ __forceinline__ float row_bcast(float x) {
  return dpp_mov<0x150 + H>(x);
}

template <int D>
struct MTile {
  static constexpr int KK = D / 32;          // MFMAs per tile
  static constexpr int W = RowGeom<D>::kWords;
  u32x4_t k[KK];                             // MFMA A operands (K rows, permuted)
  uint32_t v[kTileSteps][W];                 // V rows 4j + r, lane slice c
};

template <int D>
__device__ __forceinline__ void issue_mtile(MTile<D>& t, const char* kb, const char* vb, int lane) {
  constexpr int RB = RowGeom<D>::kRowBytes;
  const int m = lane & 15;
  const int tok = 4 * (m & 3) + (m >> 2);
  const char* krow = kb + tok * RB + 16 * (lane >> 4);
#pragma unroll
  for (int kk = 0; kk < MTile<D>::KK; ++kk)
    t.k[kk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(krow + 64 * kk));
  const int r = lane >> 4, c = lane & 15;
#pragma unroll
  for (int j = 0; j < kTileSteps; ++j) load_row<D>(vb + (kRows * j + r) * RB, c, t.v[j]);
}

template <int D, int G>
struct MState {
  static constexpr int E = RowGeom<D>::kElems;
  float m;          // running max, head l%16, row group l/16 (log2 units)
  float l;          // running sum of 2^(s - m)
  float acc[G][E];  // P.V layout: row group l/16, head-dim slice l%16
};

template <int D, int G, bool MASKED>
__device__ __forceinline__ void consume_mtile(MState<D, G>& st, MTile<D>& t,
                                              const u32x4_t (&qb)[D / 32], float c2, int tok0,
                                              int lo, int hi, int lane) {
  constexpr int W = RowGeom<D>::kWords;
  constexpr int E = RowGeom<D>::kElems;
  const int g = lane >> 4;
  const bool head_lane = (lane & 15) < G;

  f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, t.k[kk]),
                                                 __builtin_bit_cast(bf16x8_t, qb[kk]), sc, 0, 0,
                                                 0);
  if constexpr (MASKED) {
    // tokens outside [lo, hi): score -inf and a zero value row, by select
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tk = tok0 + 4 * i + g;
      sc[i] = (tk >= lo && tk < hi) ? sc[i] * c2 : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < kTileSteps; ++j) {
      const int tk = tok0 + kRows * j + g;
      const bool ok = tk >= lo && tk < hi;
#pragma unroll
      for (int w = 0; w < W; ++w) t.v[j][w] = ok ? t.v[j][w] : 0u;
    }
  }
  float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  if constexpr (!MASKED) mx *= c2;
  const bool need = head_lane && mx > st.m + kSlack;
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
    const float mn = fmaxf(st.m, mx);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float alpha = fast_exp2(st.m - mu);
    st.l *= alpha;
    st.m = mn;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a_h;
      switch (h) {   // compile-time h after unrolling
        case 0: a_h = row_bcast<0>(alpha); break;
        case 1: a_h = row_bcast<1>(alpha); break;
        case 2: a_h = row_bcast<2>(alpha); break;
        case 3: a_h = row_bcast<3>(alpha); break;
        case 4: a_h = row_bcast<4>(alpha); break;
        case 5: a_h = row_bcast<5>(alpha); break;
        case 6: a_h = row_bcast<6>(alpha); break;
        default: a_h = row_bcast<7>(alpha); break;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) st.acc[h][e] *= a_h;
    }
  }
  const float mu = st.m == -INFINITY ? 0.f : st.m;
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    p[i] = MASKED ? fast_exp2(sc[i] - mu) : fast_exp2(fmaf(sc[i], c2, -mu));
  st.l += (p[0] + p[1]) + (p[2] + p[3]);

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
      float pb;
      switch (h) {
        case 0: pb = row_bcast<0>(p[j]); break;
        case 1: pb = row_bcast<1>(p[j]); break;
        case 2: pb = row_bcast<2>(p[j]); break;
        case 3: pb = row_bcast<3>(p[j]); break;
        case 4: pb = row_bcast<4>(p[j]); break;
        case 5: pb = row_bcast<5>(p[j]); break;
        case 6: pb = row_bcast<6>(p[j]); break;
        default: pb = row_bcast<7>(p[j]); break;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) st.acc[h][e] = fmaf(pb, vf[e], st.acc[h][e]);
    }
  }
}

template <int D, int G, int NW, int DEPTH>
__global__ __launch_bounds__(NW * kWave) void decode_mfma_kernel(const DecodeParams p) {
  static_assert(G >= 1 && G <= 8, "heads per KV head");
  using RG = RowGeom<D>;
  constexpr int E = RG::kElems;
  constexpr int KK = D / 32;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane >> 4;
  const int c = lane & (kRowLanes - 1);
  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int h0 = kvh * G;

  // q as the MFMA B operand: lane l holds head l%16 (zero past G), chunk 4kk + l/16 of the head
  // dim for MFMA kk.  Loaded before the sequence length is known; a negative scale is applied
  // as |scale| on -q (sign flip, exact).
  float c2 = p.qk_scale_log2;
  const uint32_t qflip = c2 < 0.f ? 0x80008000u : 0u;
  c2 = fabsf(c2);
  u32x4_t qb[KK];
  {
    const int n = lane & 15;
    const char* qrow = reinterpret_cast<const char*>(
        p.q + ((size_t)b * p.num_q_heads + h0 + (n < G ? n : 0)) * D);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(qrow + 64 * kk + 16 * (lane >> 4));
      const uint32_t keep = n < G ? 0xFFFFFFFFu : 0u;
      x.x = (x.x ^ qflip) & keep;
      x.y = (x.y ^ qflip) & keep;
      x.z = (x.z ^ qflip) & keep;
      x.w = (x.w ^ qflip) & keep;
      qb[kk] = x;
    }
  }

  const int L = p.seq_lens[b];
  const bool split = p.psize > 0;
  const int n_parts = split ? (L > 0 ? (int)(((int64_t)L + p.psize - 1) / p.psize) : 1) : 1;
  if (part >= n_parts) return;
  bool bad = L < 0 || (int64_t)L > ((int64_t)p.stride << p.bs_log2);
  if (split && part == p.max_parts - 1 && n_parts > p.max_parts) bad = true;
  const PartRange pr = part_range(bad ? 0 : L, p.window, part, p.psize);

  MState<D, G> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < E; ++e) st.acc[h][e] = 0.f;
  }

  // full tiles [f0, f1) round-robin over the waves; table entries preloaded 64 at a time
  const TileAddr ta{p.num_blocks, p.num_kv_heads, kvh, p.bs_log2, RG::kRowBytes};
  const int32_t* bt_row = p.block_table + (size_t)b * p.stride;
  const int f0 = (pr.lo + kTileTokens - 1) / kTileTokens;
  const int f1 = pr.hi / kTileTokens;
  const int first = f0 + wave;
  const int n_w = first < f1 ? (f1 - first + NW - 1) / NW : 0;
  int phys_v = 0;
  int chunk = -1;
  bool bad_table = false;

  auto phys_of = [&](int i) -> int {
    const int ch = i >> 6;
    if (ch != chunk) {
      chunk = ch;
      const int li = (ch << 6) + lane;
      phys_v = li < n_w ? bt_row[ta.logical_block(first + NW * li)] : 0;
    }
    return __builtin_amdgcn_readlane(phys_v, i & 63);
  };
  auto issue = [&](int i, MTile<D>& regs) -> bool {
    const int64_t off = ta.offset(phys_of(i), first + NW * i);
    if (off < 0) {
      bad_table = true;
      return false;
    }
    issue_mtile<D>(regs, p.k_cache + off, p.v_cache + off, lane);
    return true;
  };

  if constexpr (DEPTH == 2) {
    MTile<D> ra, rb;
    bool oka = n_w > 0 ? issue(0, ra) : false;
    bool okb = false;
    for (int i = 0; i < n_w; i += 2) {
      if (i + 1 < n_w) okb = issue(i + 1, rb);
      if (oka) consume_mtile<D, G, false>(st, ra, qb, c2, 0, 0, 0, lane);
      if (i + 2 < n_w) oka = issue(i + 2, ra);
      if (i + 1 < n_w && okb) consume_mtile<D, G, false>(st, rb, qb, c2, 0, 0, 0, lane);
    }
  } else {
    MTile<D> ra;
    for (int i = 0; i < n_w; ++i)
      if (issue(i, ra)) consume_mtile<D, G, false>(st, ra, qb, c2, 0, 0, 0, lane);
  }

  // partial tiles at the ends of [lo, hi), on the last wave
  if (wave == NW - 1 && pr.hi > pr.lo) {
    const int head = pr.lo / kTileTokens;
    const int tail = pr.hi / kTileTokens;
    const bool has_head = head < f0;
    const bool has_tail = (pr.hi % kTileTokens) != 0 && !(has_head && tail == head);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const bool on = k == 0 ? has_head : has_tail;
      if (!on) continue;
      const int tile = k == 0 ? head : tail;
      const int64_t off =
          ta.offset(__builtin_amdgcn_readfirstlane(bt_row[ta.logical_block(tile)]), tile);
      if (off < 0) {
        bad_table = true;
        continue;
      }
      MTile<D> rt;
      issue_mtile<D>(rt, p.k_cache + off, p.v_cache + off, lane);
      consume_mtile<D, G, true>(st, rt, qb, c2, tile * kTileTokens, pr.lo, pr.hi, lane);
    }
  }

  // Row-group merge.  (m, l) of head h, row r sit in lane h + 16r; acc[h][.] of row r sits in
  // row r.  M_h = max over rows; each row's share is scaled by 2^(m_r - M_h) and summed.
  const float M = rows_max(st.m);
  const float Mu = M == -INFINITY ? 0.f : M;
  const float f = fast_exp2(st.m - Mu);
  const float lt = rows_sum(st.l * f);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float f_h;
    switch (h) {
      case 0: f_h = row_bcast<0>(f); break;
      case 1: f_h = row_bcast<1>(f); break;
      case 2: f_h = row_bcast<2>(f); break;
      case 3: f_h = row_bcast<3>(f); break;
      case 4: f_h = row_bcast<4>(f); break;
      case 5: f_h = row_bcast<5>(f); break;
      case 6: f_h = row_bcast<6>(f); break;
      default: f_h = row_bcast<7>(f); break;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) st.acc[h][e] = rows_sum(st.acc[h][e] * f_h);
  }

  // wave merge through LDS
  __shared__ float s_acc[NW][G][D];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];
  __shared__ int s_bad[NW];
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < E; ++e) s_acc[wave][h][RG::dim(c, e)] = st.acc[h][e];
    }
    if (c < G) {
      s_m[wave][c] = M;
      s_l[wave][c] = lt;
    }
    if (c == 0) s_bad[wave] = bad_table ? 1 : 0;
  }
  __syncthreads();

  bool any_bad = bad;
#pragma unroll
  for (int w = 0; w < NW; ++w) any_bad |= s_bad[w] != 0;

  const bool fold_sink = p.sinks != nullptr && part == pr.first_part;
  for (int i = threadIdx.x; i < G * D; i += NW * kWave) {
    const int h = i / D;
    const int d = i - h * D;
    float Mw = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) Mw = fmaxf(Mw, s_m[w][h]);
    const float Mwu = Mw == -INFINITY ? 0.f : Mw;
    float lw = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float fw = fast_exp2(s_m[w][h] - Mwu);
      lw = fmaf(s_l[w][h], fw, lw);
      o = fmaf(s_acc[w][h][d], fw, o);
    }
    const int hq = h0 + h;
    if (fold_sink) {
      const float s2 = p.sinks[hq] * kLog2e;
      const float M2 = fmaxf(Mw, s2);
      const float M2u = M2 == -INFINITY ? 0.f : M2;
      const float fs = fast_exp2(Mw - M2u);
      lw = fmaf(lw, fs, fast_exp2(s2 - M2u));
      o *= fs;
      Mw = M2;
    }
    float ov = lw > 0.f ? o / lw : 0.f;
    float lv = lw > 0.f ? (Mw + fast_log2(lw)) * kLn2 : -INFINITY;
    if (any_bad) {
      ov = __builtin_nanf("");
      lv = __builtin_nanf("");
    }
    const size_t row = (size_t)b * p.num_q_heads + hq;
    if (split) {
      p.out[(row * p.max_parts + part) * D + d] = ov;
      if (d == 0) p.lse[row * p.max_parts + part] = lv;
    } else {
      p.out[row * D + d] = ov;
      if (d == 0 && p.lse != nullptr) p.lse[row] = lv;
    }
  }
}

namespace {

template <int D, int G>
constexpr int mfma_depth() {
  return (D * G <= 512) ? 2 : 1;
}

template <int D, int G, int NW>
hipError_t launch_m(const DecodeParams& p, int num_seqs, hipStream_t stream) {
  const dim3 grid(p.psize > 0 ? p.max_parts : 1, p.num_kv_heads, num_seqs);
  hipLaunchKernelGGL((decode_mfma_kernel<D, G, NW, mfma_depth<D, G>()>), grid, dim3(NW * kWave),
                     0, stream, p);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_mg(const DecodeParams& p, int waves, int num_seqs, hipStream_t stream) {
  switch (waves) {
    case 1: return launch_m<D, G, 1>(p, num_seqs, stream);
    case 2: return launch_m<D, G, 2>(p, num_seqs, stream);
    case 4: return launch_m<D, G, 4>(p, num_seqs, stream);
    case 8: return launch_m<D, G, 8>(p, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_md(const DecodeParams& p, int group, int waves, int num_seqs,
                     hipStream_t stream) {
  switch (group) {
    case 1: return launch_mg<D, 1>(p, waves, num_seqs, stream);
    case 2: return launch_mg<D, 2>(p, waves, num_seqs, stream);
    case 4: return launch_mg<D, 4>(p, waves, num_seqs, stream);
    case 8: return launch_mg<D, 8>(p, waves, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, int group, int waves,
                              int num_seqs, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_md<64>(p, group, waves, num_seqs, stream);
    case 128: return launch_md<128>(p, group, waves, num_seqs, stream);
    case 256: return launch_md<256>(p, group, waves, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
