// Single-token paged-attention decode for gfx950 (CDNA4), unsplit and split-KV.
//
// One workgroup per (partition, KV head, sequence).  It walks the sequence's block table tile by
// tile (16 tokens), loads each tile's K and V rows once with 16-byte coalesced loads (8 B at
// head_dim 64), and serves all G query heads that share the KV head from the same registers, so
// every K/V byte is read once per KV head.  QK^T uses bf16 dot2 with fp32 accumulation and a
// DPP reduction across the 16 lanes that hold one row; softmax is online (running max and sum);
// P.V accumulates in fp32.  Each of the 4 row groups of a wave runs its own online softmax over
// tokens 4j + r of every tile (a strided subset); the row groups, then the waves, are merged
// with the log-sum-exp rule at the end.  The epilogue folds the sink logit, normalises, and
// writes the final output and LSE (unsplit) or the partition's partial output and LSE (split).
//
// Sources: one-token split-KV decode with partial outputs + LSE and a reduce step,
// ROCm/rocm-libraries PR #13700 "prepare saved paged decode bindings once", Summary; online
// softmax reaching the same function in another order, vllm.cpp PR #564 "spec(BACKEND-ROCM): the
// ROCm head_dim=128 decode arm", "It is a mirror of merged work, not new design"; 16-byte vs
// 8-byte vector loads per head size, same page, "The gap it specs"; wave64 reductions must cross
// all four 16-lane rows, vllm.cpp PR #506 review, finding 2; sliding window with out-of-window
// blocks skipped and attention sinks, randomvariable/vllm issue #23, table "Current state".
#include <cstdio>

#include "pa_device.hpp"
#include "pa_kernels.hpp"

namespace pa {

// Rescale threshold of the online softmax, in log2 units.  The running max m of a row group is
// only raised when a tile's max exceeds it by more than this, so between raises
// p = 2^(s - m) <= 2^kRescaleSlack: no overflow risk in fp32, and most tiles skip the rescale
// multiplies entirely.  The final result does not depend on when rescales happen: every
// (m, l, acc) triple stays consistent and the merges use the exact log-sum-exp rule.
constexpr float kRescaleSlack = 8.0f;

template <int D, int G>
struct WaveState {
  static constexpr int E = RowGeom<D>::kElems;
  float m[G];       // running max of the row group's scores (log2 units), per head
  float l[G];       // running sum of 2^(s - m)
  float acc[G][E];  // running sum of 2^(s - m) v, this lane's slice of the head dim
};

// One tile (16 tokens) of K/V in registers: token 4j + r of the tile is row j of row group r.
template <int D>
struct TileRegs {
  static constexpr int W = RowGeom<D>::kWords;
  uint32_t k[kTileSteps][W];
  uint32_t v[kTileSteps][W];
};

template <int D>
__device__ __forceinline__ void issue_tile(TileRegs<D>& t, const char* kb, const char* vb, int r,
                                           int c) {
  constexpr int RB = RowGeom<D>::kRowBytes;
#pragma unroll
  for (int j = 0; j < kTileSteps; ++j) load_row<D>(kb + (kRows * j + r) * RB, c, t.k[j]);
#pragma unroll
  for (int j = 0; j < kTileSteps; ++j) load_row<D>(vb + (kRows * j + r) * RB, c, t.v[j]);
}

// Fold one tile into the row group's online-softmax state.  MASKED: some tokens of the tile
// fall outside [lo, hi); they get score -inf and a zero value row by select, so whatever their
// slots hold (NaN included) cannot reach the sums.
template <int D, int G, bool MASKED>
__device__ __forceinline__ void consume_tile(WaveState<D, G>& st, TileRegs<D>& t,
                                             const uint32_t (&qw)[G][RowGeom<D>::kWords],
                                             float c2, int tok0, int lo, int hi, int r) {
  constexpr int W = RowGeom<D>::kWords;
  constexpr int E = RowGeom<D>::kElems;
  constexpr int J = kTileSteps;

  // raw scores q.k of the row group's 4 tokens, complete in every lane of the row
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
#pragma unroll
      for (int w = 0; w < W; ++w) t.v[j][w] = ok ? t.v[j][w] : 0u;
    }
  }

  // raise the running max only when a tile's max is well above it (wave-uniform decision)
  float mx[G];
  bool need = false;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mx[h] = fmaxf(fmaxf(s[0][h], s[1][h]), fmaxf(s[2][h], s[3][h]));
    if constexpr (!MASKED) mx[h] *= c2;    // c2 >= 0: the max commutes with the scale
    need |= mx[h] > st.m[h] + kRescaleSlack;
  }
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mn = fmaxf(st.m[h], mx[h]);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(st.m[h] - mu);
      st.l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < E; ++e) st.acc[h][e] *= alpha;
      st.m[h] = mn;
    }
  }

  // probabilities (overwriting the scores), then P.V one token row at a time
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mu = st.m[h] == -INFINITY ? 0.f : st.m[h];
#pragma unroll
    for (int j = 0; j < J; ++j)
      s[j][h] = MASKED ? fast_exp2(s[j][h] - mu) : fast_exp2(fmaf(s[j][h], c2, -mu));
    st.l[h] += (s[0][h] + s[1][h]) + (s[2][h] + s[3][h]);
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
      for (int e = 0; e < E; ++e) st.acc[h][e] = fmaf(s[j][h], vf[e], st.acc[h][e]);
    }
  }
}

template <int D, int G, int NW, int DEPTH>
__global__ __launch_bounds__(NW * kWave) void decode_kernel(const DecodeParams p) {
  using RG = RowGeom<D>;
  constexpr int W = RG::kWords;
  constexpr int E = RG::kElems;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane >> 4;
  const int c = lane & (kRowLanes - 1);
  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;

  const int L = p.seq_lens[b];
  const bool split = p.psize > 0;
  const int n_parts = split ? (L > 0 ? (int)(((int64_t)L + p.psize - 1) / p.psize) : 1) : 1;
  if (part >= n_parts) return;

  // Lengths the table cannot hold, or more partitions than slots: write NaN, read nothing.
  bool bad = L < 0 || (int64_t)L > ((int64_t)p.stride << p.bs_log2);
  if (split && part == p.max_parts - 1 && n_parts > p.max_parts) bad = true;
  const PartRange pr = part_range(bad ? 0 : L, p.window, part, p.psize);

  // q for the G heads of this KV head, bf16 pairs of the lane's slice of the head dim.  A
  // negative scale is applied as |scale| on -q (a sign flip, exact), so the score scale c2 is
  // never negative and commutes with max.
  float c2 = p.qk_scale_log2;
  const uint32_t qflip = c2 < 0.f ? 0x80008000u : 0u;
  c2 = fabsf(c2);
  const int h0 = kvh * G;
  uint32_t qw[G][W];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    load_row_cached<D>(
        reinterpret_cast<const char*>(p.q + ((size_t)b * p.num_q_heads + h0 + h) * D), c,
        qw[h]);
#pragma unroll
    for (int w = 0; w < W; ++w) qw[h][w] ^= qflip;
  }

  WaveState<D, G> st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = -INFINITY;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) st.acc[h][e] = 0.f;
  }

  // Full tiles [f0, f1) are dealt round-robin to the waves: wave w takes f0 + w + NW*i,
  // i in [0, n_w).  Their block-table entries are loaded 64 at a time into one VGPR (lane i holds
  // tile i's physical block) and read back with readlane, so no scalar table load sits on a
  // tile's critical path.  The at most two partial tiles at the range ends (masked) follow.
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
    if (ch != chunk) {   // uniform: refill the lane table for tiles [64ch, 64ch+64)
      chunk = ch;
      const int li = (ch << 6) + lane;
      phys_v = li < n_w ? bt_row[ta.logical_block(first + NW * li)] : 0;
    }
    return __builtin_amdgcn_readlane(phys_v, i & 63);
  };
  auto issue = [&](int i, TileRegs<D>& regs) -> bool {
    const int64_t off = ta.offset(phys_of(i), first + NW * i);
    if (off < 0) {
      bad_table = true;
      return false;
    }
    issue_tile<D>(regs, p.k_cache + off, p.v_cache + off, r, c);
    return true;
  };
  auto consume = [&](int i, TileRegs<D>& regs) {
    consume_tile<D, G, false>(st, regs, qw, c2, 0, 0, 0, r);
  };

  if constexpr (DEPTH == 2) {
    // two tiles in flight: the loads of tile i+1 are issued before tile i is consumed
    TileRegs<D> ra, rb;
    bool oka = n_w > 0 ? issue(0, ra) : false;
    bool okb = false;
    for (int i = 0; i < n_w; i += 2) {
      if (i + 1 < n_w) okb = issue(i + 1, rb);
      if (oka) consume(i, ra);
      if (i + 2 < n_w) oka = issue(i + 2, ra);
      if (i + 1 < n_w && okb) consume(i + 1, rb);
    }
  } else {
    TileRegs<D> ra;
    for (int i = 0; i < n_w; ++i)
      if (issue(i, ra)) consume(i, ra);
  }

  // partial tiles at the ends of [lo, hi), on the last wave
  if (wave == NW - 1 && pr.hi > pr.lo) {
    const int head = pr.lo / kTileTokens;          // partial if lo is not tile-aligned
    const int tail = pr.hi / kTileTokens;          // partial if hi is not tile-aligned
    const bool has_head = head < f0;
    // the tail tile is partial whenever hi is not aligned; it is only skipped when it is the
    // head tile and the head pass (masked to [lo, hi)) already covers it
    const bool has_tail = (pr.hi % kTileTokens) != 0 && !(has_head && tail == head);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const bool on = k == 0 ? has_head : has_tail;
      if (!on) continue;
      const int tile = k == 0 ? head : tail;
      const int64_t off = ta.offset(__builtin_amdgcn_readfirstlane(bt_row[ta.logical_block(tile)]),
                                    tile);
      if (off < 0) {
        bad_table = true;
        continue;
      }
      TileRegs<D> rt;
      issue_tile<D>(rt, p.k_cache + off, p.v_cache + off, r, c);
      consume_tile<D, G, true>(st, rt, qw, c2, tile * kTileTokens, pr.lo, pr.hi, r);
    }
  }

  // merge the 4 row groups of the wave (log-sum-exp rule); every row ends with the wave total
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = rows_max(st.m[h]);
    const float Mu = M == -INFINITY ? 0.f : M;
    const float f = fast_exp2(st.m[h] - Mu);
    st.l[h] = rows_sum(st.l[h] * f);
#pragma unroll
    for (int e = 0; e < E; ++e) st.acc[h][e] = rows_sum(st.acc[h][e] * f);
    st.m[h] = M;
  }

  // merge the waves through LDS
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
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_m[wave][h] = st.m[h];
      s_l[wave][h] = st.l[h];
    }
    s_bad[wave] = bad_table ? 1 : 0;
  }
  __syncthreads();

  bool any_bad = bad;
#pragma unroll
  for (int w = 0; w < NW; ++w) any_bad |= s_bad[w] != 0;

  const bool fold_sink = p.sinks != nullptr && part == pr.first_part;
  for (int i = threadIdx.x; i < G * D; i += NW * kWave) {
    const int h = i / D;
    const int d = i - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float lt = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(s_m[w][h] - Mu);
      lt = fmaf(s_l[w][h], f, lt);
      o = fmaf(s_acc[w][h][d], f, o);
    }
    const int hq = h0 + h;
    if (fold_sink) {
      // the sink logit joins the max and the denominator with a zero value row
      const float s2 = p.sinks[hq] * kLog2e;
      const float M2 = fmaxf(M, s2);
      const float M2u = M2 == -INFINITY ? 0.f : M2;
      const float f = fast_exp2(M - M2u);
      lt = fmaf(lt, f, fast_exp2(s2 - M2u));
      o *= f;
      M = M2;
    }
    float ov = lt > 0.f ? o / lt : 0.f;
    float lv = lt > 0.f ? (M + fast_log2(lt)) * kLn2 : -INFINITY;
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

// ---------------------------------------------------------------------------------------------
// host-side variant table
// ---------------------------------------------------------------------------------------------
namespace {

// tiles in flight per wave: two where the registers allow it
template <int D, int G>
constexpr int pipeline_depth() {
  return (D * G <= 512) ? 2 : 1;
}

template <int D, int G, int NW>
hipError_t launch_dgw(const DecodeParams& p, int num_seqs, hipStream_t stream) {
  const dim3 grid(p.psize > 0 ? p.max_parts : 1, p.num_kv_heads, num_seqs);
  hipLaunchKernelGGL((decode_kernel<D, G, NW, pipeline_depth<D, G>()>), grid, dim3(NW * kWave),
                     0, stream, p);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_dg(const DecodeParams& p, int waves, int num_seqs, hipStream_t stream) {
  switch (waves) {
    case 1: return launch_dgw<D, G, 1>(p, num_seqs, stream);
    case 2: return launch_dgw<D, G, 2>(p, num_seqs, stream);
    case 4: return launch_dgw<D, G, 4>(p, num_seqs, stream);
    case 8: return launch_dgw<D, G, 8>(p, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_d(const DecodeParams& p, int group, int waves, int num_seqs,
                    hipStream_t stream) {
  switch (group) {
    case 1: return launch_dg<D, 1>(p, waves, num_seqs, stream);
    case 2: return launch_dg<D, 2>(p, waves, num_seqs, stream);
    case 4: return launch_dg<D, 4>(p, waves, num_seqs, stream);
    case 8: return launch_dg<D, 8>(p, waves, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_supported(int head_dim, int group) {
  const bool d_ok = head_dim == 64 || head_dim == 128 || head_dim == 256;
  const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8;
  return d_ok && g_ok;
}

bool decode_waves_supported(int waves) {
  return waves == 1 || waves == 2 || waves == 4 || waves == 8;
}

int decode_default_waves(int head_dim, int group, int psize) {
  (void)head_dim;
  (void)group;
  (void)psize;
  return 4;
}

QkPath decode_default_path(int head_dim, int group) {
  (void)head_dim;
  (void)group;
  return QkPath::kMfma;
}

const char* decode_variant_name(int head_dim, int group, int waves, bool split, QkPath path) {
  static thread_local char buf[64];
  std::snprintf(buf, sizeof(buf), "pa_decode_%s_d%d_g%d_w%d%s",
                path == QkPath::kMfma ? "mfma" : "valu", head_dim, group, waves,
                split ? "_split" : "");
  return buf;
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, int group, int waves, int num_seqs,
                         hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<64>(p, group, waves, num_seqs, stream);
    case 128: return launch_d<128>(p, group, waves, num_seqs, stream);
    case 256: return launch_d<256>(p, group, waves, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
