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
#include "pa_device.hpp"
#include "pa_kernels.hpp"

namespace pa {

template <int D, int G, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_kernel(const DecodeParams p) {
  using RG = RowGeom<D>;
  constexpr int W = RG::kWords;
  constexpr int E = RG::kElems;
  constexpr int J = kTileSteps;

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

  // q for the G heads of this KV head, bf16 pairs in the lane's slice of the head dim
  const int h0 = kvh * G;
  uint32_t qw[G][W];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const char* qrow = reinterpret_cast<const char*>(
        p.q + ((size_t)b * p.num_q_heads + h0 + h) * D);
    load_row<D>(qrow, c, qw[h]);
  }

  float m[G], l[G], acc[G][E];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
  }

  const TileAddr ta{p.block_table + (size_t)b * p.stride, p.num_blocks, p.num_kv_heads, kvh,
                    p.bs_log2, RG::kRowBytes};
  const int t0 = pr.lo / kTileTokens;
  const int t1 = pr.hi > pr.lo ? (pr.hi + kTileTokens - 1) / kTileTokens : t0;
  bool bad_table = false;

  for (int t = t0 + wave; t < t1; t += NW) {
    const int64_t off = ta.offset(t);
    if (off < 0) {
      bad_table = true;
      continue;
    }
    const char* kb = p.k_cache + off;
    const char* vb = p.v_cache + off;
    uint32_t kw[J][W], vw[J][W];
#pragma unroll
    for (int j = 0; j < J; ++j) load_row<D>(kb + (kRows * j + r) * RG::kRowBytes, c, kw[j]);
#pragma unroll
    for (int j = 0; j < J; ++j) load_row<D>(vb + (kRows * j + r) * RG::kRowBytes, c, vw[j]);

    // scores of the row group's 4 tokens for the G heads (log2 domain)
    float s[J][G];
#pragma unroll
    for (int j = 0; j < J; ++j) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) a = dot2_bf16(qw[h][w], kw[j][w], a);
        s[j][h] = row_sum16(a) * p.qk_scale_log2;
      }
    }

    const int tok0 = t * kTileTokens;
    if (tok0 < pr.lo || tok0 + kTileTokens > pr.hi) {
      // boundary tile: tokens outside [lo, hi) get score -inf and a zero value row, by select,
      // so whatever those slots hold (NaN included) cannot reach the sums
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int tk = tok0 + kRows * j + r;
        const bool ok = tk >= pr.lo && tk < pr.hi;
#pragma unroll
        for (int h = 0; h < G; ++h) s[j][h] = ok ? s[j][h] : -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) vw[j][w] = ok ? vw[j][w] : 0u;
      }
    }

    float vf[J][E];
#pragma unroll
    for (int j = 0; j < J; ++j) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        vf[j][2 * w] = bf16_lo(vw[j][w]);
        vf[j][2 * w + 1] = bf16_hi(vw[j][w]);
      }
    }

#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mx = fmaxf(fmaxf(s[0][h], s[1][h]), fmaxf(s[2][h], s[3][h]));
      const float mn = fmaxf(m[h], mx);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(m[h] - mu);
      float pj[J];
#pragma unroll
      for (int j = 0; j < J; ++j) pj[j] = fast_exp2(s[j][h] - mu);
      l[h] = fmaf(l[h], alpha, (pj[0] + pj[1]) + (pj[2] + pj[3]));
      m[h] = mn;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float a = acc[h][e] * alpha;
#pragma unroll
        for (int j = 0; j < J; ++j) a = fmaf(pj[j], vf[j][e], a);
        acc[h][e] = a;
      }
    }
  }

  // merge the 4 row groups of the wave (log-sum-exp rule); every row ends with the wave total
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = rows_max(m[h]);
    const float Mu = M == -INFINITY ? 0.f : M;
    const float f = fast_exp2(m[h] - Mu);
    l[h] = rows_sum(l[h] * f);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = rows_sum(acc[h][e] * f);
    m[h] = M;
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
      for (int e = 0; e < E; ++e) s_acc[wave][h][RG::dim(c, e)] = acc[h][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_m[wave][h] = m[h];
      s_l[wave][h] = l[h];
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

constexpr int kWavesPerWg = 4;

template <int D, int G>
hipError_t launch_dg(const DecodeParams& p, int num_seqs, hipStream_t stream) {
  const dim3 grid(p.psize > 0 ? p.max_parts : 1, p.num_kv_heads, num_seqs);
  hipLaunchKernelGGL((decode_kernel<D, G, kWavesPerWg>), grid, dim3(kWavesPerWg * kWave), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeParams& p, int group, int num_seqs, hipStream_t stream) {
  switch (group) {
    case 1: return launch_dg<D, 1>(p, num_seqs, stream);
    case 2: return launch_dg<D, 2>(p, num_seqs, stream);
    case 4: return launch_dg<D, 4>(p, num_seqs, stream);
    case 8: return launch_dg<D, 8>(p, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_supported(int head_dim, int group) {
  const bool d_ok = head_dim == 64 || head_dim == 128 || head_dim == 256;
  const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8;
  return d_ok && g_ok;
}

const char* decode_variant_name(int head_dim, int group, bool split) {
#define PA_NAME(D, G)                                                                 \
  if (head_dim == D && group == G)                                                  \
    return split ? "pa_decode_d" #D "_g" #G "_w4_split" : "pa_decode_d" #D "_g" #G "_w4";
  PA_NAME(64, 1) PA_NAME(64, 2) PA_NAME(64, 4) PA_NAME(64, 8)
  PA_NAME(128, 1) PA_NAME(128, 2) PA_NAME(128, 4) PA_NAME(128, 8)
  PA_NAME(256, 1) PA_NAME(256, 2) PA_NAME(256, 4) PA_NAME(256, 8)
#undef PA_NAME
  return nullptr;
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, int group, int num_seqs,
                         hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<64>(p, group, num_seqs, stream);
    case 128: return launch_d<128>(p, group, num_seqs, stream);
    case 256: return launch_d<256>(p, group, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
