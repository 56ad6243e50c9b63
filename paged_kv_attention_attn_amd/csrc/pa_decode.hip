// Single-token paged-attention decode for gfx950 (CDNA4), unsplit and split-KV.
//
// One workgroup per (partition, KV head, sequence).  It walks the sequence's block table tile by
// tile (16 tokens), loads each tile's K and V rows once with coalesced non-temporal loads, and
// serves all G query heads that share the KV head from the same registers, so every K/V byte is
// read once per KV head.  Softmax is online (running max and sum) in the log2 domain; P.V
// accumulates in fp32.  Each of the 4 row groups (16-lane DPP rows) of a wave runs its own
// online softmax over tokens 4j + r of every tile (a strided subset); the row groups, then the
// waves, are merged with the log-sum-exp rule.  The epilogue folds the sink logit, normalises,
// and writes the final output and LSE (unsplit) or the partition's partial output and LSE.
//
// Two ways to form the scores q.k, selected per variant (QkValu / QkMfma in pa_qk.hpp):
//   - vector ALUs: one KV row per 16-lane row, bf16 dot2 with fp32 accumulation, DPP sum;
//   - matrix cores: per tile the G query heads form a dense [16 x D] . [D x G] contraction,
//     D/32 v_mfma_f32_16x16x32_bf16 (bf16 products, fp32 accumulation, heads padded to 16).
// P.V is on the vector ALUs in fp32 in both: probabilities never round to bf16.
//
// Sources: one-token split-KV decode with partial outputs + LSE and a reduce step,
// ROCm/rocm-libraries PR #13700 "prepare saved paged decode bindings once", Summary; online
// softmax reaching the same function in another order, vllm.cpp PR #564 "spec(BACKEND-ROCM): the
// ROCm head_dim=128 decode arm", "It is a mirror of merged work, not new design"; GQA groups,
// same page, "What is deliberately not here"; 16-byte vs 8-byte vector loads per head size, same
// page, "The gap it specs"; a separate matrix-core arm for d=128, same page, "One deviation from
// the original commit"; wave64 reductions must cross all four 16-lane rows, vllm.cpp PR #506
// review, finding 2; sliding window with out-of-window blocks skipped and attention sinks,
// randomvariable/vllm issue #23, table "Current state".
#include <cstdio>
#include <type_traits>

#include "pa_device.hpp"
#include "pa_kernels.hpp"
#include "pa_qk.hpp"

namespace pa {

// ---------------------------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------------------------
template <int D, int G, int NW, int DEPTH, class QK>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(QK::kMinWavesPerEu)))
void decode_kernel(const DecodeParams p) {
  using RG = RowGeom<D>;
  constexpr int E = RG::kElems;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & (kRowLanes - 1);
  const WorkItem it = decode_work_item(p.num_kv_heads, p.num_seqs);
  const int h0 = it.kvh * G;
  const bool split = p.psize > 0;

  // A negative scale is applied as |scale| on -q (a sign flip, exact), so the score scale c2 is
  // never negative and commutes with max.
  const float c2 = fabsf(p.qk_scale_log2);
  const uint32_t qflip = p.qk_scale_log2 < 0.f ? 0x80008000u : 0u;
  QK qk;
  qk.init(p, make_qshape<false, G>(p), it.b, h0, lane, qflip, c2);

  // Block-table entries of this wave's tiles, 64 at a time in one VGPR (lane i: tile i).  The
  // first batch is requested before the sequence length arrives, for the range a partition has
  // without a window (indices clamped into the row, so always in bounds); a window start that
  // moves the range triggers a reload below.
  const TileAddr ta{p.num_blocks, p.bs_log2, p.kv_block_stride, it.kvh * p.kv_head_stride,
                    p.kv_row_stride};
  const int32_t* bt_row = p.block_table + (size_t)it.b * p.stride;
  const int lo_guess =
      split ? (int)((int64_t)it.part * p.psize < 0x7FFFFFF0 ? (int64_t)it.part * p.psize
                                                              : 0x7FFFFFF0)
            : 0;
  const int first_guess = (lo_guess + kTileTokens - 1) / kTileTokens + wave;
  const int row_cap = p.stride - 1;
  auto table_batch = [&](int first, int ch) -> int {
    const int li = (ch << 6) + lane;
    const int lb = ta.logical_block(first + NW * li);
    return bt_row[lb < row_cap ? lb : row_cap];
  };
  int phys_v = table_batch(first_guess, 0);

  const int L = p.seq_lens[it.b];
  const int n_parts = split ? (L > 0 ? (int)(((int64_t)L + p.psize - 1) / p.psize) : 1) : 1;
  if (it.part >= n_parts) return;   // uniform over the workgroup
  // Lengths the table cannot hold, or more partitions than slots: write NaN, read nothing.
  bool bad = L < 0 || (int64_t)L > ((int64_t)p.stride << p.bs_log2);
  if (split && it.part == p.max_parts - 1 && n_parts > p.max_parts) bad = true;
  const PartRange pr = part_range(bad ? 0 : L, p.window, it.part, p.psize);

  // full tiles [f0, f1) round-robin over the waves: wave w takes f0 + w + NW*i, i < n_w
  const int f0 = (pr.lo + kTileTokens - 1) / kTileTokens;
  const int f1 = pr.hi / kTileTokens;
  const int first = f0 + wave;
  const int n_w = first < f1 ? (f1 - first + NW - 1) / NW : 0;
  int chunk = first == first_guess ? 0 : -1;
  bool bad_table = false;

  auto phys_of = [&](int i) -> int {
    const int ch = i >> 6;
    if (ch != chunk) {   // uniform
      chunk = ch;
      phys_v = table_batch(first, ch);
    }
    return __builtin_amdgcn_readlane(phys_v, i & 63);
  };
  auto issue = [&](int i, typename QK::Tile& t) -> bool {
    const int64_t off = ta.offset(phys_of(i), first + NW * i);
    if (off < 0) {
      bad_table = true;
      return false;
    }
    qk.issue(t, p.k_cache + off, p.v_cache + off, lane);
    return true;
  };

  if constexpr (DEPTH == 2) {
    // two tiles in flight: the loads of tile i+1 are issued before tile i is consumed
    typename QK::Tile t0_, t1_;
    bool ok0 = n_w > 0 ? issue(0, t0_) : false;
    bool ok1 = false;
    for (int i = 0; i < n_w; i += 2) {
      if (i + 1 < n_w) ok1 = issue(i + 1, t1_);
      if (ok0) qk.template consume<false>(t0_, 0, 0, 0, lane);
      if (i + 2 < n_w) ok0 = issue(i + 2, t0_);
      if (i + 1 < n_w && ok1) qk.template consume<false>(t1_, 0, 0, 0, lane);
    }
  } else {
    typename QK::Tile t0_;
    for (int i = 0; i < n_w; ++i)
      if (issue(i, t0_)) qk.template consume<false>(t0_, 0, 0, 0, lane);
  }

  // the at most two partial tiles at the ends of [lo, hi), masked, on the last wave
  if (wave == NW - 1 && pr.hi > pr.lo) {
    const int head = pr.lo / kTileTokens;
    const int tail = pr.hi / kTileTokens;
    const bool has_head = head < f0;
    // the tail tile is partial whenever hi is not aligned; it is skipped only when it is the
    // head tile and the head pass (masked to [lo, hi)) already covers it
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
      typename QK::Tile t;
      qk.issue(t, p.k_cache + off, p.v_cache + off, lane);
      qk.template consume<true>(t, tile * kTileTokens, pr.lo, pr.hi, lane);
    }
  }

  // merge rows within the wave, then waves through LDS
  float Mh[G], lh[G];
  qk.merge_rows(Mh, lh);
  __shared__ float s_acc[NW][G][D];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];
  __shared__ int s_bad[NW];
  if (lane < kRowLanes) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < E; ++e) s_acc[wave][h][RG::dim(c, e)] = qk.out(h, e);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_m[wave][h] = Mh[h];
      s_l[wave][h] = lh[h];
    }
    s_bad[wave] = bad_table ? 1 : 0;
  }
  __syncthreads();

  bool any_bad = bad;
#pragma unroll
  for (int w = 0; w < NW; ++w) any_bad |= s_bad[w] != 0;

  const bool fold_sink = p.sinks != nullptr && it.part == pr.first_part;
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
    // lt is 0 only for an empty range; a NaN score (lt = NaN) must reach the outputs
    float ov = lt != 0.f ? o / lt : 0.f;
    float lv = lt != 0.f ? (M + fast_log2(lt)) * kLn2 : -INFINITY;
    if (any_bad) {
      ov = __builtin_nanf("");
      lv = __builtin_nanf("");
    }
    const size_t row = (size_t)it.b * p.num_q_heads + hq;
    if (split) {
      p.out[(row * p.max_parts + it.part) * D + d] = ov;
      if (d == 0) p.lse[row * p.max_parts + it.part] = lv;
    } else {
      p.out[row * D + d] = ov;
      if (d == 0 && p.lse != nullptr) p.lse[row] = lv;
    }
  }

  // Merge in the same launch: every partition of (b, kvh) bumps its counter after releasing its
  // partials to the device; the one that brings it to the partition count merges them all with
  // the log-sum-exp rule (as the reduce kernel does) and puts the counter back to zero.
  if (split && p.merge_counters != nullptr) {
    __shared__ int s_last;
    const int target = n_parts < p.max_parts ? n_parts : p.max_parts;
    __syncthreads();   // every thread's partial stores happen before thread 0's release
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      uint32_t* ctr = p.merge_counters + (size_t)it.b * p.num_kv_heads + it.kvh;
      const uint32_t old =
          __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = old == (uint32_t)(target - 1);
      if (last) {
        __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
      s_last = last ? 1 : 0;
    }
    __syncthreads();   // thread 0's acquire happens before every thread's loads below
    if (s_last) {
      for (int i = threadIdx.x; i < G * D; i += NW * kWave) {
        const int h = i / D;
        const int d = i - h * D;
        const size_t row = (size_t)it.b * p.num_q_heads + h0 + h;
        const float* lr = p.lse + row * p.max_parts;
        float M = -INFINITY;
        bool nan = false;
        for (int q = 0; q < target; ++q) {
          const float v = lr[q];
          nan |= v != v;
          M = fmaxf(M, v);
        }
        const float Mu = M == -INFINITY ? 0.f : M;
        float z = 0.f, o = 0.f;
        for (int q = 0; q < target; ++q) {
          const float li = lr[q];
          if (!(li > -INFINITY)) continue;   // an empty partition (or NaN, reported)
          const float f = fast_exp2((li - Mu) * kLog2e);
          z += f;
          o = fmaf(f, p.out[(row * p.max_parts + q) * D + d], o);
        }
        float ov = z > 0.f ? o / z : 0.f;
        float lv = z > 0.f ? M + fast_log2(z) * kLn2 : -INFINITY;
        if (nan) {
          ov = __builtin_nanf("");
          lv = __builtin_nanf("");
        }
        p.final_out[row * D + d] = ov;
        if (d == 0 && p.final_lse != nullptr) p.final_lse[row] = lv;
      }
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
  return D * G <= 512 ? 2 : 1;
}

template <int D, int G, int NW, QkPath PATH>
hipError_t launch_v(const DecodeParams& p, hipStream_t stream) {
  using QK = QkPolicy<D, G, PATH>;
  const unsigned grid = (unsigned)((p.psize > 0 ? p.max_parts : 1) *
                                   (int64_t)p.num_kv_heads * p.num_seqs);
  hipLaunchKernelGGL((decode_kernel<D, G, NW, pipeline_depth<D, G>(), QK>), dim3(grid),
                     dim3(NW * kWave), 0, stream, p);
  return hipGetLastError();
}

template <int D, int G, QkPath PATH>
hipError_t launch_w(const DecodeParams& p, int waves, hipStream_t stream) {
  switch (waves) {
    case 1: return launch_v<D, G, 1, PATH>(p, stream);
    case 2: return launch_v<D, G, 2, PATH>(p, stream);
    case 4: return launch_v<D, G, 4, PATH>(p, stream);
    case 8: return launch_v<D, G, 8, PATH>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D, QkPath PATH>
hipError_t launch_g(const DecodeParams& p, int group, int waves, hipStream_t stream) {
  switch (group) {
    case 1: return launch_w<D, 1, PATH>(p, waves, stream);
    case 2: return launch_w<D, 2, PATH>(p, waves, stream);
    case 4: return launch_w<D, 4, PATH>(p, waves, stream);
    case 8: return launch_w<D, 8, PATH>(p, waves, stream);
    default: return hipErrorInvalidValue;
  }
}

template <QkPath PATH>
hipError_t launch_d(const DecodeParams& p, int head_dim, int group, int waves,
                    hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_g<64, PATH>(p, group, waves, stream);
    case 128: return launch_g<128, PATH>(p, group, waves, stream);
    case 256: return launch_g<256, PATH>(p, group, waves, stream);
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
  // P.V on the matrix cores pays once a KV head serves two or more query heads; a single head
  // would use one row of sixteen.
  (void)head_dim;
  return group >= 2 ? QkPath::kMfmaPv : QkPath::kMfma;
}

const char* qk_path_name(QkPath path) {
  switch (path) {
    case QkPath::kValu: return "valu";
    case QkPath::kMfma: return "mfma";
    case QkPath::kMfmaPvFp8: return "mfmapv_fp8";
    case QkPath::kMfmaPvHeads2: return "mfmapv_headpairs";
    case QkPath::kMfmaPvFp8Heads2: return "mfmapv_fp8_headpairs";
    default: return "mfmapv";
  }
}

const char* decode_variant_name(int head_dim, int group, int waves, bool split, QkPath path) {
  static thread_local char buf[64];
  std::snprintf(buf, sizeof(buf), "pa_decode_%s_d%d_g%d_w%d%s",
                qk_path_name(path), head_dim, group, waves,
                split ? "_split" : "");
  return buf;
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, int group, int waves, QkPath path,
                         hipStream_t stream) {
  switch (path) {
    case QkPath::kValu: return launch_d<QkPath::kValu>(p, head_dim, group, waves, stream);
    case QkPath::kMfma: return launch_d<QkPath::kMfma>(p, head_dim, group, waves, stream);
    case QkPath::kMfmaPvFp8:
      return launch_d<QkPath::kMfmaPvFp8>(p, head_dim, group, waves, stream);
    default: return launch_d<QkPath::kMfmaPv>(p, head_dim, group, waves, stream);
  }
}

}  // namespace pa
