// Query blocks for several query tokens per sequence (chunked prefill, speculative decode) on
// gfx950.
//
// A block of tokens holds the columns of one wave, 32 (token, head) pairs at head_dim <= 128
// and 16 at 256, so tokens_per_block = columns / group.  A wave folds the 16-token K/V tiles its
// tokens attend (the union of their causal, windowed ranges) into its columns, forming q.k and
// P.V on the matrix cores exactly as the one-token kernels do (each column masked to its own
// token's range inside the shared tiles), and writes its outputs and LSEs.  When a batch has
// too few blocks to fill the GPU (one or a few sequences), each block's key range is cut into
// key splits, one workgroup each, that write normalised partial outputs and LSEs; a merge
// kernel then combines each row's splits by the log-sum-exp rule and folds the sink.  Two forms:
//   - qblock_lds_kernel: four waves per workgroup, four consecutive blocks of one (sequence,
//     KV head), sharing every tile through an LDS ring (used from four blocks per sequence);
//   - qblock_kernel: one wave per block, loading its own tiles (fewer blocks).
//
// All blocks of a (sequence, KV head) read the same keys.  The chip deals workgroups to its
// 8 XCDs round-robin by linear id; with xcd_pinned every workgroup of one (sequence, KV head)
// gets an id of the same residue mod 8, so they run on one XCD, close in time, and share its
// L2: the K/V loads are plain (cached) here, not non-temporal.  Within a (sequence, KV head)
// the blocks of the last tokens, which attend the most keys, are dealt first.
//
// Token i of q_total new tokens sits at position L - q_total + i and attends keys t <= its
// position, the last `window` of them when window > 0: the longer-query case that vllm.cpp
// PR #564 "spec(BACKEND-ROCM): the ROCm head_dim=128 decode arm" ("What is deliberately not
// here") leaves out and ROCm/rocm-libraries PR #13700 "prepare saved paged decode bindings
// once" fixes at one token; the causal rule is this library's reading.  Sinks: randomvariable/
// vllm issue #23, table "Current state" (a sink logit joins the softmax with a zero value row).
#include <algorithm>

#include "pa_device.hpp"
#include "pa_kernels.hpp"
#include "pa_qk.hpp"

namespace pa {

namespace {

constexpr int kXcds = 8;
// key splits (small batches): waves aimed for, tiles per split at least, splits at most
constexpr long long kQbTargetWaves = 2048;
constexpr long long kQbMinSplitTiles = 8;
constexpr int kQbMaxSplits = 64;

struct QBlockItem {
  int b, kvh, qb, split;
};

// The (sequence, KV head, query block, key split) of this workgroup; false for an idle id.
// Within a (sequence, KV head) the splits of one block are consecutive ids.
__device__ __forceinline__ bool qblock_item(const QBlockParams& qp, QBlockItem& it) {
  const int U = qp.d.num_seqs * qp.d.num_kv_heads;
  const int nqb = qp.blocks_per_seq * qp.splits;
  const unsigned id = blockIdx.x;
  unsigned u, j;
  if (qp.xcd_pinned) {
    // XCD x = id mod 8 runs units x, x + 8, ... one after another, each block by block
    const unsigned x = id % kXcds, jj = id / kXcds;
    const unsigned uu = jj / (unsigned)nqb;
    j = jj - uu * (unsigned)nqb;
    u = uu * kXcds + x;
  } else {
    u = id / (unsigned)nqb;
    j = id - u * (unsigned)nqb;
  }
  if (u >= (unsigned)U) return false;
  it.b = (int)(u / (unsigned)qp.d.num_kv_heads);
  it.kvh = (int)(u - (unsigned)it.b * (unsigned)qp.d.num_kv_heads);
  const unsigned jb = j / (unsigned)qp.splits;
  it.split = (int)(j - jb * (unsigned)qp.splits);
  it.qb = qp.blocks_per_seq - 1 - (int)jb;
  return true;
}

// Restricts a key range (tiles t0 .. t0 + T - 1) to its key split: split k takes split_tiles
// tiles from t0 + k * split_tiles, the last one everything after.
__device__ __forceinline__ void clip_to_split(const QBlockParams& qp, int split, SeqSpan& s) {
  if (qp.splits == 1) return;
  const int lo = split * qp.split_tiles;
  const int hi = split == qp.splits - 1 ? s.T : min(s.T, lo + qp.split_tiles);
  s.t0 += lo;
  s.T = max(0, hi - lo);
}

// Writes column n's result: with one split the final output row (sink folded, the caller's lse
// if any), with several the split's normalised partial and its LSE.  M, lt: the column's max
// (log2 units) and denominator; acc(e): its unnormalised output elements.
template <int D, class ACC>
__device__ __forceinline__ void write_column(const QBlockParams& qp, int split, size_t row, int hq,
                                             float M, float lt, bool bad, int c, ACC acc) {
  using RG = RowGeom<D>;
  constexpr int E = RG::kElems;
  const DecodeParams& p = qp.d;
  float scale_o = 1.f;
  if (p.sinks != nullptr && qp.splits == 1) {
    // the sink logit joins the max and the denominator with a zero value row
    const float s2 = p.sinks[hq] * kLog2e;
    const float M2 = fmaxf(M, s2);
    const float M2u = M2 == -INFINITY ? 0.f : M2;
    scale_o = fast_exp2(M - M2u);
    lt = fmaf(lt, scale_o, fast_exp2(s2 - M2u));
    M = M2;
  }
  // lt is 0 only for a column without keys; a NaN input (lt = NaN) reaches the outputs
  const float inv = lt != 0.f ? scale_o / lt : 0.f;
  float lv = lt != 0.f ? (M + fast_log2(lt)) * kLn2 : -INFINITY;
  if (bad) lv = __builtin_nanf("");
  float* dst;
  if (qp.splits == 1) {
    dst = p.out + row * D;
    if (c == 0 && p.lse != nullptr) p.lse[row] = lv;
  } else {
    const size_t slot = row * (size_t)qp.splits + split;
    dst = qp.part_out + slot * D;
    if (c == 0) qp.part_lse[slot] = lv;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) dst[RG::dim(c, e)] = bad ? __builtin_nanf("") : acc(e) * inv;
}

template <int D, class QK, int DEPTH, int WPE>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(WPE)))
void qblock_kernel(const QBlockParams qp) {
  const DecodeParams& p = qp.d;
  QBlockItem it;
  if (!qblock_item(qp, it)) return;
  const int lane = threadIdx.x;
  const int c = lane & (kRowLanes - 1);
  const int q0 = it.qb * qp.tokens_per_block;
  const int nq = min(qp.tokens_per_block, p.q_total - q0);
  const QShape qs{nq, p.q_total, q0, p.group};
  // this block's keys: the union of its tokens' ranges, ending at its last token's position
  const int swin = p.window > 0 ? p.window + nq - 1 : 0;
  SeqSpan s = seq_span(__builtin_amdgcn_readfirstlane(p.seq_lens[it.b]), swin,
                       (int64_t)p.stride << p.bs_log2, p.q_total - q0 - nq);
  clip_to_split(qp, it.split, s);

  const float c2 = fabsf(p.qk_scale_log2);
  const uint32_t qflip = p.qk_scale_log2 < 0.f ? 0x80008000u : 0u;
  const int h0 = it.kvh * qs.group;
  QK qk;
  qk.init(p, qs, it.b, h0, lane, qflip, c2);

  const TileAddr ta{p.num_blocks, p.bs_log2, p.kv_block_stride, it.kvh * p.kv_head_stride,
                    p.kv_row_stride};
  const int32_t* bt = p.block_table + (size_t)it.b * p.stride;
  bool bad = s.bad;
  // every column sees the keys in [lo_all, hi_all): from the last token's window start to the
  // first token's position
  const int hi_all = s.L - nq + 1;
  const int lo_all = (p.window > 0 && s.L > p.window) ? s.L - p.window : 0;

  // tiles s.t0 .. s.t0 + s.T - 1, DEPTH - 1 tiles' loads in flight ahead of the one being
  // consumed; the block-table entry is fetched one issue ahead
  int phys_next = s.T > 0 ? __builtin_amdgcn_readfirstlane(bt[ta.logical_block(s.t0)]) : 0;
  auto issue = [&](int k, typename QK::Tile& t) -> bool {
    const int tile = s.t0 + k;
    const int phys = phys_next;
    if (k + 1 < s.T) phys_next = __builtin_amdgcn_readfirstlane(bt[ta.logical_block(tile + 1)]);
    const int64_t off = ta.offset(phys, tile);
    if (off < 0) return false;
    qk.issue(t, p.k_cache + off, p.v_cache + off, lane);
    return true;
  };
  auto consume = [&](int k, typename QK::Tile& t, bool ok) {
    if (!ok) {   // a table entry outside the pool: never read through, NaN outputs
      bad = true;
      return;
    }
    const int tok0 = (s.t0 + k) * kTileTokens;
    if (tok0 >= lo_all && tok0 + kTileTokens <= hi_all)
      qk.template consume<false>(t, 0, 0, 0, lane);
    else
      qk.consume_cols(t, tok0, hi_all, p.window, s.start, s.L, lane);
  };
  // DEPTH tiles in flight; the loop is unrolled DEPTH times so every buffer index is a constant
  typename QK::Tile tl[DEPTH];
  bool ok[DEPTH];
#pragma unroll
  for (int j = 0; j + 1 < DEPTH; ++j)
    if (j < s.T) ok[j] = issue(j, tl[j]);
  for (int k = 0; k < s.T; k += DEPTH) {
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      const int jn = (j + DEPTH - 1) % DEPTH;
      if (k + j + DEPTH - 1 < s.T) ok[jn] = issue(k + j + DEPTH - 1, tl[jn]);
      if (k + j < s.T) consume(k + j, tl[j], ok[j]);
    }
  }

  // finish column-wise: lane (r, c) writes columns cb + 4r + i, i < 4, that exist, of each
  // 16-column half (cb = 0, 16)
  const int ncols = nq * qs.group;
  const int sh = __builtin_ctz((unsigned)qs.group);
  auto finish_half = [&](auto& half, int cb) {
    half.merge_cols();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int nl = 4 * (lane >> 4) + i;               // column within the half
      const int n = cb + nl;
      const float M = half.col_m(nl), lt = half.col_l(nl);   // every lane takes part
      if (n < ncols) {
        const int hq = h0 + (n & (qs.group - 1));
        const size_t row = ((size_t)it.b * qs.q_total + q0 + (n >> sh)) * p.num_q_heads + hq;
        write_column<D>(qp, it.split, row, hq, M, lt, bad, c,
                        [&](int e) { return half.acc(i, e); });
      }
    }
  };
  if constexpr (QK::kHalves == 2) {
    finish_half(qk.h[0], 0);
    finish_half(qk.h[1], 16);
  } else {
    finish_half(qk, 0);
  }
}

// The workgroup form: kQbWaves waves share each K/V tile through LDS.  A workgroup takes
// kQbWaves consecutive token blocks of one (sequence, KV head), wave w the w-th, and streams the
// union of their key ranges: the tile A tiles ahead is copied straight from the pool into an LDS
// ring of A + 1 tiles by direct-to-LDS loads (no registers hold it in flight), every wave waits
// for its own copies of the current tile and meets the others at a barrier, then reads the tile
// from LDS into its registers and folds it into its columns.  Each key row is read from L2 or
// HBM once per workgroup, not once per wave, and a wave never waits on its own tile loads.
constexpr int kQbWaves = 4;
constexpr int kQbTableTiles = kQbWaves * kWave;   // block-table window in LDS, one per thread

// One 16-byte piece per lane from global memory straight into LDS, lane i's piece at
// lds_wave_base + 16 i (global_load_lds_dwordx4; M0 holds the wave's LDS base).  Written as
// inline assembly so that the compiler does not treat every later LDS read as possibly aliasing
// the copy and wait for all copies in flight before it; the caller waits for the copies itself
// (vmcnt) before the barrier that publishes them.  The instruction writes no register.
__device__ __forceinline__ void copy_piece_to_lds(const char* src, const char* lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)reinterpret_cast<uintptr_t>(lds_wave_base));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               ::"s"(lds), "v"(src)
               : "memory", "m0");
}

template <int D, class QK, int A>
__global__ __launch_bounds__(kQbWaves * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void qblock_lds_kernel(const QBlockParams qp) {
  constexpr int RB = QK::kRowBytes;
  constexpr int PR = RB / 16;                          // 16-byte pieces per row
  constexpr int TB = 2 * kTileTokens * RB;             // K rows, then V rows
  constexpr int NBUF = A + 1;
  constexpr int PIECES = TB / 16;
  static_assert(PIECES % kWave == 0, "a tile is whole wave copies");
  // copies (one 16-byte piece per lane) each loading wave makes per tile
  constexpr int PW = PIECES / (kQbWaves * kWave);
  constexpr int LOADERS = PW > 0 ? kQbWaves : PIECES / kWave;
  constexpr int PL = PW > 0 ? PW : 1;
  __shared__ __attribute__((aligned(16))) char s_tiles[NBUF * TB];

  const DecodeParams& p = qp.d;
  QBlockItem it;
  if (!qblock_item(qp, it)) return;   // uniform over the workgroup
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int c = lane & (kRowLanes - 1);
  const int tpb = qp.tokens_per_block;
  const int64_t cap = (int64_t)p.stride << p.bs_log2;
  const int Lraw = __builtin_amdgcn_readfirstlane(p.seq_lens[it.b]);
  // the workgroup's tokens and the union of their keys
  const int q0w = it.qb * kQbWaves * tpb;
  const int nqw = min(kQbWaves * tpb, p.q_total - q0w);
  SeqSpan sw = seq_span(Lraw, p.window > 0 ? p.window + nqw - 1 : 0, cap,
                        p.q_total - q0w - nqw);
  clip_to_split(qp, it.split, sw);
  // this wave's tokens (none for a wave past the last block) and their keys
  const int q0 = q0w + wave * tpb;
  const int nq = max(0, min(tpb, p.q_total - q0));
  const bool active = nq > 0;
  const QShape qs{nq, p.q_total, q0, p.group};
  const SeqSpan s = seq_span(Lraw, p.window > 0 ? p.window + nq - 1 : 0, cap,
                             max(0, p.q_total - q0 - nq));

  const float c2 = fabsf(p.qk_scale_log2);
  const uint32_t qflip = p.qk_scale_log2 < 0.f ? 0x80008000u : 0u;
  const int h0 = it.kvh * p.group;
  QK qk;
  if (active) qk.init(p, qs, it.b, h0, lane, qflip, c2);

  const TileAddr ta{p.num_blocks, p.bs_log2, p.kv_block_stride, it.kvh * p.kv_head_stride,
                    p.kv_row_stride};
  const int rs = (int)p.kv_row_stride;
  const int32_t* bt = p.block_table + (size_t)it.b * p.stride;
  bool bad = sw.bad;

  // the physical blocks of workgroup tiles [base, base + kQbTableTiles), one per thread, in LDS:
  // reading them there keeps the tile loop free of vector loads other than the copies (a vector
  // load's wait would also wait for every copy in flight)
  __shared__ int s_phys[kQbTableTiles];
  auto fill_table = [&](int base) {
    const int k = base + (int)threadIdx.x;
    s_phys[threadIdx.x] = k < sw.T ? bt[ta.logical_block(sw.t0 + k)] : -1;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  fill_table(0);

  // copy workgroup tile k (tile sw.t0 + k) into ring slot k % NBUF; past the last tile, or for
  // a table entry outside the pool, the lanes copy from q instead (valid memory, never read
  // back), so that every wave always has the same number of copies in flight
  uint32_t okbits = 0;   // bit k % NBUF: tile k came from the pool
  auto copy = [&](int k) {
    int64_t off = -1;
    if (k < sw.T)
      off = ta.offset(__builtin_amdgcn_readfirstlane(s_phys[k % kQbTableTiles]), sw.t0 + k);
    const int slot = k % NBUF;
    okbits = (okbits & ~(1u << slot)) | ((off >= 0 ? 1u : 0u) << slot);
    if (wave < LOADERS) {
#pragma unroll
      for (int m = 0; m < PL; ++m) {
        const int piece = (wave * PL + m) * kWave + lane;   // its place in the tile copy
        const int h = piece / (kTileTokens * PR);
        const int row = (piece / PR) % kTileTokens;
        const int col = (piece % PR) ^ (row & QK::kLdsSwizzle);   // the pool's piece
        const char* src = off >= 0 ? (h ? p.v_cache : p.k_cache) + off + row * rs + col * 16
                                   : reinterpret_cast<const char*>(p.q) + (lane & 7) * 16;
        copy_piece_to_lds(src, s_tiles + slot * TB + (wave * PL + m) * kWave * 16);
      }
    }
  };

  // every column of this wave sees the keys in [lo_all, hi_all)
  const int hi_all = s.L - nq + 1;
  const int lo_all = (p.window > 0 && s.L > p.window) ? s.L - p.window : 0;
  typename QK::Tile t;
#pragma unroll
  for (int k = 0; k < A; ++k) copy(k);
  for (int k = 0; k < sw.T; ++k) {
    // this wave's copies of tile k are done once at most those of the A - 1 later tiles are
    // outstanding; the barrier then makes the whole tile visible, and every wave has finished
    // reading tile k - 1, whose slot the next copy reuses
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(PL * (A - 1)) : "memory");
    if ((k + A) % kQbTableTiles == 0 && k + A < sw.T) fill_table(k + A);   // uniform
    copy(k + A);
    const int tile = sw.t0 + k;
    if (active && tile >= s.t0 && tile < s.t0 + s.T) {
      if (!((okbits >> (k % NBUF)) & 1u)) {
        bad = true;   // a table entry outside the pool: never read through, NaN outputs
      } else {
        qk.fill_from_lds(t, s_tiles + (k % NBUF) * TB, lane);
        const int tok0 = tile * kTileTokens;
        if (tok0 >= lo_all && tok0 + kTileTokens <= hi_all)
          qk.template consume<false>(t, 0, 0, 0, lane);
        else
          qk.consume_cols(t, tok0, hi_all, p.window, s.start, s.L, lane);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the copies past the last tile
  if (!active) return;
  bad = bad || s.bad;

  const int ncols = nq * qs.group;
  const int sh = __builtin_ctz((unsigned)qs.group);
  auto finish_half = [&](auto& half, int cb) {
    half.merge_cols();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int nl = 4 * (lane >> 4) + i;
      const int n = cb + nl;
      const float M = half.col_m(nl), lt = half.col_l(nl);   // every lane takes part
      if (n < ncols) {
        const int hq = h0 + (n & (qs.group - 1));
        const size_t row = ((size_t)it.b * qs.q_total + q0 + (n >> sh)) * p.num_q_heads + hq;
        write_column<D>(qp, it.split, row, hq, M, lt, bad, c,
                        [&](int e) { return half.acc(i, e); });
      }
    }
  };
  if constexpr (QK::kHalves == 2) {
    finish_half(qk.h[0], 0);
    finish_half(qk.h[1], 16);
  } else {
    finish_half(qk, 0);
  }
}

// ---------------------------------------------------------------------------------------------
// The workgroup form on 32-key tiles (bf16 caches, head_dim 64 and 128): four waves, each with
// 32 (token, head) rows, share a ring of 32-key K/V tiles in LDS as in qblock_lds_kernel, and each
// wave folds a tile into its rows with 32x32x16 MFMAs in the transposed form of the two
// contractions:
//   S^T = K Q^T     A = the tile's K rows (32 keys x 16 dims per MFMA), B = the wave's q rows;
//                   lane l ends with the scores of row l % 32 for 16 of the 32 keys (C row
//                   8 (v / 4) + 4 (l / 32) + v % 4 is key v of its half), so the other 16 of its
//                   row sit in lane l ^ 32;
//   O^T += V^T P^T  A = V^T (32 head-dim values x 16 keys), B = P^T: lane l gives row l % 32's
//                   probabilities of keys 8 (j / 4) + 4 (l / 32) + j % 4 (+16 for the second half
//                   of the tile), exactly the scores it holds, so nothing moves between the two
//                   contractions; A takes, per lane, one head-dim slice of eight key rows read from
//                   LDS (rows of the lane's half, slice E (l % 32) .. + E of the row, E = D / 32)
//                   and regrouped into E operands by byte permutes: MFMA e's A row i is head-dim
//                   E i + e.
// Lanes l and l ^ 32 hold the same (token, head) row, so its running max, rescale and output
// live in its own lanes: no broadcast of softmax factors across the wave.  P enters as two bf16
// terms (hi + lo), both products exact with fp32 accumulation, as in the one-token kernels.
// ---------------------------------------------------------------------------------------------
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int D>
struct Fa {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static constexpr int kKeys = 32;             // keys per tile (two 16-token tiles)
  static constexpr int RB = 2 * D;             // bytes per K/V row
  static constexpr int PR = RB / 16;           // 16-byte pieces per row
  static constexpr int TB = 2 * kKeys * RB;    // bytes per tile: K rows, then V rows
  static constexpr int KS = D / 16;            // score MFMAs per tile (16 head dims each)
  static constexpr int E = D / 32;             // P.V MFMAs per 16 keys (head-dim slices)
  // Where piece p of a row sits: K row r at p ^ (r % PR), which spreads the 32 rows a score
  // operand read touches over the banks; V row r at p ^ (PR / 2 if bit 2 of r is set), so that
  // the two lane halves of a P.V operand read (rows 4 apart) fall on opposite halves of the
  // banks while a lane's slice keeps the same place in every row it reads.
  __device__ __host__ static constexpr int swz(int hk, int r) {
    return hk == 0 ? (r & (PR - 1)) : ((r >> 2) & 1) * (PR / 2);
  }
};

// Key of score v (0..15) in lane half h, within a 32-key tile.
__device__ __forceinline__ constexpr int fa_key(int v, int h) {
  return 8 * (v >> 2) + 4 * h + (v & 3);
}

// From head_dim 128 on, a tile's P.V is issued a step late, behind the next tile's score MFMAs
// (at head_dim 64 the score MFMAs are too few to hide it, and the ring is better spent on a third
// tile in flight).  32-key tiles copied ahead: the ring holds them, the tile being folded and,
// with P.V a step late, the one before it (its V read again from LDS): four in all.
template <int D> constexpr bool fa_defer_pv() { return D >= 128; }
template <int D> constexpr int fa_ahead() { return fa_defer_pv<D>() ? 2 : 3; }

// max and sum over the two lane halves (lanes l and l ^ 32), without the LDS crossbar:
// v_permlane32_swap exchanges the halves of its two operands, so the pair it returns holds, at
// every lane position, the values of both lanes l % 32 and l % 32 + 32
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x),
                                                  __builtin_bit_cast(int, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x),
                                                  __builtin_bit_cast(int, x), false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

template <int D, bool HILO, int A>
__global__ __launch_bounds__(kQbWaves * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void qblock_fa_kernel(const QBlockParams qp) {
  using F = Fa<D>;
  constexpr bool DEFER = fa_defer_pv<D>();
  constexpr int NBUF = A + (DEFER ? 2 : 1);
  constexpr int PIECES = F::TB / 16;
  static_assert(PIECES % (kQbWaves * kWave) == 0, "a tile is whole workgroup copies");
  constexpr int PL = PIECES / (kQbWaves * kWave);   // copies per lane per tile
  constexpr int kTablePairs = kQbTableTiles / 2;    // 32-key tiles per table window
  static_assert(kTablePairs % NBUF == 0, "table refills fall on unrolled iterations");
  __shared__ __attribute__((aligned(16))) char s_tiles[NBUF * F::TB];
  __shared__ int64_t s_off[kQbTableTiles];

  const DecodeParams& p = qp.d;
  QBlockItem it;
  if (!qblock_item(qp, it)) return;   // uniform over the workgroup
  // the wave index is uniform over the wave: kept in a scalar register, so that everything
  // derived from it (the wave's tokens, key range and tile checks) is scalar too
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int h = lane >> 5;            // lane half
  const int c = lane & 31;            // this lane's row of the wave
  const int tpb = qp.tokens_per_block;
  const int g = p.group;
  const int64_t cap = (int64_t)p.stride << p.bs_log2;
  const int Lraw = __builtin_amdgcn_readfirstlane(p.seq_lens[it.b]);
  // the workgroup's tokens and the union of their keys, in 16-token tiles
  const int q0w = it.qb * kQbWaves * tpb;
  const int nqw = min(kQbWaves * tpb, p.q_total - q0w);
  SeqSpan sw = seq_span(Lraw, p.window > 0 ? p.window + nqw - 1 : 0, cap,
                        p.q_total - q0w - nqw);
  clip_to_split(qp, it.split, sw);
  const int npairs = (sw.T + 1) >> 1;
  // this wave's tokens (none past the last block) and their keys
  const int q0 = q0w + wave * tpb;
  const int nq = max(0, min(tpb, p.q_total - q0));
  const bool active = nq > 0;
  const SeqSpan s = seq_span(Lraw, p.window > 0 ? p.window + nq - 1 : 0, cap,
                             max(0, p.q_total - q0 - nq));
  // this lane's row: token q0 + c / g, head kvh * g + c % g, at position pos; padding rows
  // (token past q_total) have zero q, and their results are not written
  const int sh = __builtin_ctz((unsigned)g);
  const int tok = q0 + (c >> sh);
  const bool row_ok = active && (c >> sh) < nq;
  const int pos = s.L - nq + (c >> sh);
  const int lo_row = p.window > 0 ? max(pos + 1 - p.window, 0) : 0;
  const int hq = it.kvh * g + (c & (g - 1));

  // q rows as B operands of the score MFMAs: dims 16 ks + 8 h .. + 8 of row c
  const float c2 = fabsf(p.qk_scale_log2);
  // the scale as applied to the scores: at least the smallest normal float, so that a masked
  // (-inf) score stays -inf under it; with a zero scale every p is exp2 of a number below
  // 1e-34 in magnitude, which is 1.0f, as with the scale itself
  const float c2k = fmaxf(c2, 1.17549435e-38f);
  const uint32_t qflip = p.qk_scale_log2 < 0.f ? 0x80008000u : 0u;
  u32x4_t qb[F::KS];
  {
    const uint32_t keep = row_ok ? 0xFFFFFFFFu : 0u;
    const char* qrow = reinterpret_cast<const char*>(
        p.q + (((size_t)it.b * p.q_total + (row_ok ? tok : 0)) * p.num_q_heads + hq) * D);
#pragma unroll
    for (int ks = 0; ks < F::KS; ++ks) {
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(qrow + 32 * ks + 16 * h);
      x.x = (x.x ^ qflip) & keep;
      x.y = (x.y ^ qflip) & keep;
      x.z = (x.z ^ qflip) & keep;
      x.w = (x.w ^ qflip) & keep;
      qb[ks] = x;
    }
  }
  f32x16_t o[F::E];
#pragma unroll
  for (int e = 0; e < F::E; ++e)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[e][v] = 0.f;
  float m = -INFINITY, l = 0.f;

  const TileAddr ta{p.num_blocks, p.bs_log2, p.kv_block_stride, it.kvh * p.kv_head_stride,
                    p.kv_row_stride};
  const int rs = (int)p.kv_row_stride;
  const int32_t* bt = p.block_table + (size_t)it.b * p.stride;
  bool bad = sw.bad;
  // a 16-token tile that is past the range or has a bad table entry is copied from the first
  // rows of block 0 instead (valid memory under the same per-lane offsets; never used unmasked)
  const int64_t fallback = ta.offset(0, 0);

  // per copy m of a tile: the lane's offset inside its 16-token tile, and which K/V half and
  // 16-row half of the tile it fills (both uniform over the wave)
  uint32_t cp_off[PL];
  int cp_hk[PL], cp_hf[PL];
#pragma unroll
  for (int mcp = 0; mcp < PL; ++mcp) {
    const int piece = (mcp * kQbWaves + wave) * kWave + lane;   // its place in the tile copy
    const int hk = piece / (F::kKeys * F::PR);                   // 0 K, 1 V
    const int row = (piece / F::PR) % F::kKeys;
    const int col = (piece % F::PR) ^ F::swz(hk, row);           // the pool's piece
    cp_off[mcp] = (uint32_t)((row & 15) * rs + col * 16);
    cp_hk[mcp] = __builtin_amdgcn_readfirstlane(hk);
    cp_hf[mcp] = __builtin_amdgcn_readfirstlane(row >> 4);
  }

  // byte offsets of the workgroup's 16-token tiles [base, base + kQbTableTiles) in the pool, in
  // LDS: past the range, the fallback; a table entry outside the pool, -1
  auto fill_table = [&](int base) {
    const int k = base + (int)threadIdx.x;
    s_off[threadIdx.x] =
        k < sw.T ? ta.offset(bt[ta.logical_block(sw.t0 + k)], sw.t0 + k) : fallback;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  fill_table(0);

  // copy 32-key tile k (16-token tiles sw.t0 + 2k, + 1) into ring slot k % NBUF
  uint32_t badbits = 0;   // bit 2 (k % NBUF) + half: that half's table entry is outside the pool
  auto copy = [&](int k, int slot) {
    int64_t off[2];
    uint32_t bits = 0;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int64_t o16 = s_off[(2 * k + hf) % kQbTableTiles];
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)o16);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)o16 >> 32));
      off[hf] = (int64_t)(((uint64_t)hi << 32) | lo);
      bits |= (off[hf] < 0 ? 1u : 0u) << hf;
      if (off[hf] < 0) off[hf] = fallback;
    }
    badbits = (badbits & ~(3u << (2 * slot))) | (bits << (2 * slot));
#pragma unroll
    for (int mcp = 0; mcp < PL; ++mcp) {
      const char* base = (cp_hk[mcp] ? p.v_cache : p.k_cache) + off[cp_hf[mcp]];
      copy_piece_to_lds_s(base, cp_off[mcp],
                          s_tiles + slot * F::TB + (mcp * kQbWaves + wave) * kWave * 16);
    }
  };

  // every row of this wave sees the keys in [lo_all, hi_all); keys from t_end on lie past the
  // workgroup's range (its key split's end, or the half tile after its last tile)
  const int hi_all = s.L - nq + 1;
  const int lo_all = (p.window > 0 && s.L > p.window) ? s.L - p.window : 0;
  const int t_end = (sw.t0 + sw.T) * kTileTokens;
  // keys in [z_lo, z_hi) are rows some token of the workgroup attends: real cache rows.  Rows
  // outside (before the window, past the sequence, past the range or from the fallback copy)
  // may hold anything and are zeroed before P.V, in the tiles that reach them: a stray NaN there
  // must not meet p = 0
  const int z_lo = sw.start;
  const int z_hi = min(sw.L, t_end);
  // LDS addresses of this lane's reads.  The score operand of step ks is K row c, piece
  // (2 ks + h) ^ (c % PR), at k_lane ^ 32 ks.  The P.V operand of MFMA e (head dims 32 e ..
  // 32 e + 31) comes from two transposing reads (ds_read_b64_tr_b16): within each 16-lane
  // group, lane L reads the 8 bytes of key row k0 + L / 4 at dims 32 e + 16 g + 4 (L % 4)
  // (g = bit 4 of the lane), and lane j of the group receives dim 32 e + 16 g + j of key rows
  // k0 .. k0 + 3, k0 = 4 h and 8 + 4 h of each 16-key half: exactly row l % 32 of V^T for the
  // keys whose probabilities the lane holds
  const uint32_t k_lane = (uint32_t)(c * F::RB + ((h ^ (c & (F::PR - 1))) << 4));
  uint32_t vt_lane[F::E];
  {
    const int L = lane & 15, gq = (lane >> 4) & 1;
#pragma unroll
    for (int e = 0; e < F::E; ++e) {
      const int piece = (4 * e + 2 * gq + ((L & 3) >> 1)) ^ F::swz(1, 4 * h);
      vt_lane[e] = (uint32_t)((F::kKeys + 4 * h + (L >> 2)) * F::RB + (piece << 4) + 8 * (L & 1));
    }
  }
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(s_tiles);

  // P^T operands (p = hi + lo in bf16) of the tile whose P.V is still to be issued
  u32x4_t pv_hi[2], pv_lo[2];
  // V^T operands of both 16-key halves of the tile at LDS address TILE (transposing LDS reads)
  auto read_vt = [&](uint32_t tile, u32x4_t (&vt)[2][F::E]) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int e = 0; e < F::E; ++e) {
        const uint32_t at = tile + vt_lane[e] + 16 * half * F::RB;
        const s16x4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(uintptr_t)at);
        const s16x4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(uintptr_t)(at + 8 * F::RB));
        const u32x2_t w0 = __builtin_bit_cast(u32x2_t, r0), w1 = __builtin_bit_cast(u32x2_t, r1);
        vt[half][e] = u32x4_t{w0.x, w0.y, w1.x, w1.y};
      }
    }
  };
  // O^T += V^T P^T for the tile whose first key is TOK0
  auto pv_mma = [&](u32x4_t (&vt)[2][F::E], int tok0) {
    if (__builtin_amdgcn_readfirstlane((tok0 < z_lo || tok0 + F::kKeys > z_hi) ? 1 : 0)) {
      // operand value j of a half is key 16 half + fa_key(j, h): keep it where that key is
      // one some token attends (two bf16 values per word)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t keep[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int t0 = tok0 + 16 * half + fa_key(2 * w, h);
          const int t1 = tok0 + 16 * half + fa_key(2 * w + 1, h);
          keep[w] = (t0 >= z_lo && t0 < z_hi ? 0x0000FFFFu : 0u) |
                    (t1 >= z_lo && t1 < z_hi ? 0xFFFF0000u : 0u);
        }
#pragma unroll
        for (int e = 0; e < F::E; ++e) {
          vt[half][e].x &= keep[0];
          vt[half][e].y &= keep[1];
          vt[half][e].z &= keep[2];
          vt[half][e].w &= keep[3];
        }
      }
    }
    // O^T += V^T P^T, one 16-key half at a time
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int e = 0; e < F::E; ++e) {
        o[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vt[half][e]),
                                                       __builtin_bit_cast(bf16x8_t, pv_hi[half]),
                                                       o[e], 0, 0, 0);
        if constexpr (HILO)
          o[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, vt[half][e]),
              __builtin_bit_cast(bf16x8_t, pv_lo[half]), o[e], 0, 0, 0);
      }
    }
  };
  // With P.V a step late, the tile waiting for it is issued behind the next tile's score MFMAs,
  // so that the matrix cores work through it while the vector ALUs run that tile's softmax.
  // Its V^T operands are read again from its ring slot then (still resident: the copies in
  // flight go to other slots), so only its P operands wait in registers.
  bool pv_have = false;
  int pv_tok0 = 0;
  auto flush_pv = [&](auto slot_c) {   // the tile waiting for its P.V sits in slot SLOT
    constexpr int SLOT = decltype(slot_c)::value;
    if (!pv_have) return;   // uniform
    pv_have = false;
    u32x4_t vt[2][F::E];
    read_vt(lds0 + SLOT * F::TB, vt);
    pv_mma(vt, pv_tok0);
  };

  // fold tile k, which sits in ring slot SLOT, into this wave's rows
  auto step = [&](int k, auto slot_c) {
    constexpr int SLOT = decltype(slot_c)::value;
    const auto prev = std::integral_constant<int, (SLOT + NBUF - 1) % NBUF>{};   // tile k - 1
    // this wave's copies of tile k are done once at most those of the A - 1 later tiles are
    // outstanding; the barrier then makes the whole tile visible, and every wave has finished
    // reading the tile whose slot the next copy reuses (tile k - 1; k - 2 with P.V a step late,
    // its V read again then)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(PL * (A - 1)) : "memory");
    if ((k + A) % kTablePairs == 0 && k + A < npairs) fill_table(2 * (k + A));   // uniform
    copy(k + A, (SLOT + A) % NBUF);
    const int tok0 = (sw.t0 + 2 * k) * kTileTokens;
    // whether this wave folds tile k (uniform per wave): its keys reach the wave's range, and
    // no table entry outside the pool lies among them (never read through: NaN outputs)
    bool fold = active && tok0 + F::kKeys > s.start && tok0 < s.L;
    const uint32_t tb = badbits >> (2 * SLOT);
    if (fold && (((tb & 1u) && tok0 + kTileTokens > s.start) ||
                 ((tb & 2u) && tok0 + kTileTokens < s.L))) {
      bad = true;
      fold = false;
    }
    const uint32_t tile = lds0 + SLOT * F::TB;
    f32x16_t sc;
    if (fold) {
      // scores S^T: 32 keys x 32 rows; every K read is issued before the first MFMA that waits
      u32x4_t kw[F::KS];
#pragma unroll
      for (int ks = 0; ks < F::KS; ++ks)
        kw[ks] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
            (uintptr_t)(tile + (k_lane ^ (32u * ks))));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < F::KS; ++ks)
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kw[ks]),
                                                     __builtin_bit_cast(bf16x8_t, qb[ks]), sc, 0,
                                                     0, 0);
    }
    u32x4_t vt[2][F::E];
    if constexpr (DEFER)
      flush_pv(prev);   // the previous tile's P.V, behind these score MFMAs
    else if (fold)
      read_vt(tile, vt);   // this tile's V^T operands go out now, under the softmax
    __builtin_amdgcn_sched_barrier(0);
    if (!fold) return;
    const int full = __builtin_amdgcn_readfirstlane(
        (tok0 >= lo_all && tok0 + F::kKeys <= min(hi_all, t_end)) ? 1 : 0);
    // one path: only the masking of keys outside the row's range is conditional (separate
    // masked and unmasked paths made the compiler copy the scores between them); the score
    // scale is applied inside the exponent's FMA, and c2k >= FLT_MIN keeps -inf * c2k = -inf
    if (!full) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = tok0 + fa_key(v, h);
        sc[v] = (key >= lo_row && key <= pos && key < t_end) ? sc[v] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[v]);
    mx *= c2k;
    mx = halves_max(mx);   // the row's other 16 keys
    if (__builtin_amdgcn_ballot_w64(row_ok && mx > m + kRescaleSlack) != 0) {
      const float mn = fmaxf(m, mx);
      const float alpha = fast_exp2(m - (mn == -INFINITY ? 0.f : mn));
      l *= alpha;
      m = mn;
#pragma unroll
      for (int e = 0; e < F::E; ++e)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[e][v] *= alpha;
    }
    const float mu = m == -INFINITY ? 0.f : m;
    float pr[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) pr[v] = fast_exp2(fmaf(sc[v], c2k, -mu));
    float ls = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) ls += pr[v];
    l += ls;
    // P^T as B operands, p = hi + lo in bf16, eight keys per 16-key half of the tile
    auto& bhi = pv_hi;
    auto& blo = pv_lo;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // hi: the upper halves of the two floats (p truncated to bf16, one byte permute); lo:
        // the exact remainder p - hi, rounded to bf16: |hi + lo - p| <= 2^-16 |p|.  With one
        // term, p rounded to the nearest bf16 instead: |hi - p| <= 2^-8 |p|
        const float a0 = pr[8 * half + 2 * w], a1 = pr[8 * half + 2 * w + 1];
        const uint32_t u0 = __builtin_bit_cast(uint32_t, a0);
        const uint32_t u1 = __builtin_bit_cast(uint32_t, a1);
        if constexpr (HILO) {
          bhi[half][w] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
        } else {
          const bf16x2_t hv = {(__bf16)a0, (__bf16)a1};
          bhi[half][w] = __builtin_bit_cast(uint32_t, hv);
        }
        if constexpr (HILO) {
          const bf16x2_t lv = {(__bf16)(a0 - __builtin_bit_cast(float, u0 & 0xFFFF0000u)),
                               (__bf16)(a1 - __builtin_bit_cast(float, u1 & 0xFFFF0000u))};
          blo[half][w] = __builtin_bit_cast(uint32_t, lv);
        }
      }
    }
    if constexpr (DEFER) {
      pv_have = true;
      pv_tok0 = tok0;
    } else {
      pv_mma(vt, tok0);
    }
  };

#pragma unroll
  for (int k = 0; k < A; ++k) copy(k, k);
  // the ring slot of tile k is k % NBUF: unrolled NBUF times, so that every LDS address is a
  // lane register plus a constant
  for (int k = 0; k < npairs; k += NBUF) {
    step(k, std::integral_constant<int, 0>{});
    if (k + 1 < npairs) step(k + 1, std::integral_constant<int, 1>{});
    if (k + 2 < npairs) step(k + 2, std::integral_constant<int, 2>{});
    if (k + 3 < npairs) step(k + 3, std::integral_constant<int, 3>{});
  }
  static_assert(NBUF == 4, "the loop above is unrolled for a ring of four");
  // the last tile's P.V, a step late: it sat in slot (npairs - 1) % NBUF
  if constexpr (DEFER) switch ((npairs - 1) & 3) {
    case 0: flush_pv(std::integral_constant<int, 0>{}); break;
    case 1: flush_pv(std::integral_constant<int, 1>{}); break;
    case 2: flush_pv(std::integral_constant<int, 2>{}); break;
    default: flush_pv(std::integral_constant<int, 3>{}); break;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the copies past the last tile
  if (!active) return;
  bad = bad || s.bad;

  // finish: the row's sum over both halves, the sink (one split), normalise, write
  const float lt = halves_sum(l);
  if (!row_ok) return;
  float M = m, L2 = lt, scale_o = 1.f;
  if (p.sinks != nullptr && qp.splits == 1) {
    const float s2 = p.sinks[hq] * kLog2e;
    const float M2 = fmaxf(M, s2);
    const float M2u = M2 == -INFINITY ? 0.f : M2;
    scale_o = fast_exp2(M - M2u);
    L2 = fmaf(L2, scale_o, fast_exp2(s2 - M2u));
    M = M2;
  }
  const float inv = L2 != 0.f ? scale_o / L2 : 0.f;
  float lv = L2 != 0.f ? (M + fast_log2(L2)) * kLn2 : -INFINITY;
  if (bad) lv = __builtin_nanf("");
  const size_t row = ((size_t)it.b * p.q_total + tok) * p.num_q_heads + hq;
  float* dst;
  if (qp.splits == 1) {
    dst = p.out + row * D;
    if (h == 0 && p.lse != nullptr) p.lse[row] = lv;
  } else {
    const size_t slot = row * (size_t)qp.splits + it.split;
    dst = qp.part_out + slot * D;
    if (h == 0) qp.part_lse[slot] = lv;
  }
  // o[e][v] is head dim 32 e + fa_key(v, h): four consecutive dims per group of four v
#pragma unroll
  for (int e = 0; e < F::E; ++e) {
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      float4 x;
      x.x = bad ? __builtin_nanf("") : o[e][4 * v4 + 0] * inv;
      x.y = bad ? __builtin_nanf("") : o[e][4 * v4 + 1] * inv;
      x.z = bad ? __builtin_nanf("") : o[e][4 * v4 + 2] * inv;
      x.w = bad ? __builtin_nanf("") : o[e][4 * v4 + 3] * inv;
      *reinterpret_cast<float4*>(dst + 32 * e + fa_key(4 * v4, h)) = x;
    }
  }
}

// Merge of the key splits: one wave per output row (sequence, token, query head).  Over the
// splits with a finite LSE l_k: M = max l_k, w_k = e^(l_k - M), out = sum w_k o_k / sum w_k and
// lse = M + ln sum w_k, the log-sum-exp rule of split-KV decode (ROCm/rocm-libraries PR #13700,
// the reducer's output and LSE arguments); the sink logit, when given, joins M and the
// denominator with a zero output row.  A NaN partial LSE (a bad length or table entry, a NaN key)
// makes the row NaN; a row with no keys and no sink gets out 0, lse -inf.
constexpr int kMergeRows = 4;   // rows (waves) per workgroup

template <int D>
__global__ __launch_bounds__(kMergeRows * kWave) void qblock_merge_kernel(const QBlockParams qp) {
  constexpr int E = D / kWave;   // contiguous floats per lane: 1, 2 or 4
  const DecodeParams& p = qp.d;
  const size_t rows = (size_t)p.num_seqs * p.q_total * p.num_q_heads;
  const size_t row = (size_t)blockIdx.x * kMergeRows +
                     (size_t)__builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (row >= rows) return;
  const int lane = threadIdx.x % kWave;
  const int S = qp.splits;
  const float* lp = qp.part_lse + row * S;
  const float* op = qp.part_out + row * S * D + lane * E;
  float m = -INFINITY, den = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  bool nan = false;
#pragma unroll 4
  for (int k = 0; k < S; ++k) {
    const float l = lp[k] * kLog2e;
    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = op[(size_t)k * D + e];
    nan = nan || l != l;
    if (l > -INFINITY) {   // false for NaN and for an empty split
      const float mn = fmaxf(m, l);
      const float a = fast_exp2(m - mn), w = fast_exp2(l - mn);
      den = fmaf(den, a, w);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(acc[e], a, w * o[e]);
      m = mn;
    }
  }
  if (p.sinks != nullptr) {
    const float s2 = p.sinks[row % p.num_q_heads] * kLog2e;
    const float M2 = fmaxf(m, s2);
    const float M2u = M2 == -INFINITY ? 0.f : M2;
    const float a = fast_exp2(m - M2u);
    den = fmaf(den, a, fast_exp2(s2 - M2u));
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= a;
    m = M2;
  }
  const float inv = den != 0.f ? 1.f / den : 0.f;
  float lv = den != 0.f ? (m + fast_log2(den)) * kLn2 : -INFINITY;
  if (nan) lv = __builtin_nanf("");
  if (lane == 0 && p.lse != nullptr) p.lse[row] = lv;
  float* dst = p.out + row * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) dst[e] = nan ? __builtin_nanf("") : acc[e] * inv;
}

template <int D>
using QbQk = typename std::conditional<D <= 128, QkMfmaPvPair<D, false, false>,
                                       QkMfmaPvT<D, 16, false, false>>::type;
template <int D>
using QbQkFp8 = typename std::conditional<D <= 128, QkMfmaPvPair<D, true, false>,
                                          QkMfmaPvT<D, 16, true, false>>::type;

// One wave per block: one tile in flight and at least two waves per SIMD.  The keys mostly come
// from L2 here, and a second wave hides the tile step's latency better than a second tile buffer
// (which leaves room for one wave only).  Measured on the Llama-8B-shaped batch with 512 new
// tokens per sequence: 3555 us per step against 6044 us for two tiles in flight at one wave per
// SIMD; two tiles at two waves spill registers (9278 us).  The workgroup form: 3068 us.
template <int D>
hipError_t launch_d(const QBlockParams& qp, QkPath path, hipStream_t stream) {
  constexpr int DEPTH = 1, WPE = 2;
  constexpr int A = D == 256 ? 3 : 4;   // tiles copied ahead (LDS ring of A + 1; 4, 6 and 8
                                        // measured the same at D = 128)
  if (qp.waves == kQbWaves) {
    if (path == QkPath::kMfmaPvFp8)
      hipLaunchKernelGGL((qblock_lds_kernel<D, QbQkFp8<D>, A>), dim3(qp.grid),
                         dim3(kQbWaves * kWave), 0, stream, qp);
    else if constexpr (D <= 128) {
      if (qp.p_one_term)
        hipLaunchKernelGGL((qblock_fa_kernel<D, false, fa_ahead<D>()>), dim3(qp.grid),
                           dim3(kQbWaves * kWave), 0, stream, qp);
      else
        hipLaunchKernelGGL((qblock_fa_kernel<D, true, fa_ahead<D>()>), dim3(qp.grid),
                           dim3(kQbWaves * kWave), 0, stream, qp);
    }
    else
      hipLaunchKernelGGL((qblock_lds_kernel<D, QbQk<D>, A>), dim3(qp.grid),
                         dim3(kQbWaves * kWave), 0, stream, qp);
    return hipGetLastError();
  }
  if (path == QkPath::kMfmaPvFp8)
    hipLaunchKernelGGL((qblock_kernel<D, QbQkFp8<D>, DEPTH, WPE>), dim3(qp.grid), dim3(kWave), 0,
                       stream, qp);
  else
    hipLaunchKernelGGL((qblock_kernel<D, QbQk<D>, DEPTH, WPE>), dim3(qp.grid), dim3(kWave), 0,
                       stream, qp);
  return hipGetLastError();
}

template <int D>
hipError_t launch_merge(const QBlockParams& qp, hipStream_t stream) {
  const size_t rows = (size_t)qp.d.num_seqs * qp.d.q_total * qp.d.num_q_heads;
  const size_t grid = (rows + kMergeRows - 1) / kMergeRows;
  hipLaunchKernelGGL((qblock_merge_kernel<D>), dim3((uint32_t)grid), dim3(kMergeRows * kWave), 0,
                     stream, qp);
  return hipGetLastError();
}

}  // namespace

int qblock_columns(int head_dim) { return head_dim <= 128 ? 32 : 16; }

void qblock_geometry(QBlockParams& qp, int head_dim, int max_seq_len) {
  const int cols = qblock_columns(head_dim);
  qp.tokens_per_block = cols / qp.d.group;
  // the workgroup form once there are blocks for all its waves; one wave per block otherwise
  const int blocks = (qp.d.q_total + qp.tokens_per_block - 1) / qp.tokens_per_block;
  qp.waves = blocks >= kQbWaves ? kQbWaves : 1;
  const int per_wg = qp.tokens_per_block * qp.waves;
  qp.blocks_per_seq = (qp.d.q_total + per_wg - 1) / per_wg;
  const long long units = (long long)qp.d.num_seqs * qp.d.num_kv_heads;
  qp.xcd_pinned = units % kXcds == 0 ? 1 : 0;
  // Key splits: with few workgroups (small batches) each one's key range is cut into up to
  // kQbMaxSplits splits of at least kQbMinSplitTiles tiles, so that about kQbTargetWaves waves
  // run; a merge then combines each row's partials.  Sized from the longest range a workgroup
  // can attend (the length bound, within the window plus its tokens); a longer range only makes
  // the last split longer.
  qp.splits = 1;
  qp.split_tiles = 0;
  const long long waves_now = units * qp.blocks_per_seq * qp.waves;
  if (max_seq_len > 0 && waves_now > 0 && waves_now < kQbTargetWaves) {
    long long keys = max_seq_len;
    if (qp.d.window > 0) keys = std::min(keys, (long long)qp.d.window + per_wg - 1);
    const long long tiles = (keys + kTileTokens - 1) / kTileTokens + 1;   // one straddled tile
    long long want = (kQbTargetWaves + waves_now - 1) / waves_now;
    want = std::min(want, std::min(tiles / kQbMinSplitTiles, (long long)kQbMaxSplits));
    if (want > 1) {
      qp.split_tiles = (int)((tiles + want - 1) / want);
      qp.splits = (int)((tiles + qp.split_tiles - 1) / qp.split_tiles);
    }
  }
  const long long per_unit = (long long)qp.blocks_per_seq * qp.splits;
  const long long grid = qp.xcd_pinned ? (units / kXcds) * kXcds * per_unit : units * per_unit;
  qp.grid = (uint32_t)grid;
}

hipError_t launch_qblock(const QBlockParams& qp, int head_dim, QkPath path, hipStream_t stream) {
  if (qp.grid == 0) return hipSuccess;
  switch (head_dim) {
    case 64: return launch_d<64>(qp, path, stream);
    case 128: return launch_d<128>(qp, path, stream);
    case 256: return launch_d<256>(qp, path, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_qblock_merge(const QBlockParams& qp, int head_dim, hipStream_t stream) {
  if (qp.grid == 0 || qp.splits == 1) return hipSuccess;
  switch (head_dim) {
    case 64: return launch_merge<64>(qp, stream);
    case 128: return launch_merge<128>(qp, stream);
    default: return launch_merge<256>(qp, stream);
  }
}

}  // namespace pa
