// Balanced split-KV decode for gfx950: persistent one-wave workers over the flattened tile
// sequence, then a fix-up merge.
//
// The split-KV method (partitions of a sequence's KV each emit a partial output plus a
// log-sum-exp; a second kernel merges them) with the partition boundaries placed where the work
// balances instead of at fixed token offsets.  Every (sequence b, KV head kvh) is a unit of
// T_b 16-token tiles (its attended range); units are laid end to end in (b, kvh) order, and
// worker w of N takes the contiguous tiles [A(w), A(w+1)), A(w) = floor(w * T_total / N).  A
// worker streams its tiles with the loads of the next tile in flight, and at every unit boundary
// inside its range flushes the unit's piece: a unit that starts and ends inside one worker is
// final and written to the output directly (sink folded, normalised); a unit cut by a range
// boundary leaves one partial per worker that holds part of it (at most two per worker: the
// first and the last unit it touches), and the fix-up kernel merges them with the
// log-sum-exp rule.
//
// With several query tokens per sequence (q_len > 1) a unit's tiles span the union of the
// tokens' key ranges, G counts (token, head) columns, and every column keeps its own causal
// range inside the shared tiles.
//
// All workers finish within about one tile of each other, no workgroup is launched per unit, and
// the partial traffic is at most 2 * N * G * (D + 1) floats.  Measured on MI355X for a
// 64-sequence, 512..4096-token Llama-8B-shaped step: fixed-partition grids left a quarter of the
// workgroup slots idle and a long tail; persistent workers over the same tiles stream at the
// rate of a plain gather.
//
// Sources: one-token split-KV decode with partial outputs + LSE merged by a reduce step,
// ROCm/rocm-libraries PR #13700 "prepare saved paged decode bindings once", Summary and review
// finding N1 (the reducer takes the output, the sequence lengths and the LSE buffer); the tile
// math as in pa_qk.hpp; sliding window and attention sinks, randomvariable/vllm issue #23, table
// "Current state".
#include <cstdio>
#include <type_traits>

#include "pa_device.hpp"
#include "pa_kernels.hpp"
#include "pa_qk.hpp"

namespace pa {

// A worker gets at least this many tiles (fewer workers for tiny batches).
constexpr int kMinTilesPerWorker = 4;

// Window that decides a unit's tiles: with q_len query tokens the union of their windows is
// window + q_len - 1 keys ending at the last position (0 = no window).  The host keeps the sum
// in range.
__device__ __forceinline__ int span_window(const DecodeParams& p, const QShape& qs) {
  return p.window > 0 ? p.window + qs.q_len - 1 : 0;
}

// Query tokens of the sequence after this launch's last one.
__device__ __forceinline__ int q_rest(const QShape& qs) {
  return qs.q_total - qs.q_first - qs.q_len;
}

// Workers actually used for T_total tiles, out of at most n.
__device__ __forceinline__ int effective_workers(int64_t total, int n) {
  const int64_t want = (total + kMinTilesPerWorker - 1) / kMinTilesPerWorker;
  return (int)(want < 1 ? 1 : (want < n ? want : n));
}

// First tile of worker w: floor(w * total / n), evaluated as w*q + (w*r)/n with
// total = q*n + r so that no product overflows (w < n <= 2^20).
__device__ __forceinline__ int64_t worker_begin(int64_t total, int n, int w) {
  const int64_t q = total / n, r = total - q * n;
  return (int64_t)w * q + ((int64_t)w * r) / n;
}

// The worker whose range holds tile x (0 <= x < total): the largest w with
// floor(w * total / n) <= x, i.e. ceil((x + 1) * n / total) - 1.  Exact in 64 bits while
// total * n < 2^63 (2^43 tiles at the 2^20-worker limit).
__device__ __forceinline__ int worker_of(int64_t total, int n, int64_t x) {
  return (int)(((x + 1) * n + total - 1) / total) - 1;
}

__device__ __forceinline__ int64_t shfl_up64(int64_t x, int off, int lane) {
  const int src = (lane >= off ? lane - off : lane) << 2;
  const int lo = __builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)x);
  const int hi = __builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)((uint64_t)x >> 32));
  const int64_t y = (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
  return lane >= off ? y : 0;
}

__device__ __forceinline__ int64_t wave_incl_scan64(int64_t x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) x += shfl_up64(x, off, lane);
  return x;
}

__device__ __forceinline__ int64_t readlane64(int64_t x, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)x >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Position in the flattened tile sequence: unit (b, kvh), tile ti of the unit, and the span of
// sequence b.  All fields are wave-uniform.
struct Cursor {
  int b, kvh, ti;
  SeqSpan s;
};

// A wave-uniform read of a kernel-constant int32 array through the scalar data cache (a scalar
// load, counted apart from the vector loads): waiting for it does not wait for the K/V loads in
// flight, as a vector load's would (vector loads complete in order).  Reads only.
__device__ __forceinline__ int32_t scalar_read(const int32_t* base, size_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)(uintptr_t)base)[i];
}

struct BalancedCtx {
  const DecodeParams* p;
  int64_t cap;
  int swin, qrest;   // span_window and q_rest of the launch
  __device__ __forceinline__ SeqSpan span(int b) const {
    return seq_span(scalar_read(p->seq_lens, b), swin, cap, qrest);
  }
  // next tile; skips sequences without tiles (callers never step past the last tile)
  __device__ __forceinline__ void advance(Cursor& c) const {
    if (++c.ti < c.s.T) return;
    c.ti = 0;
    if (++c.kvh < p->num_kv_heads) return;
    c.kvh = 0;
    do {
      ++c.b;
      c.s = span(c.b);
    } while (c.s.T == 0 && c.b + 1 < p->num_seqs);
  }
  // physical block of the cursor's tile
  __device__ __forceinline__ int phys(const Cursor& c) const {
    const int tile = c.s.t0 + c.ti;
    return scalar_read(p->block_table,
                       (size_t)c.b * p->stride + ((tile * kTileTokens) >> p->bs_log2));
  }
};

// Worker w's share of the flattened tiles: n tiles from the tile under `cur`.  Pass 1 totals
// the tiles (worker 0 also records the per-sequence prefix the fix-up reads, when `prefix` is
// given); the first 64 sequences' tiles and inclusive prefix stay in registers for pass 2, which
// finds the unit holding the worker's first tile (with up to 64 sequences nothing is loaded
// again).  False when the worker has no tiles.
__device__ __forceinline__ bool worker_share(const DecodeParams& p, const BalancedCtx& ctx,
                                             int num_workers, int w, int lane, int64_t* prefix,
                                             int& n, Cursor& cur) {
  int64_t carry = 0, T_first = 0, incl_first = 0;
  for (int base = 0; base < p.num_seqs; base += kWave) {
    const int j = base + lane;
    const int64_t T =
        j < p.num_seqs ? seq_span(p.seq_lens[j], ctx.swin, ctx.cap, ctx.qrest).T : 0;
    const int64_t incl = wave_incl_scan64(T, lane) + carry;
    if (base == 0) {
      T_first = T;
      incl_first = incl;
    }
    if (prefix != nullptr && w == 0 && j < p.num_seqs) prefix[j] = incl - T;
    carry = readlane64(incl, kWave - 1);
  }
  if (prefix != nullptr && w == 0 && lane == 0) prefix[p.num_seqs] = carry;
  const int64_t total = carry * p.num_kv_heads;
  const int n_eff = effective_workers(total, num_workers);
  if (w >= n_eff) return false;
  const int64_t A = worker_begin(total, n_eff, w);
  n = (int)(worker_begin(total, n_eff, w + 1) - A);
  if (n <= 0) return false;

  cur = Cursor{0, 0, 0, {}};
  carry = 0;
  for (int base = 0; base < p.num_seqs; base += kWave) {
    const int j = base + lane;
    int64_t T = T_first, incl = incl_first;
    if (base != 0) {
      T = j < p.num_seqs ? seq_span(p.seq_lens[j], ctx.swin, ctx.cap, ctx.qrest).T : 0;
      incl = wave_incl_scan64(T, lane) + carry;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(j < p.num_seqs &&
                                                     incl * p.num_kv_heads > A);
    if (hit != 0) {
      const int f = __builtin_ctzll(hit);
      const int64_t P = readlane64(incl, f) - readlane64(T, f);
      const int64_t Tb = readlane64(T, f);
      const int64_t off = A - P * p.num_kv_heads;   // tiles into sequence base + f
      cur.b = base + f;
      cur.s = ctx.span(cur.b);
      cur.kvh = (int)(off / Tb);
      cur.ti = (int)(off - (int64_t)cur.kvh * Tb);
      break;
    }
    carry = readlane64(incl, kWave - 1);
  }
  return true;
}

// The issue side of a worker's walk: the cursor of the next tile to load, with its block-table
// entry fetched one issue ahead.  It only advances while another tile of the worker follows, so
// it never walks past the last sequence that has tiles.
struct IssueWalk {
  Cursor iss;
  int phys_next;
  __device__ __forceinline__ IssueWalk(const BalancedCtx& ctx, const Cursor& first)
      : iss(first), phys_next(ctx.phys(first)) {}
  // tile k of n: its cursor and the byte offset of its first K/V row (-1 for a table entry
  // outside the pool, which must not be read)
  __device__ __forceinline__ int64_t next(const BalancedCtx& ctx, int k, int n, Cursor& at) {
    const DecodeParams& p = *ctx.p;
    at = iss;
    const int phys = phys_next;
    if (k + 1 < n) {
      ctx.advance(iss);
      phys_next = ctx.phys(iss);
    }
    const TileAddr ta{p.num_blocks, p.bs_log2, p.kv_block_stride, at.kvh * p.kv_head_stride,
                      p.kv_row_stride};
    return ta.offset(phys, at.s.t0 + at.ti);
  }
};

// MULTI: the launch may have several query tokens (reads q_len, q_total, q_first, group);
// otherwise they are the constants of one token, which keeps them out of the scalar registers.
// Tiles in flight: AHEAD = 0, DEPTH tiles held in registers (the loads of tile k + DEPTH - 1
// issued before tile k is consumed); AHEAD > 0, AHEAD tiles copied ahead into a ring of
// AHEAD + 1 tile slots in LDS by direct-to-LDS loads, which hold no registers while in flight,
// and read from there into the tile registers just before they are consumed.
template <int D, int G, int DEPTH, class QK, bool MULTI, int AHEAD = 0>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(QK::kMinWavesPerEu)))
void balanced_decode_kernel(const BalancedParams bp) {
  using RG = RowGeom<D>;
  constexpr int E = RG::kElems;
  const DecodeParams& p = bp.d;
  const QShape qs = make_qshape<MULTI, G>(p);
  const int lane = threadIdx.x;
  const int c = lane & (kRowLanes - 1);
  const int w = blockIdx.x;
  const BalancedCtx ctx{&p, (int64_t)p.stride << p.bs_log2, span_window(p, qs), q_rest(qs)};
  int n = 0;
  Cursor cur;
  if (!worker_share(p, ctx, bp.num_workers, w, lane, bp.prefix, n, cur)) return;

  const float c2 = fabsf(p.qk_scale_log2);
  const uint32_t qflip = p.qk_scale_log2 < 0.f ? 0x80008000u : 0u;
  QK qk;
  qk.init(p, qs, cur.b, cur.kvh * qs.group, lane, qflip, c2);

  // the issue side walks ahead of the consume side by the tiles in flight; each keeps its own
  // cursor, so a tile in flight carries nothing but its registers and whether it was read
  IssueWalk walk(ctx, cur);
  Cursor con = cur;   // the tile consumed next
  auto issue = [&](int k, typename QK::Tile& t, bool& ok) {
    Cursor at;
    const int64_t off = walk.next(ctx, k, n, at);
    ok = off >= 0;
    if (ok) qk.issue(t, p.k_cache + off, p.v_cache + off, lane);
  };

  int piece_start = cur.ti;
  bool first_piece = true;
  bool piece_bad = false;

  // flush the current piece of unit (at.b, at.kvh), which ends at tile at.ti
  auto flush = [&](const Cursor& at) {
    if constexpr (QK::kColumns) {
      // by columns: lane (r, c) finishes columns cb + 4r + i, i < 4, that exist, of each
      // 16-column half (cb = 0, 16)
      const bool whole = piece_start == 0 && at.ti == at.s.T - 1;
      const int ncols = qs.q_len * qs.group;
      const int sh = __builtin_ctz((unsigned)qs.group);
      auto finish_half = [&](auto& half, int cb) {
        half.merge_cols();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int nl = 4 * (lane >> 4) + i;         // column within the half
          const int n = cb + nl;
          float M = half.col_m(nl), lt = half.col_l(nl);   // every lane takes part in the reads
          if (n < ncols) {
            const int hq = at.kvh * qs.group + (n & (qs.group - 1));
            float scale_o = 1.f;
            if (whole && p.sinks != nullptr) {
              // the sink logit joins the max and the denominator with a zero value row
              const float s2 = p.sinks[hq] * kLog2e;
              const float M2 = fmaxf(M, s2);
              const float M2u = M2 == -INFINITY ? 0.f : M2;
              scale_o = fast_exp2(M - M2u);
              lt = fmaf(lt, scale_o, fast_exp2(s2 - M2u));
              M = M2;
            }
            // lt is 0 only for an empty piece; a NaN input (lt = NaN) must reach the outputs
            const float inv = lt != 0.f ? scale_o / lt : 0.f;
            float lv = lt != 0.f ? (M + fast_log2(lt)) * kLn2 : -INFINITY;
            if (piece_bad) lv = __builtin_nanf("");
            float* dst;
            if (whole) {
              const size_t row =
                  ((size_t)at.b * qs.q_total + qs.q_first + (n >> sh)) * p.num_q_heads + hq;
              dst = p.out + row * D;
              if (c == 0 && p.lse != nullptr) p.lse[row] = lv;
            } else {
              const size_t slot = ((size_t)w * 2 + (first_piece ? 0 : 1)) * G + n;
              dst = bp.ws_o + slot * D;
              if (c == 0) bp.ws_lse[slot] = lv;
            }
#pragma unroll
            for (int e = 0; e < E; ++e)
              dst[RG::dim(c, e)] = piece_bad ? __builtin_nanf("") : half.acc(i, e) * inv;
          }
        }
      };
      if constexpr (QK::kHalves == 2) {
        finish_half(qk.h[0], 0);
        finish_half(qk.h[1], 16);
      } else {
        finish_half(qk, 0);
      }
      first_piece = false;
      piece_bad = false;
      piece_start = 0;
      return;
    } else {
    // by heads, on the lanes of row group 0: column h (query token h / group) for h < G
    float Mh[G], lh[G];
    qk.merge_rows(Mh, lh);
    const bool whole = piece_start == 0 && at.ti == at.s.T - 1;
    const int h0 = at.kvh * qs.group;
    const int ncols = qs.q_len * qs.group;
    const int sh = __builtin_ctz((unsigned)qs.group);
    if (lane < kRowLanes) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (h >= ncols) break;   // padding columns (uniform)
        const int hq = h0 + (h & (qs.group - 1));
        float M = Mh[h], lt = lh[h];
        float scale_o = 1.f;
        if (whole && p.sinks != nullptr) {
          // the sink logit joins the max and the denominator with a zero value row
          const float s2 = p.sinks[hq] * kLog2e;
          const float M2 = fmaxf(M, s2);
          const float M2u = M2 == -INFINITY ? 0.f : M2;
          scale_o = fast_exp2(M - M2u);
          lt = fmaf(lt, scale_o, fast_exp2(s2 - M2u));
          M = M2;
        }
        // lt is 0 only for an empty piece; a NaN input (lt = NaN) must reach the outputs
        const float inv = lt != 0.f ? scale_o / lt : 0.f;
        float lv = lt != 0.f ? (M + fast_log2(lt)) * kLn2 : -INFINITY;
        if (piece_bad) lv = __builtin_nanf("");
        float* dst;
        if (whole) {
          const size_t row =
              ((size_t)at.b * qs.q_total + qs.q_first + (h >> sh)) * p.num_q_heads + hq;
          dst = p.out + row * D;
          if (c == 0 && p.lse != nullptr) p.lse[row] = lv;
        } else {
          const size_t slot = ((size_t)w * 2 + (first_piece ? 0 : 1)) * G + h;
          dst = bp.ws_o + slot * D;
          if (c == 0) bp.ws_lse[slot] = lv;
        }
#pragma unroll
        for (int e = 0; e < E; ++e)
          dst[RG::dim(c, e)] = piece_bad ? __builtin_nanf("") : qk.out(h, e) * inv;
      }
    }
    first_piece = false;
    piece_bad = false;
    piece_start = 0;
    }
  };

  auto consume = [&](int k, typename QK::Tile& t, bool ok) {
    const Cursor& at = con;
    if (ok) {
      const int tok0 = (at.s.t0 + at.ti) * kTileTokens;
      if constexpr (QK::kQueryTokens) {
        // every column sees the keys inside [lo_all, hi_all): from the last query token's
        // window start to the first query token's position (with one token: the attended range)
        const int hi_all = at.s.L - qs.q_len + 1;
        const int lo_all = (p.window > 0 && at.s.L > p.window) ? at.s.L - p.window : 0;
        // each lane's column: its query token's keys, masked only where some column's range
        // ends inside the tile
        qk.consume_cols_flex(t, tok0 >= lo_all && tok0 + kTileTokens <= hi_all, tok0, hi_all,
                             p.window, at.s.start, at.s.L, lane);
      } else {
        if (tok0 >= at.s.start && tok0 + kTileTokens <= at.s.L)
          qk.template consume<false>(t, 0, 0, 0, lane);
        else
          qk.template consume<true>(t, tok0, at.s.start, at.s.L, lane);
      }
    } else {
      piece_bad = true;
    }
    if (at.ti == at.s.T - 1 || k == n - 1) {
      flush(at);
      if (k + 1 < n) {
        // the next tile starts the next unit: its q, fresh state
        ctx.advance(con);
        qk.load_q(p, qs, con.b, con.kvh * qs.group, lane, qflip);
        qk.reset();
      }
    } else {
      ++con.ti;   // the next tile is in the same unit
    }
  };

  if constexpr (AHEAD > 0) {
    // the ring: slot k % NBUF holds tile k (per head of the unit: K rows, then V rows,
    // kRowBytes each, pieces placed as QK::fill_from_lds reads them); copy m of a tile moves
    // pieces 64 m .. 64 m + 63, lane i piece 64 m + i, which is, within its head's part, one
    // half's row (piece / PR) % 16, pool piece (piece % PR) ^ (row & swizzle)
    constexpr int RB = QK::kRowBytes;
    constexpr int PR = RB / 16;
    constexpr int HP = QK::kHeads;
    constexpr int TBH = 2 * kTileTokens * RB;   // one head's part
    constexpr int TB = HP * TBH;
    constexpr int NBUF = AHEAD + 1;
    constexpr int PL = TB / (16 * kWave);
    constexpr int PLH = PL / HP;                // copies per head
    static_assert(PLH * 16 * kWave == TBH && (kTileTokens * PR) % kWave == 0,
                  "a tile half is whole copies");
    __shared__ __attribute__((aligned(16))) char s_tiles[NBUF * TB];
    const int rs = (int)p.kv_row_stride;
    uint32_t voff[PLH];
#pragma unroll
    for (int m = 0; m < PLH; ++m) {
      const int piece = m * kWave + lane;
      const int row = (piece / PR) % kTileTokens;
      voff[m] = (uint32_t)(row * rs + (((piece % PR) ^ (row & QK::kLdsSwizzle)) << 4));
    }
    uint32_t okbits = 0;   // bit k % NBUF: tile k came from the pool
    // copy tile k into its slot; a tile whose table entry lies outside the pool is copied from
    // q instead (valid memory, never read back) so that every tile counts the same copies
    auto copy = [&](int k) {
      Cursor at;
      const int64_t off = walk.next(ctx, k, n, at);
      const int slot = k % NBUF;
      const bool good = off >= 0;
      okbits = (okbits & ~(1u << slot)) | ((good ? 1u : 0u) << slot);
#pragma unroll
      for (int m = 0; m < PL; ++m) {
        const int mh = m % PLH;                                  // constants
        const bool vh = mh * kWave >= kTileTokens * PR;          // the copy's half
        const int64_t ho = m / PLH == 0 ? 0 : p.kv_pair_off;     // the copy's head
        const char* base = good ? (vh ? p.v_cache : p.k_cache) + off + ho
                                : reinterpret_cast<const char*>(p.q);
        copy_piece_to_lds_s<true>(base, good ? voff[mh] : (uint32_t)(lane & 7) * 16,
                                  s_tiles + slot * TB + m * kWave * 16);
      }
    };
#pragma unroll
    for (int j = 0; j < AHEAD; ++j)
      if (j < n) copy(j);
    for (int k = 0; k < n; ++k) {
      // tile k's copies are done once at most those of the AHEAD - 1 later tiles are in flight
      // (vector memory operations complete in order; anything else issued since only makes the
      // wait stricter); near the end fewer follow and everything is waited for.  The slot the
      // next copy fills held tile k - 1, read into registers and consumed before this point.
      if (k + AHEAD - 1 < n)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PL * (AHEAD - 1)) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (k + AHEAD < n) copy(k + AHEAD);
      typename QK::Tile t;
      const bool ok = (okbits >> (k % NBUF)) & 1u;
      if (ok) qk.fill_from_lds(t, s_tiles + (k % NBUF) * TB, lane);
      consume(k, t, ok);
    }
  } else if constexpr (DEPTH > 1) {
    // DEPTH tiles in flight: the loads of tiles k+1 .. k+DEPTH-1 are issued before tile k is
    // consumed; the loop is unrolled DEPTH times so every buffer index is a constant
    typename QK::Tile t[DEPTH];
    bool ok[DEPTH];
#pragma unroll
    for (int j = 0; j + 1 < DEPTH; ++j)
      if (j < n) issue(j, t[j], ok[j]);
    for (int k = 0; k < n; k += DEPTH) {
#pragma unroll
      for (int j = 0; j < DEPTH; ++j) {
        if (k + j + DEPTH - 1 < n)
          issue(k + j + DEPTH - 1, t[(j + DEPTH - 1) % DEPTH], ok[(j + DEPTH - 1) % DEPTH]);
        if (k + j < n) consume(k + j, t[j], ok[j]);
      }
    }
  } else {
    typename QK::Tile t0_;
    bool ok0;
    for (int k = 0; k < n; ++k) {
      issue(k, t0_, ok0);
      consume(k, t0_, ok0);
    }
  }
}

// Gather witness of the balanced schedule: each worker runs the decode kernel's walk over its
// share (worker_share, IssueWalk: unit cursor, block-table entry one issue ahead, tile offset
// under the pool layout's strides) and copies the rows of every tile it would load, the attended
// ones only, to row (token - window start) of its (sequence, KV head) in k_rows / v_rows, 32-bit
// words spread over the 16 lanes of each row group.  A tile whose table entry lies outside the
// pool is not read: its attended rows are written as 0xFF bytes.
__global__ __launch_bounds__(kWave) void balanced_witness_kernel(const BalancedParams bp,
                                                                 char* k_rows, char* v_rows,
                                                                 int row_bytes, int max_rows) {
  const DecodeParams& p = bp.d;
  const QShape qs = make_qshape<false, 1>(p);
  const int lane = threadIdx.x;
  const BalancedCtx ctx{&p, (int64_t)p.stride << p.bs_log2, span_window(p, qs), q_rest(qs)};
  int n = 0;
  Cursor cur;
  if (!worker_share(p, ctx, bp.num_workers, blockIdx.x, lane, nullptr, n, cur)) return;
  IssueWalk walk(ctx, cur);
  const int r = lane >> 4, c = lane & (kRowLanes - 1);
  const int words = row_bytes / 4;
  for (int k = 0; k < n; ++k) {
    Cursor at;
    const int64_t off = walk.next(ctx, k, n, at);
    const int tok0 = (at.s.t0 + at.ti) * kTileTokens;
#pragma unroll
    for (int j = 0; j < kTileSteps; ++j) {
      const int row = kRows * j + r;
      const int i = tok0 + row - at.s.start;
      if (tok0 + row < at.s.start || tok0 + row >= at.s.L || i >= max_rows) continue;
      const size_t dst =
          (((size_t)at.b * p.num_kv_heads + at.kvh) * max_rows + i) * (size_t)row_bytes;
      uint32_t* kd = reinterpret_cast<uint32_t*>(k_rows + dst);
      uint32_t* vd = reinterpret_cast<uint32_t*>(v_rows + dst);
      if (off < 0) {
        for (int x = c; x < words; x += kRowLanes) kd[x] = vd[x] = 0xFFFFFFFFu;
      } else {
        const int64_t src = off + (int64_t)row * p.kv_row_stride;
        const uint32_t* ks = reinterpret_cast<const uint32_t*>(p.k_cache + src);
        const uint32_t* vs = reinterpret_cast<const uint32_t*>(p.v_cache + src);
        for (int x = c; x < words; x += kRowLanes) {
          kd[x] = ks[x];
          vd[x] = vs[x];
        }
      }
    }
  }
}

// Fix-up: one workgroup per (sequence b, KV head kvh, group of H of its G query heads).  Units
// inside one worker were written by the decode kernel; empty units get 0 (or the sink alone); a
// cut unit merges its pieces head by head: M = max lse_i, out = sum e^(lse_i - M) o_i /
// sum e^(lse_i - M), lse = M + ln sum e^(lse_i - M).  The H heads of a piece are H*D contiguous
// floats; each thread takes a 16-byte slice of every RPS-th piece (one pass, a running max per
// slice, the piece's lse loaded with its slice), and the row slots then meet in LDS with the
// same rule.
// The kernel is latency-bound.  Two tilings: with few pieces per unit (workers <= 8 per unit),
// wide workgroups, H = min(G, 1024 / D), one per unit at D = 128 for one query token, because
// dealing out the workgroups then weighs most (7.45 -> 5.76 us on the 128-sequence mixed batch,
// 4.88 -> 4.65 us on the Llama-8B step); with many pieces per unit (long or few sequences),
// H = min(G, 256 / D), four piece rows in flight per step and more workgroups per unit (the wide
// tiling took 6.7 us more on the long-context step, 64 pieces per unit).
constexpr int kFixupThreads = 256;

template <int D, int G, bool WIDE>
constexpr int fixup_heads() {
  constexpr int cap = (WIDE ? 1024 : 256) / D;
  return G < cap ? G : (cap < 1 ? 1 : cap);
}
// the wide tiling when a unit averages at most this many pieces
constexpr int kFixupWideMaxWorkersPerUnit = 8;

template <int D, int G, bool WIDE>
__global__ __launch_bounds__(kFixupThreads) void balanced_fixup_kernel(const BalancedParams bp) {
  constexpr int H = fixup_heads<D, G, WIDE>();
  constexpr int F = H * D / 4;                          // float4 slices per piece row
  constexpr int RPS = kFixupThreads / F;                // piece rows per step
  static_assert(G % H == 0 && kFixupThreads % F == 0, "fix-up tiling");
  const DecodeParams& p = bp.d;
  const int ug = blockIdx.x;
  const int u = ug / (G / H);
  const int h0 = (ug - u * (G / H)) * H;                // first head of this group, within G
  const int b = u / p.num_kv_heads;
  const int kvh = u - b * p.num_kv_heads;
  const int tid = threadIdx.x;
  const int Lb = p.seq_lens[b];
  const int64_t pre_b = bp.prefix[b];
  const int64_t pre_B = bp.prefix[p.num_seqs];
  const QShape qs = make_qshape<true, G>(p);
  const SeqSpan s = seq_span(Lb, span_window(p, qs), (int64_t)p.stride << p.bs_log2, q_rest(qs));
  const int64_t total = pre_B * p.num_kv_heads;
  const int n_eff = effective_workers(total, bp.num_workers);

  int wa = 0, np = 0, first_slot = 0;
  if (s.T > 0) {
    const int64_t S = pre_b * p.num_kv_heads + (int64_t)kvh * s.T;
    wa = worker_of(total, n_eff, S);
    const int wb = worker_of(total, n_eff, S + s.T - 1);
    if (wa == wb) return;   // written by the decode kernel
    np = wb - wa + 1;
    first_slot = worker_begin(total, n_eff, wa) < S ? 1 : 0;
  }

  // piece i of the unit: worker wa + i, slot first_slot for i == 0, else 0
  const int pr = tid / F;
  const int f = tid - pr * F;                           // slice f covers column h0 + 4f / D
  const int hl = (4 * f) / D;
  const int ncols = qs.q_len * qs.group;                // columns past it are padding
  const bool col_ok = h0 + hl < ncols;
  float m = -INFINITY, z = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  bool nan = s.bad;
#pragma unroll 4
  for (int i = pr; i < np; i += RPS) {
    const size_t slot = (size_t)(wa + i) * 2 + (i == 0 ? first_slot : 0);
    const float li = bp.ws_lse[slot * G + h0 + hl];
    const float4 o = *reinterpret_cast<const float4*>(bp.ws_o + (slot * G + h0) * D + 4 * f);
    nan |= col_ok && li != li;   // padding columns' slots are never written
    // a piece with lse = -inf has no weight; selects instead of a branch keep the loads of
    // several pieces in flight
    const float mn = fmaxf(m, li);
    const float e0 = m == mn ? 1.f : fast_exp2((m - mn) * kLog2e);
    const float e1 = li > -INFINITY ? fast_exp2((li - mn) * kLog2e) : 0.f;
    a.x = fmaf(a.x, e0, e1 * o.x);
    a.y = fmaf(a.y, e0, e1 * o.y);
    a.z = fmaf(a.z, e0, e1 * o.z);
    a.w = fmaf(a.w, e0, e1 * o.w);
    z = fmaf(z, e0, e1);
    m = mn;
  }

  __shared__ float s_acc[RPS][H * D];
  __shared__ float s_m[RPS][H], s_z[RPS][H];
  // NaN column by column: a NaN key or length reaches only the columns whose pieces carry it
  // (with KV-head pairs a unit holds two KV heads, and with several query tokens a column may
  // not attend the key)
  __shared__ int s_nan[H];
  if (tid < H) s_nan[tid] = 0;
  __syncthreads();
  if (nan) s_nan[hl] = 1;
  *reinterpret_cast<float4*>(&s_acc[pr][4 * f]) = a;
  if ((4 * f) % D == 0) {   // the first slice of a head carries the head's (max, sum)
    s_m[pr][hl] = m;
    s_z[pr][hl] = z;
  }
  __syncthreads();

  const int sh = __builtin_ctz((unsigned)qs.group);
  for (int e = tid; e < H * D; e += kFixupThreads) {
    const int h = e / D;
    const int n = h0 + h;                               // column: query token n / group
    if (n >= ncols) continue;
    const int hq = kvh * qs.group + (n & (qs.group - 1));
    // the sink logit joins the max and the denominator with a zero value row
    const float sink = p.sinks != nullptr ? p.sinks[hq] : -INFINITY;
    float M = sink;
#pragma unroll
    for (int k = 0; k < RPS; ++k) M = fmaxf(M, s_m[k][h]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float o = 0.f, Z = sink > -INFINITY ? fast_exp2((sink - Mu) * kLog2e) : 0.f;
#pragma unroll
    for (int k = 0; k < RPS; ++k) {
      const float w = fast_exp2((s_m[k][h] - Mu) * kLog2e);   // 0 for an empty row slot
      o = fmaf(s_acc[k][e], w, o);
      Z = fmaf(s_z[k][h], w, Z);
    }
    float ov = Z > 0.f ? o / Z : 0.f;
    float lv = Z > 0.f ? M + fast_log2(Z) * kLn2 : -INFINITY;
    if (s_nan[h]) {
      ov = __builtin_nanf("");
      lv = __builtin_nanf("");
    }
    const size_t row = ((size_t)b * qs.q_total + qs.q_first + (n >> sh)) * p.num_q_heads + hq;
    p.out[row * D + (e - h * D)] = ov;
    if (e == h * D && p.lse != nullptr) p.lse[row] = lv;
  }
}

// ---------------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------------
namespace {

template <int D, int G, QkPath PATH>
using BQK = QkPolicy<D, G, PATH>;

// tiles in flight per worker: two in registers where the registers allow it
template <int D, int G, QkPath PATH>
constexpr int bal_depth() {
  return (D * G <= 512 || G == 32) ? 2 : 1;
}
// or, for FP8 tiles (half the bytes of a bf16 tile, and twice the instructions per byte), tiles
// copied ahead into a ring in LDS: its registers are then free for more workers per SIMD.
// Measured (decode µs, FP8 Llama-8B-shaped step / mixed batch / head_dim 256 sweep point):
// one tile ahead 62.5 / 109.3 / 172.9, two 63.6 / 119.9 / 179.8, three 63.8 / 124.4 / 174.7;
// at head_dim 64 two ahead (52.5) beat one (57.8).  bf16 tiles stay in registers: a ring of
// three or four 8 KiB tiles at one worker per SIMD measured 113.9 µs against 110.4 for the
// register form at two.
#ifndef PA_BAL_AHEAD_FP8_PAIRS
#define PA_BAL_AHEAD_FP8_PAIRS 1
#endif
template <int D, int G, QkPath PATH>
constexpr int bal_ahead() {
  if (PATH == QkPath::kMfmaPvFp8Heads2) return PA_BAL_AHEAD_FP8_PAIRS;
  return PATH == QkPath::kMfmaPvFp8 ? (D == 64 ? 2 : 1) : 0;
}

template <int D, int G, QkPath PATH, bool MULTI>
const void* balanced_kernel_ptr() {
  return reinterpret_cast<const void*>(
      &balanced_decode_kernel<D, G, bal_depth<D, G, PATH>(), BQK<D, G, PATH>, MULTI,
                              bal_ahead<D, G, PATH>()>);
}

template <int D, int G, QkPath PATH, bool MULTI>
hipError_t launch_bal(const BalancedParams& bp, hipStream_t stream) {
  hipLaunchKernelGGL((balanced_decode_kernel<D, G, bal_depth<D, G, PATH>(), BQK<D, G, PATH>,
                                             MULTI, bal_ahead<D, G, PATH>()>),
                     dim3(bp.num_workers), dim3(kWave), 0, stream, bp);
  return hipGetLastError();
}

template <int D, int G, bool WIDE>
hipError_t launch_fix_t(const BalancedParams& bp, hipStream_t stream) {
  hipLaunchKernelGGL((balanced_fixup_kernel<D, G, WIDE>),
                     dim3((unsigned)bp.d.num_seqs * (unsigned)bp.d.num_kv_heads *
                          (unsigned)(G / fixup_heads<D, G, WIDE>())),
                     dim3(kFixupThreads), 0, stream, bp);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_fix(const BalancedParams& bp, hipStream_t stream) {
  const long long units = (long long)bp.d.num_seqs * bp.d.num_kv_heads;
  if ((long long)bp.num_workers <= kFixupWideMaxWorkersPerUnit * units)
    return launch_fix_t<D, G, true>(bp, stream);
  return launch_fix_t<D, G, false>(bp, stream);
}

template <int D>
hipError_t launch_fix_g(const BalancedParams& bp, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_fix<D, 1>(bp, stream);
    case 2: return launch_fix<D, 2>(bp, stream);
    case 4: return launch_fix<D, 4>(bp, stream);
    case 8: return launch_fix<D, 8>(bp, stream);
    case 16: return launch_fix<D, 16>(bp, stream);
    case 32:
      if constexpr (D <= 128) return launch_fix<D, 32>(bp, stream);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

// Sixteen columns exist only for the matrix-core P.V policies (several query tokens), and
// thirty-two (a pair of sixteen) for those at D <= 128.
template <QkPath PATH>
constexpr bool has_16_columns() {
  return PATH == QkPath::kMfmaPv || PATH == QkPath::kMfmaPvFp8;
}
template <int D, QkPath PATH>
constexpr bool has_32_columns() {
  return has_16_columns<PATH>() && D <= 128;
}

// The kernel for (D, columns, path, several query tokens or one).  One token: every path at
// up to 8 columns (heads); several: the matrix-core P.V paths at 2 to 32 columns.
template <int D, int G, QkPath PATH, bool MULTI>
constexpr bool bal_exists() {
  // head pairs: one query token, 4 or 8 columns (the query heads of two KV heads of a group of
  // 2 or 4), head_dim 64 (the plans pair KV heads there only)
  if constexpr (PATH == QkPath::kMfmaPvHeads2 || PATH == QkPath::kMfmaPvFp8Heads2)
    return !MULTI && (G == 4 || G == 8) && D == 64;
  if constexpr (G == 32) return MULTI && has_32_columns<D, PATH>();
  if constexpr (G == 16) return MULTI && has_16_columns<PATH>();
  if constexpr (MULTI) return G >= 2 && has_16_columns<PATH>();
  return true;
}

template <int D, int G, QkPath PATH>
hipError_t launch_bal_m(const BalancedParams& bp, bool multi, hipStream_t stream) {
  if (multi) {
    if constexpr (bal_exists<D, G, PATH, true>()) return launch_bal<D, G, PATH, true>(bp, stream);
  } else {
    if constexpr (bal_exists<D, G, PATH, false>())
      return launch_bal<D, G, PATH, false>(bp, stream);
  }
  return hipErrorInvalidValue;
}

template <int D, int G, QkPath PATH>
const void* bal_ptr_m(bool multi) {
  if (multi) {
    if constexpr (bal_exists<D, G, PATH, true>()) return balanced_kernel_ptr<D, G, PATH, true>();
  } else {
    if constexpr (bal_exists<D, G, PATH, false>())
      return balanced_kernel_ptr<D, G, PATH, false>();
  }
  return nullptr;
}

template <int D, QkPath PATH>
hipError_t launch_bal_g(const BalancedParams& bp, int group, bool multi, hipStream_t stream) {
  switch (group) {
    case 1: return launch_bal_m<D, 1, PATH>(bp, multi, stream);
    case 2: return launch_bal_m<D, 2, PATH>(bp, multi, stream);
    case 4: return launch_bal_m<D, 4, PATH>(bp, multi, stream);
    case 8: return launch_bal_m<D, 8, PATH>(bp, multi, stream);
    case 16: return launch_bal_m<D, 16, PATH>(bp, multi, stream);
    case 32: return launch_bal_m<D, 32, PATH>(bp, multi, stream);
    default: return hipErrorInvalidValue;
  }
}

template <QkPath PATH>
hipError_t launch_bal_d(const BalancedParams& bp, int head_dim, int group, bool multi,
                        hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_bal_g<64, PATH>(bp, group, multi, stream);
    case 128: return launch_bal_g<128, PATH>(bp, group, multi, stream);
    case 256: return launch_bal_g<256, PATH>(bp, group, multi, stream);
    default: return hipErrorInvalidValue;
  }
}

template <QkPath PATH>
const void* bal_ptr(int head_dim, int group, bool multi) {
#define PA_BP(D)                                                   \
  if (head_dim == D) {                                             \
    switch (group) {                                               \
      case 1: return bal_ptr_m<D, 1, PATH>(multi);                 \
      case 2: return bal_ptr_m<D, 2, PATH>(multi);                 \
      case 4: return bal_ptr_m<D, 4, PATH>(multi);                 \
      case 8: return bal_ptr_m<D, 8, PATH>(multi);                 \
      case 16: return bal_ptr_m<D, 16, PATH>(multi);               \
      case 32: return bal_ptr_m<D, 32, PATH>(multi);               \
      default: return nullptr;                                     \
    }                                                              \
  }
  PA_BP(64) PA_BP(128) PA_BP(256)
#undef PA_BP
  return nullptr;
}

}  // namespace

hipError_t launch_balanced(const BalancedParams& bp, int head_dim, int group, QkPath path,
                           bool multi, hipStream_t stream) {
  switch (path) {
    case QkPath::kValu: return launch_bal_d<QkPath::kValu>(bp, head_dim, group, multi, stream);
    case QkPath::kMfma: return launch_bal_d<QkPath::kMfma>(bp, head_dim, group, multi, stream);
    case QkPath::kMfmaPvFp8:
      return launch_bal_d<QkPath::kMfmaPvFp8>(bp, head_dim, group, multi, stream);
    case QkPath::kMfmaPvHeads2:
      return launch_bal_d<QkPath::kMfmaPvHeads2>(bp, head_dim, group, multi, stream);
    case QkPath::kMfmaPvFp8Heads2:
      return launch_bal_d<QkPath::kMfmaPvFp8Heads2>(bp, head_dim, group, multi, stream);
    default: return launch_bal_d<QkPath::kMfmaPv>(bp, head_dim, group, multi, stream);
  }
}

hipError_t launch_balanced_fixup(const BalancedParams& bp, int head_dim, int group,
                                 hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_fix_g<64>(bp, group, stream);
    case 128: return launch_fix_g<128>(bp, group, stream);
    case 256: return launch_fix_g<256>(bp, group, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_balanced_witness(const BalancedParams& bp, char* k_rows, char* v_rows,
                                   int row_bytes, int max_rows, hipStream_t stream) {
  hipLaunchKernelGGL(balanced_witness_kernel, dim3(bp.num_workers), dim3(kWave), 0, stream, bp,
                     k_rows, v_rows, row_bytes, max_rows);
  return hipGetLastError();
}

int balanced_default_workers(int head_dim, int group, QkPath path, bool multi,
                             int64_t units) {
  const void* k = path == QkPath::kValu ? bal_ptr<QkPath::kValu>(head_dim, group, multi)
                  : path == QkPath::kMfma ? bal_ptr<QkPath::kMfma>(head_dim, group, multi)
                  : path == QkPath::kMfmaPvFp8
                      ? bal_ptr<QkPath::kMfmaPvFp8>(head_dim, group, multi)
                  : path == QkPath::kMfmaPvHeads2
                      ? bal_ptr<QkPath::kMfmaPvHeads2>(head_dim, group, multi)
                  : path == QkPath::kMfmaPvFp8Heads2
                      ? bal_ptr<QkPath::kMfmaPvFp8Heads2>(head_dim, group, multi)
                      : bal_ptr<QkPath::kMfmaPv>(head_dim, group, multi);
  if (k == nullptr) return -1;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kWave, 0) != hipSuccess)
    return -1;
  // a whole number of workers per SIMD (four per CU): a SIMD with one worker more than the
  // others runs each of its workers slower, and the launch waits for the slowest (measured:
  // ten FP8 workers per CU took 83 us where eight took 66)
  if (per_cu >= 4) per_cu &= ~3;
  // FP8 tiles through the LDS ring at head_dim 128 (16 workers per CU fit): with fewer than
  // four (sequence, KV head) units per CU, 8 workers per CU stream faster (decode µs at 8 / 16
  // per CU, one query token: the B64 Llama-8B-shaped step, 512 units, 61.6 / 64.8 and 62.4 /
  // 63.8 on two boxes; the B32 L8192 sweep point, 256 units, 91.2 / 92.0; the B4 L131072 step,
  // 32 units, 177.0 / 206.0); with more units the extra workers pay (the B128 mixed batch,
  // 1024 units of 1 to 4096 keys: 115.6 / 110.7)
  if (path == QkPath::kMfmaPvFp8 && head_dim == 128 && !multi && units > 0 &&
      units < 4LL * cus && per_cu > 8)
    per_cu = 8;
  const long long n = (long long)cus * (per_cu > 0 ? per_cu : 1);
  return (int)(n < (1 << 20) ? n : (1 << 20));
}

}  // namespace pa
