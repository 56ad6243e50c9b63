// Device helpers for the gfx950 paged-attention kernels: wave64 cross-lane reductions, bf16
// unpacking and the tile -> KV address generator shared by the decode and witness kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#if !defined(__HIP_DEVICE_COMPILE__) || defined(__gfx950__)
#else
#error "these kernels are written for gfx950 (CDNA4) only"
#endif

namespace pa {

// ---------------------------------------------------------------------------------------------
// Lane geometry.  A wave64 is four DPP rows of 16 lanes.  One KV row (head_dim bf16 values) is
// spread over the 16 lanes of one DPP row, so one wave-wide load instruction covers four
// consecutive rows, a contiguous 4 * head_dim * 2 bytes (1 KiB at head_dim 128).  A tile is
// 16 consecutive tokens: row group r (lane / 16) handles tokens 4j + r, j = 0..3.
// ---------------------------------------------------------------------------------------------
constexpr int kWave = 64;
constexpr int kRowLanes = 16;
constexpr int kRows = kWave / kRowLanes;   // 4 row groups per wave
constexpr int kTileTokens = 16;
constexpr int kTileSteps = kTileTokens / kRows;   // 4 tokens per row group per tile

static_assert(kWave == 64, "wave64 only");

// 32-bit words (bf16 pairs) a lane holds of one row: 2 (8 B) at head_dim 64, 4 (16 B) at 128,
// 8 (two 16 B pieces) at 256.
template <int D>
struct RowGeom {
  static_assert(D == 64 || D == 128 || D == 256, "head_dim 64/128/256");
  static constexpr int kWords = D / 32;
  static constexpr int kElems = 2 * kWords;   // bf16 values per lane per row
  static constexpr int kRowBytes = D * 2;
  // head-dim index of element e held by lane c of a row group
  __device__ __host__ static constexpr int dim(int c, int e) {
    return D == 256 ? (e < 8 ? 8 * c + e : 128 + 8 * c + (e - 8)) : c * kElems + e;
  }
};

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// A KV load: non-temporal (NT) where a row is read exactly once per step (on gfx950 streaming
// reads with the hint reach a markedly higher HBM rate than plain loads), plain where several
// workgroups read the same rows and should find them in L2.
template <bool NT, class T>
__device__ __forceinline__ T kv_load(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// One 16-byte piece per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane i's piece from base + voff (base wave-uniform, in scalar registers; voff the lane's
// 32-bit offset) to lds_wave_base + 16 i (M0 holds the wave's LDS base).  NT: with the
// non-temporal hint.  The instruction writes no register and is counted by vmcnt until its
// data sits in LDS, so the caller waits for it (s_waitcnt vmcnt) before reading the piece.
// Inline assembly, so that the compiler does not take every later LDS read as possibly
// aliasing a copy in flight and wait for all copies before it.
template <bool NT = false>
__device__ __forceinline__ void copy_piece_to_lds_s(const char* base, uint32_t voff,
                                                    const char* lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)reinterpret_cast<uintptr_t>(lds_wave_base));
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 ::"s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 ::"s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
}

// Load the kWords words lane c holds of the row starting at byte address `row`.
template <int D, bool NT = true>
__device__ __forceinline__ void load_row(const char* __restrict__ row, int c,
                                         uint32_t (&w)[RowGeom<D>::kWords]) {
  if constexpr (D == 64) {
    const u32x2_t x = kv_load<NT>(reinterpret_cast<const u32x2_t*>(row + c * 8));
    w[0] = x.x; w[1] = x.y;
  } else if constexpr (D == 128) {
    const u32x4_t x = kv_load<NT>(reinterpret_cast<const u32x4_t*>(row + c * 16));
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else {
    const u32x4_t x = kv_load<NT>(reinterpret_cast<const u32x4_t*>(row + c * 16));
    const u32x4_t y = kv_load<NT>(reinterpret_cast<const u32x4_t*>(row + 256 + c * 16));
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    w[4] = y.x; w[5] = y.y; w[6] = y.z; w[7] = y.w;
  }
}

// q rows are small and reused: plain loads
template <int D>
__device__ __forceinline__ void load_row_cached(const char* __restrict__ row, int c,
                                                uint32_t (&w)[RowGeom<D>::kWords]) {
  if constexpr (D == 64) {
    const uint2 x = *reinterpret_cast<const uint2*>(row + c * 8);
    w[0] = x.x; w[1] = x.y;
  } else if constexpr (D == 128) {
    const uint4 x = *reinterpret_cast<const uint4*>(row + c * 16);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else {
    const uint4 x = *reinterpret_cast<const uint4*>(row + c * 16);
    const uint4 y = *reinterpret_cast<const uint4*>(row + 256 + c * 16);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    w[4] = y.x; w[5] = y.y; w[6] = y.z; w[7] = y.w;
  }
}

template <int D>
__device__ __forceinline__ void store_row(char* __restrict__ row, int c,
                                          const uint32_t (&w)[RowGeom<D>::kWords]) {
  if constexpr (D == 64) {
    *reinterpret_cast<uint2*>(row + c * 8) = make_uint2(w[0], w[1]);
  } else if constexpr (D == 128) {
    *reinterpret_cast<uint4*>(row + c * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *reinterpret_cast<uint4*>(row + c * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(row + 256 + c * 16) = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// bf16 pair -> two fp32 (exact: bf16 is the upper half of an fp32)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// acc + a.x*b.x + a.y*b.y on two bf16 pairs, fp32 accumulate (v_dot2c_f32_bf16).  Products of
// two bf16 values are exact in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// ---------------------------------------------------------------------------------------------
// wave64 reductions.
//
// row_sum16: sum over the 16 lanes of each DPP row, result in every lane of the row.  Four DPP
// steps: row_mirror (i <-> 15-i), row_half_mirror (i <-> 7-i within each half), then the two
// quad permutations xor 2 and xor 1.  After the two mirrors, the four lanes of each quad hold
// sums over four disjoint 4-lane sets that together cover the row, so the quad steps finish the
// sum.  DPP moves stay inside a 16-lane row, so this is the same on any wave size; the
// cross-row steps below are what a 64-wide wave adds.
// ---------------------------------------------------------------------------------------------
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<kDppRowMirror>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppQuadXor1>(x);
  return x;
}

// Lanes l and l ^ MASK (MASK = 16: the two rows of a row pair; 32: the two halves of the wave)
// cross DPP rows.  v_permlane16_swap / v_permlane32_swap exchange them without the LDS crossbar:
// given x twice, each returns the pair (value of the pair's first row or half, value of its
// second) at both lanes of the pair.
template <int MASK>
__device__ __forceinline__ void lane_pair(float x, float& first, float& second) {
  static_assert(MASK == 16 || MASK == 32, "row pairs or wave halves");
  const int xi = __builtin_bit_cast(int, x);
  int a, b;
  if constexpr (MASK == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
    a = (int)r[0];
    b = (int)r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
    a = (int)r[0];
    b = (int)r[1];
  }
  first = __builtin_bit_cast(float, a);
  second = __builtin_bit_cast(float, b);
}

// Value of x in lane (lane ^ MASK), MASK = 16 or 32.
template <int MASK>
__device__ __forceinline__ float xor_lane(float x) {
  float first, second;
  lane_pair<MASK>(x, first, second);
  return (__lane_id() & MASK) == 0 ? second : first;
}

// Max / sum over the four rows of a wave64 (both steps are needed; stopping at the row pair
// would only combine two rows).  Every lane of a pair combines the same two values in the same
// order, so the four rows end with identical bits.
__device__ __forceinline__ float rows_max(float x) {
  float a, b;
  lane_pair<16>(x, a, b);
  lane_pair<32>(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float rows_sum(float x) {
  float a, b;
  lane_pair<16>(x, a, b);
  lane_pair<32>(a + b, a, b);
  return a + b;
}

// full-wave sum / max (every lane gets the result)
__device__ __forceinline__ float wave_sum(float x) { return rows_sum(row_sum16(x)); }

__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<kDppRowMirror>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  return x;
}

__device__ __forceinline__ float wave_max(float x) { return rows_max(row_max16(x)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One sequence's attended range [start, L) in 16-token tiles: tiles [t0, t0 + T).  T = 0 for an
// empty sequence or one whose length the block table cannot hold (bad).
struct SeqSpan {
  int L, start, t0, T;
  bool bad;
};

// (q_rest: query tokens after this launch's last one; its keys end q_rest before L)
__device__ __forceinline__ SeqSpan seq_span(int L, int window, int64_t cap, int q_rest = 0) {
  SeqSpan s;
  s.bad = L < 0 || (int64_t)L > cap;
  const int Lc = s.bad ? 0 : (L > q_rest ? L - q_rest : 0);
  s.L = s.bad ? L : Lc;
  s.start = (window > 0 && Lc > window) ? Lc - window : 0;
  s.t0 = s.start / kTileTokens;
  s.T = Lc > 0 ? (Lc + kTileTokens - 1) / kTileTokens - s.t0 : 0;
  return s;
}

// ---------------------------------------------------------------------------------------------
// Tile addressing (block-table walk).  Tile t covers tokens [16t, 16t+16), which never straddle
// a block because block_size is a multiple of 16.  Token 16t is slot (16t mod block_size) of
// logical block 16t / block_size; its physical block comes from the sequence's block-table row.
// Byte offset of the tile's first row: phys * block_stride + kvh * head_stride + slot *
// row_stride, computed in 64 bits.  The default pool [num_blocks][Hkv][block_size][D] has
// row_stride = D * element bytes, head_stride = block_size * row_stride and block_stride =
// Hkv * head_stride; other layouts (token-major, K and V interleaved per block, padded rows)
// only change the three strides.  A table entry outside [0, num_blocks) yields -1: the caller
// must not read.  All operands are wave-uniform, so this is scalar code.
// ---------------------------------------------------------------------------------------------
struct TileAddr {
  int32_t num_blocks;
  int32_t bs_log2;
  int64_t block_stride;   // bytes between physical blocks
  int64_t head_off;       // kvh * head stride, bytes
  int64_t row_stride;     // bytes between a block's consecutive tokens

  // index into the sequence's block-table row of the block holding tile t
  __device__ __forceinline__ int logical_block(int tile) const {
    return (tile * kTileTokens) >> bs_log2;
  }
  // byte offset of tile t's first row given its physical block, -1 if phys is out of range
  __device__ __forceinline__ int64_t offset(int phys, int tile) const {
    if (phys < 0 || phys >= num_blocks) return -1;
    const int slot = (tile * kTileTokens) & ((1 << bs_log2) - 1);
    return (int64_t)phys * block_stride + head_off + (int64_t)slot * row_stride;
  }
};

// Workgroup -> (partition, KV head, sequence).  The chip deals workgroups to its 8 XCDs
// round-robin by linear id, so the KV head varies fastest, then the sequence, then the
// partition: every XCD gets an even share of full and partial partitions, and the empty
// partitions of short sequences (high partition index) come last.  (With the partition index
// fastest, XCD k would receive only partition k mod 8 of every sequence: measured 12x more
// work on one XCD than on another for 512-token partitions of a 512..4096-token batch.)
struct WorkItem {
  int part, kvh, b;
};

__device__ __forceinline__ WorkItem decode_work_item(int num_kv_heads, int num_seqs) {
  const unsigned id = blockIdx.x;
  const unsigned per_part = (unsigned)num_kv_heads * (unsigned)num_seqs;
  WorkItem w;
  w.part = (int)(id / per_part);
  const unsigned rem = id - (unsigned)w.part * per_part;
  w.b = (int)(rem / (unsigned)num_kv_heads);
  w.kvh = (int)(rem - (unsigned)w.b * (unsigned)num_kv_heads);
  return w;
}

// Attended token range of partition `part` of a sequence of length L, and the validity of L.
struct PartRange {
  int lo, hi;        // tokens [lo, hi)
  int first_part;    // partition that holds the sink (the first non-empty one)
};

__device__ __forceinline__ PartRange part_range(int L, int window, int part, int psize) {
  PartRange r;
  const int start = (window > 0 && L > window) ? L - window : 0;
  if (psize > 0) {
    const int64_t plo = (int64_t)part * psize;
    const int64_t phi = plo + psize;
    r.lo = (int)(plo > start ? plo : start);
    r.hi = (int)(phi < L ? phi : L);
    if (r.hi < r.lo) r.hi = r.lo;
    r.first_part = start / psize;
  } else {
    r.lo = start;
    r.hi = L;
    r.first_part = 0;
  }
  return r;
}

}  // namespace pa
