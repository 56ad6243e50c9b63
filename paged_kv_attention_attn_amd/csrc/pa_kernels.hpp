// Kernel parameter blocks and the host-side launch entry points of the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct DecodeParams {
  const uint16_t* q;          // bf16 [B][Hq][D]
  const char* k_cache;        // bf16 rows of D values (FP8 path: E4M3 bytes), placed by the
  const char* v_cache;        // layout strides below (default [NB][Hkv][bs][D])
  const int32_t* block_table; // [B][stride]
  const int32_t* seq_lens;    // [B]
  const float* sinks;         // [Hq] or null
  float* out;                 // unsplit [B][Hq][D]; split [B][Hq][Pmax][D]
  float* lse;                 // unsplit [B][Hq] or null; split [B][Hq][Pmax]
  float qk_scale_log2;        // scale * log2(e) (FP8 path: times the K scale)
  float v_scale;              // FP8 path: multiplier on the output; unused otherwise
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t stride;
  int32_t bs_log2;
  int32_t window;
  int32_t psize;              // 0 = unsplit
  int32_t max_parts;          // split: partition slots; unsplit: 1
  // Query tokens (1 = one-token decode; more only on the balanced schedule): q
  // [B][q_total][Hq][D], out [B][q_total][Hq][D], lse [B][q_total][Hq]; token t of sequence b
  // sits at position seq_lens[b] - q_total + t and attends causally.  A launch serves tokens
  // [q_first, q_first + q_len).  group = Hq / Hkv; a kernel's G template parameter counts
  // columns (query token, head) per KV head, q_len * group <= G.
  int32_t q_len;
  int32_t q_total;
  int32_t q_first;
  int32_t group;
  // KV pool layout in bytes, the same for K and V: row of (block phys, head kvh, slot s) at
  // phys * kv_block_stride + kvh * kv_head_stride + s * kv_row_stride.  Rows are 16-byte aligned.
  int64_t kv_block_stride;
  int64_t kv_head_stride;
  int64_t kv_row_stride;
  // Head-pair kernels (QkPath::kMfmaPvHeads2, kMfmaPvFp8Heads2): a unit is KV heads 2u and 2u + 1, num_kv_heads
  // and kv_head_stride count pairs, group counts the pair's query heads, and the second head's
  // rows sit kv_pair_off bytes after the first's.  0 otherwise.
  int64_t kv_pair_off;
  // Split only, optional: the last partition of each (sequence, KV head) to finish merges them
  // all into final_out [B][Hq][D] / final_lse [B][Hq] (or null).  merge_counters [B][Hkv] are
  // zero on entry and left zero.
  uint32_t* merge_counters;
  float* final_out;
  float* final_lse;
};

// The query tokens of a launch (see DecodeParams).  Kernels built for one query token use the
// constant shape {1, 1, 0, G}, so that the general fields cost no registers there.
struct QShape {
  int q_len, q_total, q_first, group;
};
template <bool MULTI, int G>
__host__ __device__ inline QShape make_qshape(const DecodeParams& p) {
  if constexpr (MULTI) return QShape{p.q_len, p.q_total, p.q_first, p.group};
  return QShape{1, 1, 0, G};
}

// Balanced decode: persistent workers over the flattened tiles, partials in a workspace.
struct BalancedParams {
  DecodeParams d;             // out/lse are the final outputs; psize/max_parts unused
  int64_t* prefix;            // [B + 1] tiles per KV head before sequence b (written by worker 0)
  float* ws_lse;              // [N][2][G] partial LSEs (natural log)
  float* ws_o;                // [N][2][G][D] partial outputs (normalised)
  int32_t num_workers;        // N, one wave each
};

// Query-block grid for several query tokens per sequence: one workgroup per (sequence, KV head,
// waves blocks of tokens_per_block query tokens, key split), each streaming its share of the
// keys its tokens attend.  With one split it writes the outputs; with several, each split writes
// a normalised partial output and its LSE, and the merge kernel combines them.
struct QBlockParams {
  DecodeParams d;             // q_total = query tokens per sequence; q_len and q_first unused
  int32_t tokens_per_block;   // columns per wave / group
  int32_t waves;              // waves per workgroup, each one block of tokens (1, or 4 sharing
                              // the K/V tiles through LDS)
  int32_t blocks_per_seq;     // workgroup blocks per (sequence, KV head):
                              // ceil(q_total / (tokens_per_block * waves))
  int32_t xcd_pinned;         // 1: every workgroup of a (sequence, KV head) on one XCD
  int32_t p_one_term;         // 1: the 32-key workgroup form takes P as one bf16 term
  int32_t splits;             // key splits per workgroup block (1 = none)
  int32_t split_tiles;        // splits > 1: tiles per split, counted from the first tile of the
                              // workgroup's key range; the last split takes the rest
  uint32_t grid;              // workgroups launched: units * blocks_per_seq * splits (rounded
                              // up to whole XCD rounds when xcd_pinned)
  float* part_out;            // splits > 1: [B * q_total * Hq][splits][D] normalised partials
  float* part_lse;            // splits > 1: [B * q_total * Hq][splits] (natural log, no sink)
};

struct ReduceParams {
  const float* partials;      // [B][Hq][Pmax][D]
  const float* lse_partials;  // [B][Hq][Pmax]
  const int32_t* seq_lens;
  float* out;                 // [B][Hq][D]
  float* lse;                 // [B][Hq] or null
  int32_t num_q_heads;
  int32_t psize;
  int32_t max_parts;
};

struct WitnessParams {
  const char* k_cache;
  const char* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  char* k_rows;               // bf16 [B][Hkv][max_rows][D]
  char* v_rows;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t stride;
  int32_t bs_log2;
  int32_t window;
  int32_t max_rows;
};

// Launchers return hipSuccess or the launch error.  Grid and variant choice is theirs; the
// caller has validated the parameters.
// Decode kernels: q.k on the vector ALUs (dot2 + DPP) with P.V in fp32 on the vector ALUs
// (kValu); q.k on the matrix cores with P.V on the vector ALUs (kMfma); or both on the matrix
// cores, P carried as two bf16 terms (kMfmaPv); the same for a KV cache of FP8 E4M3 codes with
// per-tensor scales, converted to bf16 in registers (kMfmaPvFp8).
enum class QkPath {
  kValu = 0,
  kMfma = 1,
  kMfmaPv = 2,
  kMfmaPvFp8 = 3,
  kMfmaPvHeads2 = 4,      // bf16 KV-head pairs (balanced, one query token)
  kMfmaPvFp8Heads2 = 5,   // FP8 KV-head pairs
};
// Short name of a path ("valu", "mfma", "mfmapv").
const char* qk_path_name(QkPath path);
// Grid: one workgroup per (partition slot, KV head, sequence), 1-D.
hipError_t launch_decode(const DecodeParams& p, int head_dim, int group, int waves, QkPath path,
                         hipStream_t stream);
// Variant name; the string lives in thread-local storage until the next call on this thread.
const char* decode_variant_name(int head_dim, int group, int waves, bool split, QkPath path);
QkPath decode_default_path(int head_dim, int group);
bool decode_supported(int head_dim, int group);
bool decode_waves_supported(int waves);
int decode_default_waves(int head_dim, int group, int psize);

hipError_t launch_reduce(const ReduceParams& p, int head_dim, int num_seqs, hipStream_t stream);

// Balanced decode: the worker kernel, and the fix-up merge, each on `stream`.  `group` is the
// kernels' column count: Hq/Hkv, or with q_len > 1 the (token, head) pairs rounded up to a power
// of two (32 at most, matrix-core P.V paths only).  `multi` selects the kernels that read the
// query-token fields (needed whenever q_len or q_total is above 1).
hipError_t launch_balanced(const BalancedParams& bp, int head_dim, int group, QkPath path,
                           bool multi, hipStream_t stream);
hipError_t launch_balanced_fixup(const BalancedParams& bp, int head_dim, int group,
                                 hipStream_t stream);
// The balanced workers' walk (shares, cursors, table entries, tile offsets under the layout
// strides of bp.d) copying each attended K/V row of (b, kvh) to row (token - window start) of
// k_rows / v_rows [B][Hkv][max_rows][row_bytes] instead of computing; bp.prefix is not used.
hipError_t launch_balanced_witness(const BalancedParams& bp, char* k_rows, char* v_rows,
                                   int row_bytes, int max_rows, hipStream_t stream);
// Default persistent workers for a balanced launch on the current device: as many as fit at
// once (CUs x resident one-wave workgroups per CU, a whole number per SIMD); with `units`
// (sequences x KV heads, 0 = not known) some paths take fewer when the batch has few units.
// -1 if the query fails.
int balanced_default_workers(int head_dim, int group, QkPath path, bool multi = false,
                             int64_t units = 0);

// Query-block grid: (token, head) columns per wave (32 at head_dim <= 128, 16 at 256; the
// matrix-core P.V paths only), the grid for the shape, and the launch.
int qblock_columns(int head_dim);
// Fills tokens_per_block, waves, blocks_per_seq, xcd_pinned, splits, split_tiles and grid;
// max_seq_len (a host-side bound on the lengths, 0 if unknown) sizes the key splits.
void qblock_geometry(QBlockParams& qp, int head_dim, int max_seq_len);
// The query-block kernels; with key splits (splits > 1) launch_qblock_merge then merges the
// partials into d.out / d.lse (a no-op without splits).
hipError_t launch_qblock(const QBlockParams& qp, int head_dim, QkPath path, hipStream_t stream);
hipError_t launch_qblock_merge(const QBlockParams& qp, int head_dim, hipStream_t stream);

hipError_t launch_witness(const WitnessParams& p, int head_dim, int num_seqs, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, size_t bytes, int num_wg, uint32_t* sink,
                              hipStream_t stream);
hipError_t launch_gather_read(const void* buf, int64_t num_chunks, int chunk_bytes,
                              const int32_t* ids, int64_t n_ids, int num_wg, uint32_t* sink,
                              hipStream_t stream);
hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

}  // namespace pa
