/*
 * paged_attn_debug.h — test and measurement entry points of the paged-attention library.
 *
 * These are not part of the decode path.  They exist so that tests can see, byte for byte, what
 * the decode kernels' address generation selects, and so that the bench can relate the decode
 * kernel's bandwidth to what a plain streaming kernel reaches on the same device.  Same
 * conventions as paged_attn.h: host-side validation first, asynchronous on the given stream,
 * nothing allocated.
 */
#ifndef PAGED_ATTN_DEBUG_H
#define PAGED_ATTN_DEBUG_H

#include <stddef.h>
#include <stdint.h>

#include "paged_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Gather witness.  Copies the K and V rows that the decode kernels' tile address generator
 * selects for every (sequence b, KV head kvh) into contiguous buffers, through the same device
 * code the decode kernels use: row i of (b, kvh) is attended token start + i, where
 * start = max(0, L - window) (0 without a window).  Kernel-resident evidence of the integer path
 * (block-table walk, slot and head offsets, window start, tail), compared bit-exactly with the
 * oracle's gather.  Paged KV cache with block tables: ROCm/rocm-libraries PR #13700, "Runnable
 * saved-binding HIP-event comparison" (page size 16); window skip: randomvariable/vllm issue #23,
 * "Attention parity", table "Current state".
 *
 *   k_rows, v_rows  bf16 [B][Hkv][max_rows][head_dim], device; rows past the attended count
 *                   are not written.  Rows of a (b, kvh) whose table holds an id outside
 *                   [0, num_blocks) are written as bf16 NaN (0x7FC0) instead of being read.
 *   max_rows        >= the largest attended count min(L, window or L); the kernel writes at most
 *                   max_rows rows per (b, kvh).
 */
pa_status paged_attn_gather_witness(const pa_shape* shape, const void* k_cache,
                                    const void* v_cache, const int32_t* block_table,
                                    const int32_t* seq_lens, int32_t head_dim,
                                    int32_t block_size, int32_t window, int32_t max_rows,
                                    void* k_rows, void* v_rows, void* stream);

/*
 * Gather witness of the balanced schedule: the same rows as paged_attn_gather_witness, selected
 * by the balanced decode kernel's own walk instead of a per-(sequence, KV head) loop.  num_workers
 * persistent workers each take their contiguous share of the flattened 16-token tiles (so units
 * are cut between workers exactly as in paged_attn_decode_balanced with that worker count), step
 * the unit cursor, fetch each tile's block-table entry and form its row offsets under the pool
 * layout, then copy the attended rows.  Balanced persistent workers over split-KV pieces:
 * ROCm/rocm-libraries PR #13700 (split-KV partials and their reducer), placed where the work
 * balances; kernel-resident witnesses of an integer path: vllm.cpp PR #2472 "cooperate across
 * Q8_K activation blocks", Evidence.
 *
 *   kv_dtype     PA_KV_BF16 (rows of 2 * head_dim bytes) or PA_KV_FP8_E4M3 (head_dim bytes)
 *   kv_layout    NULL for [num_blocks][Hkv][block_size][head_dim], else the strides of
 *                pa_kv_layout (checked as for paged_attn_plan_create)
 *   num_workers  1 .. 2^20 (no default: the caller picks the cut)
 *   k_rows, v_rows  [B][Hkv][max_rows][row bytes], device; row i of (b, kvh) is attended token
 *                start + i; rows past the attended count are not written.  A row whose table
 *                entry lies outside [0, num_blocks) is written as 0xFF bytes instead of being
 *                read.
 */
pa_status paged_attn_gather_witness_balanced(const pa_shape* shape, const void* k_cache,
                                             const void* v_cache, const int32_t* block_table,
                                             const int32_t* seq_lens, int32_t head_dim,
                                             int32_t block_size, int32_t window,
                                             int32_t kv_dtype, const pa_kv_layout* kv_layout,
                                             int32_t num_workers, int32_t max_rows, void* k_rows,
                                             void* v_rows, void* stream);

/*
 * Streaming-read probe: reads `bytes` (a multiple of 16) from `buf` with 16-byte coalesced
 * non-temporal loads (the load kind the decode kernels use for K/V), as many workgroups as
 * `num_workgroups`, and writes one 32-bit checksum per workgroup to
 * `sink` (uint32 [num_workgroups]) so the loads cannot be elided.  Attainable HBM read
 * bandwidth next to the nominal figure.
 */
pa_status paged_attn_stream_read(const void* buf, size_t bytes, int32_t num_workgroups,
                                 uint32_t* sink, void* stream);

/*
 * Gather-read probe: the decode kernels' access pattern without their arithmetic.  `buf` holds
 * bytes / chunk_bytes chunks of chunk_bytes (2048, 4096 or 8192: a 16-token tile of one KV head at
 * head_dim 64, 128 or 256); the probe reads the chunks listed in chunk_ids (int32 [num_ids],
 * device; any order, e.g. a random permutation as a shuffled block pool gives) with 16-byte
 * non-temporal loads, one wave per chunk, each wave of num_workgroups * 4 taking a contiguous
 * share of the list with two chunks in flight, and writes one checksum per workgroup to
 * `sink` (uint32 [num_workgroups]).  Ids outside [0, bytes / chunk_bytes) are skipped, never read.
 * The rate this reaches is what a decode kernel that streams the same tiles can attain.
 */
pa_status paged_attn_gather_read(const void* buf, size_t bytes, int32_t chunk_bytes,
                                 const int32_t* chunk_ids, int64_t num_ids,
                                 int32_t num_workgroups, uint32_t* sink, void* stream);

/* Plain device copy of `bytes` (a multiple of 16): a kernel of known traffic for calibrating
 * hardware byte counters. */
pa_status paged_attn_copy(void* dst, const void* src, size_t bytes, void* stream);

/*
 * paged_attn_plan_run with the decode kernel bracketed by two HIP events: ev_before (a
 * hipEvent_t, NULL for none) is recorded on `stream` right before the plan's decode launch
 * (the query-block launch on that schedule) and ev_after right after it, ahead of any merge
 * launch, so that hipEventElapsedTime(ev_before, ev_after) is that kernel's own duration.  When
 * a plan runs several passes of query tokens, the events bracket the first pass's decode
 * launch.  Arguments, checks and results otherwise as paged_attn_plan_run; an event that fails
 * to record is PA_ERR_LAUNCH.
 */
pa_status paged_attn_plan_run_timed(const pa_plan* plan, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* block_table,
                                    const int32_t* seq_lens, float scale, float k_scale,
                                    float v_scale, const float* sinks, float* out, float* lse,
                                    void* workspace, void* stream, void* ev_before,
                                    void* ev_after);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_DEBUG_H */
