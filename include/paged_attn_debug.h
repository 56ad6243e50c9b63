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
 * Streaming-read probe: reads `bytes` (a multiple of 16) from `buf` with 16-byte coalesced
 * non-temporal loads (the load kind the decode kernels use for K/V), as many workgroups as
 * `num_workgroups`, and writes one 32-bit checksum per workgroup to
 * `sink` (uint32 [num_workgroups]) so the loads cannot be elided.  Attainable HBM read
 * bandwidth next to the nominal figure.
 */
pa_status paged_attn_stream_read(const void* buf, size_t bytes, int32_t num_workgroups,
                                 uint32_t* sink, void* stream);

/* Plain device copy of `bytes` (a multiple of 16): a kernel of known traffic for calibrating
 * hardware byte counters. */
pa_status paged_attn_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_DEBUG_H */
