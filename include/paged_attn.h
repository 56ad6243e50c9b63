/*
 * paged_attn.h — C ABI of the MI355X (gfx950) single-token paged-attention decode library.
 *
 * The operation: for each sequence b and query head h, one new query token q[b][h] attends over
 * the sequence's cached keys and values, which live in fixed-size physical blocks of a shared KV
 * pool and are located through the sequence's block table.  The library computes
 *
 *     out[b][h] = sum_t softmax_t(scale * q[b][h] . k_t) v_t,     lse[b][h] = ln(denominator)
 *
 * over the attended tokens t, with grouped-query sharing (Hq/Hkv query heads per KV head), an
 * optional sliding window and optional per-head attention-sink logits.  Long sequences may be
 * split into partitions that each emit a partial output plus a log-sum-exp, merged by a second
 * call.  Sources for the definition:
 *   - one-token split-KV decode with an optional LSE output and a reducer that takes the output,
 *     the sequence lengths and the LSE buffer: ROCm/rocm-libraries PR #13700 "prepare saved paged
 *     decode bindings once", Summary and review finding N1;
 *   - online softmax that only changes the reduction order: vllm.cpp PR #564 "spec(BACKEND-ROCM):
 *     the ROCm head_dim=128 decode arm", section "It is a mirror of merged work, not new design";
 *   - GQA groups of query heads per KV head (qg = 2/4/8): same page, "What is deliberately not
 *     here";
 *   - sliding window with out-of-window blocks skipped, and attention sinks: randomvariable/vllm
 *     issue #23 "Attention parity", table "Current state".
 *
 * Readings where the pages are silent (fixed here as the contract):
 *   - KV pools k_cache and v_cache are bf16 [num_blocks][Hkv][block_size][head_dim], contiguous.
 *     Token t of sequence b is slot (t % block_size) of physical block
 *     block_table[b * block_table_stride + t / block_size].
 *   - q is bf16 [num_seqs][Hq][head_dim]; query head h reads KV head h / (Hq / Hkv).
 *   - out is fp32 [num_seqs][Hq][head_dim]; lse is fp32, natural log.
 *   - window W > 0 keeps the last min(L, W) tokens, t in [L - W, L); W = 0 means no window.
 *   - a sink is one fp32 logit per query head that joins the softmax max and denominator with a
 *     zero value row; lse includes it.
 *   - split mode: partition p covers tokens [p*P, (p+1)*P) of the attended range; a sequence of
 *     length L owns max(1, ceil(L / P)) partitions; the sink is folded into the first non-empty
 *     partition, floor(start / P); an empty partition writes o = 0 and lse = -inf.
 *   - L = 0 yields out = 0 and lse = -inf (lse = sink when a sink is given).
 *
 * Ownership and concurrency: the caller owns every buffer.  The library allocates nothing, keeps
 * no global state (apart from the device array of paged_attn_decode_balanced_noalloc and its
 * address per GPU) and is safe to call from several host threads.  Calls are asynchronous on the
 * given stream (a hipStream_t passed as void*, NULL = the null stream); outputs are valid once
 * that stream reaches the call.
 *
 * Errors: every check below runs on the host before anything is launched; a failed check
 * returns its status and touches no memory.  Values that live in device memory (block-table
 * entries, sequence lengths) cannot be checked on the host without a copy; the kernels check
 * them and, instead of reading out of bounds, write NaN to every output of the affected
 * (sequence, head): a physical block id outside [0, num_blocks), a length L < 0 or
 * L > block_table_stride * block_size, or (split mode) a sequence needing more than
 * max_partitions partitions.  paged_attn_check_tables() runs the same checks on host copies.
 * NaN inputs propagate as in the definition: a NaN in an attended key row makes the outputs and
 * LSEs of that KV head's query heads NaN; a NaN in an attended value row makes that one output
 * dimension NaN; NaNs outside the attended range (unused slots, masked tokens) are never read
 * into a result.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,          /* a required pointer is NULL                                     */
  PA_ERR_SHAPE = -2,         /* sizes inconsistent or out of range                             */
  PA_ERR_UNSUPPORTED = -3,   /* (head_dim, Hq/Hkv, block_size) outside the compiled set        */
  PA_ERR_LSE_REQUIRED = -4,  /* split mode (partition_size > 0) without an lse buffer          */
  PA_ERR_LAUNCH = -5,        /* the HIP runtime rejected the launch                            */
  PA_ERR_TABLE = -6          /* paged_attn_check_tables found a bad entry or length            */
} pa_status;

/* Host-side sizes; nothing in here is read from device memory. */
typedef struct {
  int32_t num_seqs;            /* B >= 0                                                        */
  int32_t num_q_heads;         /* Hq >= 1                                                       */
  int32_t num_kv_heads;        /* Hkv >= 1, Hq % Hkv == 0                                       */
  int32_t num_blocks;          /* physical blocks in each of k_cache / v_cache, >= 1            */
  int32_t block_table_stride;  /* int32 entries per block-table row, >= 1                       */
  int32_t partition_size;      /* 0 = unsplit; else tokens per partition, a multiple of 16      */
  int32_t max_partitions;      /* split mode: partition slots per (b, h) in the partial buffers */
} pa_shape;

/*
 * One decode step over the whole batch.
 *
 *   q            bf16 [B][Hq][head_dim]                                   device, read
 *   k_cache      bf16 [num_blocks][Hkv][block_size][head_dim]             device, read
 *   v_cache      bf16 [num_blocks][Hkv][block_size][head_dim]             device, read
 *   block_table  int32 [B][block_table_stride]; entries past ceil(L/bs) are never read
 *   seq_lens     int32 [B]                                                device, read
 *   scale        fp32 multiplier on q.k (finite)
 *   head_dim     64, 128 or 256;   Hq / Hkv in {1, 2, 4, 8}
 *   block_size   16, 32, 64, 128 or 256 tokens
 *   window       0 (none) or W > 0
 *   sinks        fp32 [Hq] sink logits, or NULL
 *   out          unsplit: fp32 [B][Hq][head_dim]
 *                split:   partial outputs fp32 [B][Hq][max_partitions][head_dim], each normalised
 *                         within its partition
 *   lse          unsplit: fp32 [B][Hq], or NULL (then nothing but out is written)
 *                split:   REQUIRED, fp32 [B][Hq][max_partitions]
 *   stream       hipStream_t
 *
 * Slots p >= max(1, ceil(L/P)) of the partial buffers are not written.
 */
pa_status paged_attn_decode(const pa_shape* shape, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            const int32_t* seq_lens, float scale, int32_t head_dim,
                            int32_t block_size, int32_t window, const float* sinks, float* out,
                            float* lse, void* stream);

/*
 * Merge the split-mode partials of paged_attn_decode (same shape, partition_size > 0):
 * for each (b, h) over its max(1, ceil(L/P)) partitions, M = max lse_p,
 * w_p = exp(lse_p - M), out = sum w_p o_p / sum w_p, lse_out = M + ln sum w_p.  Partitions with
 * lse = -inf carry no weight and their o is not read; if all are empty, out = 0, lse = -inf.
 *
 *   partials      fp32 [B][Hq][max_partitions][head_dim]   device, read
 *   lse_partials  fp32 [B][Hq][max_partitions]             device, read
 *   seq_lens      int32 [B]                                device, read (the same lengths)
 *   out           fp32 [B][Hq][head_dim]                   device, written
 *   lse_out       fp32 [B][Hq] or NULL                     device, written
 */
pa_status paged_attn_reduce(const pa_shape* shape, int32_t head_dim, const float* partials,
                            const float* lse_partials, const int32_t* seq_lens, float* out,
                            float* lse_out, void* stream);

/*
 * Balanced split-KV decode: the same operation as paged_attn_decode + paged_attn_reduce, with the
 * split placed where the work balances.  Every (sequence, KV head) is a unit of 16-token tiles
 * over its attended range; units are laid end to end and num_workers persistent one-wave workers
 * each take an equal contiguous share of all tiles, so a long sequence is split across several
 * workers and several short ones may share one.  paged_attn_decode_balanced writes every unit
 * that lies inside one worker's share to out/lse directly, and leaves partial outputs plus
 * log-sum-exps in the workspace for units cut by share boundaries; paged_attn_reduce_balanced
 * (same stream, same arguments) merges those with the log-sum-exp rule and handles empty
 * sequences.  out/lse are complete only after both calls.  Sources as for paged_attn_decode /
 * paged_attn_reduce (split-KV partitions with partial output + LSE merged by a reducer that
 * takes the output, the sequence lengths and the LSE buffer).
 *
 *   shape->partition_size and max_partitions are not used.
 *   out          fp32 [B][Hq][head_dim]      device, written
 *   lse          fp32 [B][Hq] or NULL        device, written
 *   workspace    device memory of at least paged_attn_balanced_workspace_size(...) bytes,
 *                16-byte aligned, owned by the caller; no initialisation needed.  It carries
 *                the partials from the decode call to the reduce call; calls that overlap in
 *                time must use different workspaces.
 *   num_workers  persistent workers (waves); 0 = paged_attn_balanced_default_workers(...).
 *                Both calls must resolve to the same count.
 *
 * Errors and NaN reporting as for paged_attn_decode; a workspace that is too small or misaligned
 * is PA_ERR_SHAPE.
 */
pa_status paged_attn_decode_balanced(const pa_shape* shape, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_table,
                                     const int32_t* seq_lens, float scale, int32_t head_dim,
                                     int32_t block_size, int32_t window, const float* sinks,
                                     float* out, float* lse, void* workspace,
                                     size_t workspace_bytes, int32_t num_workers, void* stream);

pa_status paged_attn_reduce_balanced(const pa_shape* shape, const int32_t* seq_lens,
                                     int32_t head_dim, int32_t block_size, int32_t window,
                                     const float* sinks, float* out, float* lse,
                                     void* workspace, size_t workspace_bytes,
                                     int32_t num_workers, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the whole balanced step, paged_attn_decode_balanced
 * followed by paged_attn_reduce_balanced, with the partials kept in a device array the library
 * holds instead of a caller workspace.  Same arguments, results and errors as those two calls
 * (out/lse complete when the stream reaches the call), minus the workspace.
 *
 *   Limit: the balanced workspace of the shape and worker count
 *   (paged_attn_balanced_workspace_size) must fit in 32 MiB, else PA_ERR_SHAPE; for example the
 *   default 2048 workers at head_dim 128 and Hq/Hkv 4 need 8.4 MB (plus 8 bytes per sequence).
 *   Allocates nothing: the array is a static device array of the library, one per GPU, which the
 *   GPU holds from the library's loading until the process ends.  Its address on the current
 *   device is looked up on the first call there (the only global state of the library).  No
 *   initialisation is needed: each call writes what it reads.  Every call on one GPU uses the
 *   same array, so calls that overlap in time on one GPU (several streams, several host threads)
 *   race and corrupt each other's results: serialise them (one stream) or use
 *   paged_attn_decode_balanced with separate workspaces.
 */
pa_status paged_attn_decode_balanced_noalloc(const pa_shape* shape, const void* q,
                                             const void* k_cache, const void* v_cache,
                                             const int32_t* block_table, const int32_t* seq_lens,
                                             float scale, int32_t head_dim, int32_t block_size,
                                             int32_t window, const float* sinks, float* out,
                                             float* lse, int32_t num_workers, void* stream);

/* Workspace bytes paged_attn_decode_balanced needs for this shape and worker count (0 = the
 * default count on the current device), or a negative pa_status. */
int64_t paged_attn_balanced_workspace_size(const pa_shape* shape, int32_t head_dim,
                                           int32_t num_workers);

/* Workers that run at once on the current device for this head_dim and Hq/Hkv (compute units
 * times resident one-wave workers per unit), or a negative pa_status.  Queries the device; does
 * not launch anything. */
int32_t paged_attn_balanced_default_workers(int32_t head_dim, int32_t group);

/* Partitions a sequence of length seq_len occupies: max(1, ceil(seq_len / partition_size));
 * 1 when partition_size == 0; -1 for a negative length or partition size. */
int32_t paged_attn_num_partitions(int32_t seq_len, int32_t partition_size);

/* Name of the kernel variant paged_attn_decode would launch for these sizes, or NULL if the
 * combination is unsupported.  The string stays valid until the next call of this function on
 * the same thread. */
const char* paged_attn_variant_name(const pa_shape* shape, int32_t head_dim, int32_t block_size);

/* Static text for a status code. */
const char* paged_attn_status_string(int32_t status);

/*
 * Host-side check of host copies of the block table and lengths against the shape: every
 * length in [0, block_table_stride * block_size], every entry a sequence reads (the first
 * ceil(L / block_size), or only those from the window start when window > 0) in
 * [0, num_blocks), and in split mode max(1, ceil(L/P)) <= max_partitions.  Returns PA_OK or
 * PA_ERR_TABLE (PA_ERR_NULL / PA_ERR_SHAPE for bad arguments).  Reads host memory only.
 */
pa_status paged_attn_check_tables(const pa_shape* shape, int32_t block_size, int32_t window,
                                  const int32_t* host_block_table,
                                  const int32_t* host_seq_lens);

/*
 * Suggested partition size for a batch: 0 (unsplit) when the batch alone fills the GPU,
 * otherwise a multiple of block_size (and of 16) sized so that roughly
 * num_seqs * num_kv_heads * partitions reaches several workgroups per compute unit.
 * max_seq_len is a host-side upper bound on the lengths; num_cus the device's CU count.
 */
int32_t paged_attn_suggest_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                          int32_t max_seq_len, int32_t block_size,
                                          int32_t num_cus);

/*
 * Prepared decode (a "plan"): every check, the variant choice and the launch geometry are done
 * once by paged_attn_plan_create; paged_attn_plan_run then only fills the pointers and launches
 * the kernels of one whole step (decode, plus the merge for a split schedule), so a step costs
 * one call with no validation, no environment lookups and no device queries.  This is the
 * small-batch latency path: at one to four sequences the device work is a few microseconds and
 * host preparation dominates, the problem ROCm/rocm-libraries PR #13700 "prepare saved paged
 * decode bindings once" (Summary, and its host-overhead measurements at B = 1 and 4) prepares
 * paged-decode bindings once for.  A run records nothing but kernel launches on `stream`, so it
 * can be captured into a HIP graph and replayed.
 *
 *   schedule       PA_SCHEDULE_UNSPLIT (one workgroup per sequence and KV head; requires
 *                  shape->partition_size == 0), PA_SCHEDULE_PARTITIONED (fixed partitions of
 *                  shape->partition_size tokens, shape->max_partitions slots, then the reduce),
 *                  PA_SCHEDULE_BALANCED (persistent workers, then the fix-up merge), or
 *                  PA_SCHEDULE_PARTITIONED_FUSED (fixed partitions as PARTITIONED, merged in
 *                  the same launch by whichever partition of a (sequence, KV head) finishes
 *                  last: one kernel per step, for small batches; its device-scope release per
 *                  partition makes it slow for large ones), or PA_SCHEDULE_QUERY_BLOCKS (one
 *                  wave per (sequence, KV head, block of 32 / (Hq/Hkv) query tokens,
 *                  16 / (Hq/Hkv) at head_dim 256), each reading the keys its tokens attend and
 *                  writing its outputs; the blocks of a (sequence, KV head) share the keys
 *                  through one XCD's L2 when num_seqs * num_kv_heads is a multiple of 8:
 *                  chunked prefill and whole prompts; requires shape->partition_size == 0.
 *                  When the batch has too few blocks to fill the GPU and max_seq_len is given,
 *                  each block's key range is cut into up to 64 key splits whose partial outputs
 *                  a merge kernel combines; the plan then needs a workspace of
 *                  B * q_len * Hq * splits * (head_dim + 1) floats (256-byte aligned sections),
 *                  and its name carries "_s<splits>".  Otherwise it needs none).
 *   kv_dtype       PA_KV_BF16, or PA_KV_FP8_E4M3: k_cache and v_cache then hold one byte per
 *                  value, [num_blocks][Hkv][block_size][head_dim] uint8, each code standing for
 *                  its E4M3 value times the tensor's scale (given per run).  The FP8 KV cache is
 *                  the sibling the one-token decode work sets aside (ROCm/rocm-libraries PR
 *                  #13700, Summary: the prepared path is the non-FP8 one); the format and the
 *                  per-tensor scales are this library's reading, the pages give none.  Every
 *                  schedule supports it; other values give PA_ERR_UNSUPPORTED.
 *   kv_layout      NULL for the default pool [num_blocks][Hkv][block_size][head_dim], else the
 *                  strides of pa_kv_layout (copied; the plan keeps no pointer to it).
 *   q_len          new query tokens per sequence, >= 1 (1 = one-token decode).  With q_len > 1
 *                  the run takes q bf16 [B][q_len][Hq][head_dim] and writes out fp32
 *                  [B][q_len][Hq][head_dim] and lse fp32 [B][q_len][Hq]; seq_lens count the new
 *                  tokens, token i of sequence b sits at position seq_lens[b] - q_len + i and
 *                  attends causally: keys t <= its position, the last `window` of them when
 *                  window > 0 (a position below 0 attends nothing: out 0, lse -inf or the sink).
 *                  This is the query length the one-token decode benchmark of ROCm/rocm-libraries
 *                  PR #13700 fixes at 1, and the longer-query case vllm.cpp PR #564 ("What is
 *                  deliberately not here") leaves out; the causal rule is this library's reading.
 *                  On the balanced schedule up to 32 (token, head) pairs per KV head share each
 *                  K/V tile (16 at head_dim 256), so with q_len * Hq/Hkv within that every K/V
 *                  row is read once per KV head for all q_len tokens; more tokens run in passes
 *                  of 32 / (Hq/Hkv) (16 / (Hq/Hkv)) tokens, each pass reading the keys its tokens
 *                  attend.  The query-block schedule runs every block of tokens at once instead.
 *                  Requires PA_SCHEDULE_BALANCED or PA_SCHEDULE_QUERY_BLOCKS (else
 *                  PA_ERR_UNSUPPORTED) and q_len <= 4096 (else PA_ERR_SHAPE); bf16 and FP8 caches
 *                  alike.
 *   max_seq_len    host-side upper bound on the lengths the plan will see, or 0 if unknown.
 *                  Balanced plans launch no more workers than that many tiles can keep busy
 *                  (a small batch then does not pay for thousands of idle workers); a length
 *                  above the bound still gives correct results, only fewer workers.
 *   num_workers    balanced only: 0 = paged_attn_balanced_default_workers (queries the current
 *                  device at creation; an FP8 plan at head_dim 128 for one query token takes
 *                  half of it, 8 per compute unit, when num_seqs * num_kv_heads is below four
 *                  per compute unit), else 1 .. 2^20.
 *   plan           receives a host-memory object owned by the caller until
 *                  paged_attn_plan_destroy.  A plan is immutable: several threads may run it at
 *                  once, each with its own workspace and outputs.
 *
 * Errors at creation are those of paged_attn_decode / paged_attn_decode_balanced for the same
 * arguments (PA_ERR_SHAPE for a schedule that does not match the shape, PA_ERR_NULL for a NULL
 * plan pointer).
 */
typedef struct pa_plan pa_plan;

/*
 * KV pool layout for plans: where the row of (physical block, KV head, slot) starts, in elements
 * of the cache's type, the same for k_cache and v_cache:
 *     block * block_stride + kv_head * head_stride + slot * token_stride
 * with the head_dim values of a row contiguous.  The default pool [num_blocks][Hkv][bs][D] is
 * (Hkv*bs*D, bs*D, D); a token-major pool [num_blocks][bs][Hkv][D] is (bs*Hkv*D, D, Hkv*D); K and
 * V interleaved per block, [num_blocks][2][Hkv][bs][D], is (2*Hkv*bs*D, bs*D, D) with v_cache
 * pointing Hkv*bs*D elements past k_cache.  Strides must be positive, token_stride >= head_dim,
 * every stride a multiple of 16 bytes, token_stride * element size <= 2^26 bytes, block and head
 * strides <= 2^40 elements (else PA_ERR_SHAPE).  The pages name a strided-KV decode mode
 * (ROCm/rocm-libraries PR #13700, its file list: a strided-KV decode document and numeric test)
 * without its layout; this descriptor is this library's reading.
 */
typedef struct {
  int64_t block_stride;
  int64_t head_stride;
  int64_t token_stride;
} pa_kv_layout;

/* KV cache element formats a plan reads. */
enum {
  PA_KV_BF16 = 0,       /* bf16 rows of head_dim values (2 * head_dim bytes)                 */
  PA_KV_FP8_E4M3 = 1    /* OCP FP8 E4M3 codes, one byte per value (head_dim bytes per row),
                           with one fp32 scale for all of K and one for all of V             */
};

enum {
  PA_SCHEDULE_UNSPLIT = 0,
  PA_SCHEDULE_PARTITIONED = 1,
  PA_SCHEDULE_BALANCED = 2,
  PA_SCHEDULE_PARTITIONED_FUSED = 3,
  PA_SCHEDULE_QUERY_BLOCKS = 4
};

/*
 * The schedule a plan for these sizes should use, from timings of every schedule on one MI355X
 * over batches of 1-128 sequences, 256-16384 keys and 4-128 query tokens (HIP-graph replay of
 * plan runs): returns a PA_SCHEDULE_* value (>= 0) and sets *partition_size to the tokens per
 * partition for PA_SCHEDULE_PARTITIONED (256, or block_size if larger), else 0.  Negative
 * pa_status for bad arguments (PA_ERR_NULL for a NULL partition_size, PA_ERR_UNSUPPORTED for a
 * head_dim or block_size no kernel takes).
 *   one query token: BALANCED when max_seq_len is 0 (unknown); UNSPLIT when the attended keys
 *     (max_seq_len, or the window if smaller) are at most 256, or at most 1024 with at least
 *     num_cus (sequence, KV head) units; PARTITIONED when units * keys <= 1024 * num_cus (little
 *     work: the small-batch latency case); BALANCED otherwise, which also absorbs any spread of
 *     lengths the bound does not show.
 *   q_len > 1: QUERY_BLOCKS above 32 (token, head) pairs per KV head (16 at head_dim 256),
 *     and from 17 (9) pairs when num_seqs * num_kv_heads > 32; BALANCED below.
 *   PA_ERR_UNSUPPORTED as well for a group Hq/Hkv no kernel takes (1, 2, 4 and 8 are built),
 *     since no plan could be created for it.
 *   num_cus: compute units of the target device, 0 = query the current device (PA_ERR_LAUNCH
 *     if there is none).  Reads nothing else; launches nothing.
 */
int32_t paged_attn_suggest_schedule(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t window,
                                    int32_t q_len, int32_t max_seq_len, int32_t num_cus,
                                    int32_t* partition_size);

pa_status paged_attn_plan_create(const pa_shape* shape, int32_t head_dim, int32_t block_size,
                                 int32_t window, int32_t schedule, int32_t kv_dtype,
                                 const pa_kv_layout* kv_layout, int32_t q_len,
                                 int32_t max_seq_len, int32_t num_workers, pa_plan** plan);

/* Plan options for paged_attn_plan_create_flags (bits). */
enum {
  /* P.V with P rounded to one bf16 term (round to nearest: |p~ - p| <= 2^-8 p) instead of the
     two terms hi + lo (|hi + lo - p| <= 2^-16 p).  Applies to the query-block schedule's 32-key
     workgroup form (bf16 caches, head_dim 64 and 128, four or more blocks of tokens per
     (sequence, KV head)); the plan name then ends in "_p1", and other plans ignore the bit.
     The softmax denominator keeps fp32 p, so an output moves by at most 2^-8 times the largest
     |v| the row attends: within the 3e-2 contract for N(0,1) values, not within 1e-3.  It
     takes a third of the P.V matrix work and the vector work of the low term away: the 512-new-
     token Llama-8B-shaped step runs about 18% faster on MI355X.  The pages give no precision for
     P (the contract is the 3e-2 tolerance with fp32 accumulation); this option is this
     library's. */
  PA_PLAN_P_ONE_BF16 = 1
};

/* paged_attn_plan_create with option bits (PA_PLAN_*); unknown bits give PA_ERR_UNSUPPORTED.
 * flags = 0 is paged_attn_plan_create. */
pa_status paged_attn_plan_create_flags(const pa_shape* shape, int32_t head_dim,
                                       int32_t block_size, int32_t window, int32_t schedule,
                                       int32_t kv_dtype, const pa_kv_layout* kv_layout,
                                       int32_t q_len, int32_t max_seq_len, int32_t num_workers,
                                       int32_t flags, pa_plan** plan);

/* Device workspace bytes a run needs (0 for the unsplit schedule): the partition partials and
 * their LSEs (plus one merge counter per (sequence, KV head) for the fused schedule), or the
 * balanced workspace.  Caller-owned and 256-byte aligned.  A fused plan's workspace must be
 * zero-filled before its first run; every run leaves its counters at zero again.  Other plans
 * need no initialisation.  Runs that overlap in time need separate workspaces. */
int64_t paged_attn_plan_workspace_size(const pa_plan* plan);

/*
 * One decode step with a plan: the operation of paged_attn_decode (+ paged_attn_reduce) on the
 * sizes fixed at creation.  Pointers, layouts and the scale / sinks / lse conventions are those
 * of paged_attn_decode; out is always the final fp32 [B][Hq][head_dim] and lse the final
 * [B][Hq] (or NULL).  k_scale and v_scale are the FP8 cache's per-tensor scales (a key is
 * k_scale times its decoded code, a value v_scale times its code); a bf16 plan requires both to
 * be 1.  Returns PA_ERR_NULL for a missing pointer (workspace included when the plan needs
 * one), PA_ERR_SHAPE for a non-finite scale, a bf16 plan given scales other than 1, or a
 * misaligned workspace, and PA_ERR_LAUNCH when HIP rejects a launch.  Bad tables and lengths are
 * reported as NaN, as for paged_attn_decode; a NaN code in an attended FP8 row gives NaN outputs
 * for that (sequence, KV head), as a NaN bf16 value does.
 */
pa_status paged_attn_plan_run(const pa_plan* plan, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, float scale, float k_scale, float v_scale,
                              const float* sinks, float* out, float* lse, void* workspace,
                              void* stream);

/* Kernel variants a run launches (static storage owned by the plan). */
const char* paged_attn_plan_name(const pa_plan* plan);

/* Frees a plan (NULL is a no-op).  No run may be in progress on the host. */
void paged_attn_plan_destroy(pa_plan* plan);

/* ABI version, bumped on any incompatible change. */
int32_t paged_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
