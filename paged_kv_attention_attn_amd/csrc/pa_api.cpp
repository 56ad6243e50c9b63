// C ABI of the paged-attention decode library: host-side validation, variant selection and
// launches.  Every check runs before any HIP call, so a rejected call touches no device state
// (and can be exercised on a machine without a GPU).  Nothing is allocated.
//
// The shape-envelope checks fail loudly instead of falling back to another path: a head size
// that silently fell to a slower kernel is the defect vllm.cpp PR #564 "spec(BACKEND-ROCM): the
// ROCm head_dim=128 decode arm" specs ("The gap it specs"), and shapes outside a native envelope
// silently taking another path is open gap 6 of randomvariable/vllm issue #23 "Attention parity".
// Split mode without an LSE buffer is an error, as an LSE request without LSE emission raises in
// ROCm/rocm-libraries PR #13700 "prepare saved paged decode bindings once", review finding N1.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/paged_attn.h"
#include "../../include/paged_attn_debug.h"
#include "pa_kernels.hpp"

namespace {

// Default pool layout [num_blocks][Hkv][block_size][D]: the three byte strides.
void set_default_layout(pa::DecodeParams& p, int32_t num_kv_heads, int32_t block_size,
                        int64_t row_bytes) {
  p.kv_row_stride = row_bytes;
  p.kv_head_stride = row_bytes * block_size;
  p.kv_block_stride = p.kv_head_stride * num_kv_heads;
}

}  // namespace

namespace {

constexpr int32_t kAbiVersion = 5;
#ifndef PA_HEAD_PAIRS
#define PA_HEAD_PAIRS 1
#endif
constexpr bool kHeadPairs = PA_HEAD_PAIRS != 0;
#ifndef PA_HEAD_PAIRS_FP8
#define PA_HEAD_PAIRS_FP8 1
#endif
constexpr bool kHeadPairsFp8 = PA_HEAD_PAIRS_FP8 != 0;
constexpr int32_t kMaxGridYZ = 65535;

int log2_exact(int32_t v) {
  if (v <= 0 || (v & (v - 1)) != 0) return -1;
  int k = 0;
  while ((1 << k) < v) ++k;
  return k;
}

bool block_size_ok(int32_t bs) { return bs == 16 || bs == 32 || bs == 64 || bs == 128 || bs == 256; }

bool head_dim_ok(int32_t d) { return d == 64 || d == 128 || d == 256; }

pa_status check_shape(const pa_shape* s) {
  if (s == nullptr) return PA_ERR_NULL;
  if (s->num_seqs < 0 || s->num_q_heads < 1 || s->num_kv_heads < 1 || s->num_blocks < 1 ||
      s->block_table_stride < 1 || s->partition_size < 0)
    return PA_ERR_SHAPE;
  if (s->num_q_heads % s->num_kv_heads != 0) return PA_ERR_SHAPE;
  if (s->num_seqs > kMaxGridYZ || s->num_kv_heads > kMaxGridYZ) return PA_ERR_SHAPE;
  if (s->partition_size > 0 && (s->partition_size % 16 != 0 || s->max_partitions < 1))
    return PA_ERR_SHAPE;
  // decode grid: (partition slots) x Hkv x B workgroups in one dimension
  const int64_t slots = s->partition_size > 0 ? s->max_partitions : 1;
  if (slots * s->num_kv_heads * (int64_t)s->num_seqs > 0x7FFFFFFF) return PA_ERR_SHAPE;
  return PA_OK;
}

// Waves per decode workgroup: the library's choice, or PA_DECODE_WAVES (exactly "1", "2", "4"
// or "8") for tuning runs.  Any other value of the variable is rejected, not ignored.
int decode_waves(int head_dim, int group, int psize) {
  const char* v = std::getenv("PA_DECODE_WAVES");
  if (v == nullptr) return pa::decode_default_waves(head_dim, group, psize);
  if (v[0] != '\0' && v[1] == '\0' && pa::decode_waves_supported(v[0] - '0')) return v[0] - '0';
  return -1;
}

// Score path: the library's choice, or PA_DECODE_PATH (exactly "valu", "mfma" or "mfma_pv")
// for tuning and for testing every path.  Any other value is rejected.
int decode_path(int head_dim, int group, pa::QkPath* out) {
  const char* v = std::getenv("PA_DECODE_PATH");
  if (v == nullptr) {
    *out = pa::decode_default_path(head_dim, group);
    return 0;
  }
  if (std::strcmp(v, "valu") == 0) {
    *out = pa::QkPath::kValu;
    return 0;
  }
  if (std::strcmp(v, "mfma") == 0) {
    *out = pa::QkPath::kMfma;
    return 0;
  }
  if (std::strcmp(v, "mfma_pv") == 0) {
    *out = pa::QkPath::kMfmaPv;
    return 0;
  }
  return -1;
}

bool debug_log() {
  static const int on = [] {
    const char* v = std::getenv("PA_LOG");
    return (v != nullptr && v[0] == '1' && v[1] == '\0') ? 1 : 0;
  }();
  return on != 0;
}

}  // namespace

extern "C" {

int32_t paged_attn_abi_version(void) { return kAbiVersion; }

const char* paged_attn_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "sizes inconsistent or out of range";
    case PA_ERR_UNSUPPORTED: return "head_dim / group / block_size combination not supported";
    case PA_ERR_LSE_REQUIRED: return "split mode requires an lse buffer";
    case PA_ERR_LAUNCH: return "HIP launch failed";
    case PA_ERR_TABLE: return "block table or sequence lengths out of range";
    default: return "unknown status";
  }
}

int32_t paged_attn_num_partitions(int32_t seq_len, int32_t partition_size) {
  if (seq_len < 0 || partition_size < 0) return -1;
  if (partition_size == 0 || seq_len == 0) return 1;
  return (int32_t)(((int64_t)seq_len + partition_size - 1) / partition_size);
}

const char* paged_attn_variant_name(const pa_shape* shape, int32_t head_dim, int32_t block_size) {
  if (check_shape(shape) != PA_OK || !head_dim_ok(head_dim) || !block_size_ok(block_size))
    return nullptr;
  const int group = shape->num_q_heads / shape->num_kv_heads;
  if (!pa::decode_supported(head_dim, group)) return nullptr;
  const int waves = decode_waves(head_dim, group, shape->partition_size);
  pa::QkPath path;
  if (waves < 0 || decode_path(head_dim, group, &path) != 0) return nullptr;
  return pa::decode_variant_name(head_dim, group, waves, shape->partition_size > 0, path);
}

pa_status paged_attn_decode(const pa_shape* shape, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            const int32_t* seq_lens, float scale, int32_t head_dim,
                            int32_t block_size, int32_t window, const float* sinks, float* out,
                            float* lse, void* stream) {
  const pa_status st = check_shape(shape);
  if (st != PA_OK) return st;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  const int group = shape->num_q_heads / shape->num_kv_heads;
  if (!pa::decode_supported(head_dim, group)) return PA_ERR_UNSUPPORTED;
  if (window < 0 || !std::isfinite(scale)) return PA_ERR_SHAPE;
  const bool split = shape->partition_size > 0;
  if (split && lse == nullptr) return PA_ERR_LSE_REQUIRED;
  const int waves = decode_waves(head_dim, group, shape->partition_size);
  pa::QkPath path;
  if (waves < 0 || decode_path(head_dim, group, &path) != 0) return PA_ERR_UNSUPPORTED;
  if (shape->num_seqs == 0) return PA_OK;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || block_table == nullptr ||
      seq_lens == nullptr || out == nullptr)
    return PA_ERR_NULL;

  pa::DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k_cache = static_cast<const char*>(k_cache);
  p.v_cache = static_cast<const char*>(v_cache);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.sinks = sinks;
  p.out = out;
  p.lse = lse;
  p.qk_scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.v_scale = 1.f;
  p.num_seqs = shape->num_seqs;
  p.num_q_heads = shape->num_q_heads;
  p.num_kv_heads = shape->num_kv_heads;
  p.num_blocks = shape->num_blocks;
  p.stride = shape->block_table_stride;
  p.bs_log2 = log2_exact(block_size);
  p.window = window;
  p.psize = shape->partition_size;
  p.max_parts = split ? shape->max_partitions : 1;
  p.q_len = 1;
  p.q_total = 1;
  p.q_first = 0;
  p.group = group;
  set_default_layout(p, shape->num_kv_heads, block_size, 2 * (int64_t)head_dim);
  if (debug_log())
    std::fprintf(stderr, "[paged_attn] decode %s B=%d Hq=%d Hkv=%d bs=%d P=%d Pmax=%d W=%d\n",
                 pa::decode_variant_name(head_dim, group, waves, split, path), shape->num_seqs,
                 shape->num_q_heads, shape->num_kv_heads, block_size, p.psize, p.max_parts,
                 window);
  const hipError_t e =
      pa::launch_decode(p, head_dim, group, waves, path, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

namespace {

constexpr int32_t kMaxWorkers = 1 << 20;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// workspace layout: prefix int64 [B+1] | lse fp32 [N][2][G] | o fp32 [N][2][G][D]
struct WsLayout {
  size_t prefix, lse, o, total;
};

WsLayout ws_layout(int32_t num_seqs, int32_t group, int32_t head_dim, int32_t workers) {
  WsLayout l;
  l.prefix = 0;
  l.lse = align256(((size_t)num_seqs + 1) * sizeof(int64_t));
  l.o = l.lse + align256((size_t)workers * 2 * group * sizeof(float));
  l.total = l.o + align256((size_t)workers * 2 * group * head_dim * sizeof(float));
  return l;
}

}  // namespace

int32_t paged_attn_balanced_default_workers(int32_t head_dim, int32_t group) {
  if (!head_dim_ok(head_dim) || !pa::decode_supported(head_dim, group)) return PA_ERR_UNSUPPORTED;
  pa::QkPath path;
  if (decode_path(head_dim, group, &path) != 0) return PA_ERR_UNSUPPORTED;
  const int n = pa::balanced_default_workers(head_dim, group, path);
  return n > 0 ? n : PA_ERR_LAUNCH;
}

int64_t paged_attn_balanced_workspace_size(const pa_shape* shape, int32_t head_dim,
                                           int32_t num_workers) {
  const pa_status st = check_shape(shape);
  if (st != PA_OK) return st;
  const int group = shape->num_q_heads / shape->num_kv_heads;
  if (!head_dim_ok(head_dim) || !pa::decode_supported(head_dim, group)) return PA_ERR_UNSUPPORTED;
  if (num_workers < 0 || num_workers > kMaxWorkers) return PA_ERR_SHAPE;
  if (num_workers == 0) {
    num_workers = paged_attn_balanced_default_workers(head_dim, group);
    if (num_workers < 0) return num_workers;
  }
  return (int64_t)ws_layout(shape->num_seqs, group, head_dim, num_workers).total;
}

// Validation and parameter block shared by the two balanced calls; returns PA_OK and fills bp,
// or the status to return.  q/k/v/table may be null for the reduce call (not used there).
pa_status balanced_setup(const pa_shape* shape, int32_t head_dim, int32_t block_size,
                         int32_t window, const int32_t* seq_lens, const float* sinks, float* out,
                         float* lse, void* workspace, size_t workspace_bytes,
                         int32_t num_workers, pa::BalancedParams* bp, pa::QkPath* path,
                         int* group_out) {
  const pa_status st = check_shape(shape);
  if (st != PA_OK) return st;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  const int group = shape->num_q_heads / shape->num_kv_heads;
  if (!pa::decode_supported(head_dim, group)) return PA_ERR_UNSUPPORTED;
  if (window < 0) return PA_ERR_SHAPE;
  if (num_workers < 0 || num_workers > kMaxWorkers) return PA_ERR_SHAPE;
  if ((int64_t)shape->num_seqs * shape->num_q_heads > 0x7FFFFFFF) return PA_ERR_SHAPE;
  if (decode_path(head_dim, group, path) != 0) return PA_ERR_UNSUPPORTED;
  *group_out = group;
  if (shape->num_seqs == 0) return PA_OK;
  if (seq_lens == nullptr || out == nullptr || workspace == nullptr) return PA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return PA_ERR_SHAPE;
  if (num_workers == 0) {
    num_workers = pa::balanced_default_workers(head_dim, group, *path);
    if (num_workers <= 0) return PA_ERR_LAUNCH;
  }
  const WsLayout wl = ws_layout(shape->num_seqs, group, head_dim, num_workers);
  if (workspace_bytes < wl.total) return PA_ERR_SHAPE;
  pa::DecodeParams& p = bp->d;
  p.seq_lens = seq_lens;
  p.sinks = sinks;
  p.out = out;
  p.lse = lse;
  p.num_seqs = shape->num_seqs;
  p.num_q_heads = shape->num_q_heads;
  p.num_kv_heads = shape->num_kv_heads;
  p.num_blocks = shape->num_blocks;
  p.stride = shape->block_table_stride;
  p.bs_log2 = log2_exact(block_size);
  p.window = window;
  p.psize = 0;
  p.max_parts = 1;
  p.q_len = 1;
  p.q_total = 1;
  p.q_first = 0;
  p.group = group;
  set_default_layout(p, shape->num_kv_heads, block_size, 2 * (int64_t)head_dim);
  char* ws = static_cast<char*>(workspace);
  bp->prefix = reinterpret_cast<int64_t*>(ws + wl.prefix);
  bp->ws_lse = reinterpret_cast<float*>(ws + wl.lse);
  bp->ws_o = reinterpret_cast<float*>(ws + wl.o);
  bp->num_workers = num_workers;
  return PA_OK;
}

pa_status paged_attn_decode_balanced(const pa_shape* shape, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_table,
                                     const int32_t* seq_lens, float scale, int32_t head_dim,
                                     int32_t block_size, int32_t window, const float* sinks,
                                     float* out, float* lse, void* workspace,
                                     size_t workspace_bytes, int32_t num_workers, void* stream) {
  if (!std::isfinite(scale)) {
    const pa_status st = check_shape(shape);
    return st != PA_OK ? st : PA_ERR_SHAPE;
  }
  pa::BalancedParams bp{};
  pa::QkPath path;
  int group = 0;
  const pa_status st = balanced_setup(shape, head_dim, block_size, window, seq_lens, sinks, out,
                                      lse, workspace, workspace_bytes, num_workers, &bp, &path,
                                      &group);
  if (st != PA_OK || shape->num_seqs == 0) return st;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || block_table == nullptr)
    return PA_ERR_NULL;
  pa::DecodeParams& p = bp.d;
  p.q = static_cast<const uint16_t*>(q);
  p.k_cache = static_cast<const char*>(k_cache);
  p.v_cache = static_cast<const char*>(v_cache);
  p.block_table = block_table;
  p.qk_scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.v_scale = 1.f;
  if (debug_log())
    std::fprintf(stderr, "[paged_attn] balanced %s B=%d Hq=%d Hkv=%d bs=%d W=%d workers=%d\n",
                 pa::qk_path_name(path), shape->num_seqs,
                 shape->num_q_heads, shape->num_kv_heads, block_size, window, bp.num_workers);
  const hipError_t e =
      pa::launch_balanced(bp, head_dim, group, path, false, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status paged_attn_reduce_balanced(const pa_shape* shape, const int32_t* seq_lens,
                                     int32_t head_dim, int32_t block_size, int32_t window,
                                     const float* sinks, float* out, float* lse,
                                     void* workspace, size_t workspace_bytes,
                                     int32_t num_workers, void* stream) {
  pa::BalancedParams bp{};
  pa::QkPath path;
  int group = 0;
  const pa_status st = balanced_setup(shape, head_dim, block_size, window, seq_lens, sinks, out,
                                      lse, workspace, workspace_bytes, num_workers, &bp, &path,
                                      &group);
  if (st != PA_OK || shape->num_seqs == 0) return st;
  const hipError_t e =
      pa::launch_balanced_fixup(bp, head_dim, group, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// The balanced step without a caller workspace: the partials live in a device array of the
// library, one per GPU (each GPU holds its own copy of a __device__ array, at its own address).
// Host code never passes the array's name to a kernel (on the host it only stands in for the
// symbol); each device's address is looked up once, with that device current, and kept.
// ---------------------------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's scratch array, looked up on the first call per device.
pa_status current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
    return PA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return PA_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status paged_attn_decode_balanced_noalloc(const pa_shape* shape, const void* q,
                                             const void* k_cache, const void* v_cache,
                                             const int32_t* block_table, const int32_t* seq_lens,
                                             float scale, int32_t head_dim, int32_t block_size,
                                             int32_t window, const float* sinks, float* out,
                                             float* lse, int32_t num_workers, void* stream) {
  if (!std::isfinite(scale)) {
    const pa_status st = check_shape(shape);
    return st != PA_OK ? st : PA_ERR_SHAPE;
  }
  // every check first, against a stand-in of the scratch array's size and alignment (nothing is
  // read through it); the array's device address only once they pass
  pa::BalancedParams bp{};
  pa::QkPath path;
  int group = 0;
  void* ws = reinterpret_cast<void*>((uintptr_t)256);
  pa_status st = balanced_setup(shape, head_dim, block_size, window, seq_lens, sinks, out, lse,
                                ws, kScratchBytes, num_workers, &bp, &path, &group);
  if (st != PA_OK || shape->num_seqs == 0) return st;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || block_table == nullptr)
    return PA_ERR_NULL;
  st = current_scratch(&ws);
  if (st != PA_OK) return st;
  st = balanced_setup(shape, head_dim, block_size, window, seq_lens, sinks, out, lse, ws,
                      kScratchBytes, bp.num_workers, &bp, &path, &group);
  if (st != PA_OK) return st;
  pa::DecodeParams& p = bp.d;
  p.q = static_cast<const uint16_t*>(q);
  p.k_cache = static_cast<const char*>(k_cache);
  p.v_cache = static_cast<const char*>(v_cache);
  p.block_table = block_table;
  p.qk_scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.v_scale = 1.f;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = pa::launch_balanced(bp, head_dim, group, path, false, hs);
  if (e == hipSuccess) e = pa::launch_balanced_fixup(bp, head_dim, group, hs);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status paged_attn_reduce(const pa_shape* shape, int32_t head_dim, const float* partials,
                            const float* lse_partials, const int32_t* seq_lens, float* out,
                            float* lse_out, void* stream) {
  const pa_status st = check_shape(shape);
  if (st != PA_OK) return st;
  if (!head_dim_ok(head_dim)) return PA_ERR_UNSUPPORTED;
  if (shape->partition_size <= 0) return PA_ERR_SHAPE;
  if (shape->num_q_heads > kMaxGridYZ * 32) return PA_ERR_SHAPE;
  if (shape->num_seqs == 0) return PA_OK;
  if (partials == nullptr || lse_partials == nullptr || seq_lens == nullptr || out == nullptr)
    return PA_ERR_NULL;
  pa::ReduceParams p{};
  p.partials = partials;
  p.lse_partials = lse_partials;
  p.seq_lens = seq_lens;
  p.out = out;
  p.lse = lse_out;
  p.num_q_heads = shape->num_q_heads;
  p.psize = shape->partition_size;
  p.max_parts = shape->max_partitions;
  const hipError_t e = pa::launch_reduce(p, head_dim, shape->num_seqs,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status paged_attn_check_tables(const pa_shape* shape, int32_t block_size, int32_t window,
                                  const int32_t* host_block_table, const int32_t* host_seq_lens) {
  const pa_status st = check_shape(shape);
  if (st != PA_OK) return st;
  if (!block_size_ok(block_size) || window < 0) return PA_ERR_SHAPE;
  if (shape->num_seqs == 0) return PA_OK;
  if (host_block_table == nullptr || host_seq_lens == nullptr) return PA_ERR_NULL;
  const int64_t cap = (int64_t)shape->block_table_stride * block_size;
  for (int32_t b = 0; b < shape->num_seqs; ++b) {
    const int32_t L = host_seq_lens[b];
    if (L < 0 || L > cap) return PA_ERR_TABLE;
    if (shape->partition_size > 0 &&
        paged_attn_num_partitions(L, shape->partition_size) > shape->max_partitions)
      return PA_ERR_TABLE;
    const int32_t start = (window > 0 && L > window) ? L - window : 0;
    if (L == 0) continue;
    const int32_t first = start / block_size;
    const int32_t last = (L - 1) / block_size;
    const int32_t* row = host_block_table + (size_t)b * shape->block_table_stride;
    for (int32_t i = first; i <= last; ++i)
      if (row[i] < 0 || row[i] >= shape->num_blocks) return PA_ERR_TABLE;
  }
  return PA_OK;
}

int32_t paged_attn_suggest_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                          int32_t max_seq_len, int32_t block_size,
                                          int32_t num_cus) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || max_seq_len <= 0 || num_cus <= 0 ||
      !block_size_ok(block_size))
    return 0;
  // Aim for about 16 partition workgroups per CU, with partitions of 256..2048 tokens that are
  // multiples of the block size; batches that already fill the GPU and are short stay unsplit.
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  const int64_t want = (int64_t)num_cus * 16;
  if (units >= want && max_seq_len <= 1024) return 0;
  int64_t parts = (want + units - 1) / units;
  int64_t P = ((int64_t)max_seq_len + parts - 1) / parts;
  if (P < 256) P = 256;
  if (P > 2048) P = 2048;
  const int64_t unit = block_size > 16 ? block_size : 16;
  P = ((P + unit - 1) / unit) * unit;
  return (int32_t)P;
}

pa_status paged_attn_gather_witness(const pa_shape* shape, const void* k_cache,
                                    const void* v_cache, const int32_t* block_table,
                                    const int32_t* seq_lens, int32_t head_dim,
                                    int32_t block_size, int32_t window, int32_t max_rows,
                                    void* k_rows, void* v_rows, void* stream) {
  const pa_status st = check_shape(shape);
  if (st != PA_OK) return st;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (window < 0 || max_rows < 1) return PA_ERR_SHAPE;
  if (shape->num_seqs == 0) return PA_OK;
  if (k_cache == nullptr || v_cache == nullptr || block_table == nullptr ||
      seq_lens == nullptr || k_rows == nullptr || v_rows == nullptr)
    return PA_ERR_NULL;
  pa::WitnessParams p{};
  p.k_cache = static_cast<const char*>(k_cache);
  p.v_cache = static_cast<const char*>(v_cache);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.k_rows = static_cast<char*>(k_rows);
  p.v_rows = static_cast<char*>(v_rows);
  p.num_kv_heads = shape->num_kv_heads;
  p.num_blocks = shape->num_blocks;
  p.stride = shape->block_table_stride;
  p.bs_log2 = log2_exact(block_size);
  p.window = window;
  p.max_rows = max_rows;
  const hipError_t e = pa::launch_witness(p, head_dim, shape->num_seqs,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status paged_attn_stream_read(const void* buf, size_t bytes, int32_t num_workgroups,
                                 uint32_t* sink, void* stream) {
  if (buf == nullptr || sink == nullptr) return PA_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0 || num_workgroups < 1) return PA_ERR_SHAPE;
  const hipError_t e = pa::launch_stream_read(buf, bytes, num_workgroups, sink,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status paged_attn_gather_read(const void* buf, size_t bytes, int32_t chunk_bytes,
                                 const int32_t* chunk_ids, int64_t num_ids,
                                 int32_t num_workgroups, uint32_t* sink, void* stream) {
  if (buf == nullptr || sink == nullptr || (chunk_ids == nullptr && num_ids > 0))
    return PA_ERR_NULL;
  if (chunk_bytes != 2048 && chunk_bytes != 4096 && chunk_bytes != 8192) return PA_ERR_SHAPE;
  if (bytes < (size_t)chunk_bytes || num_ids < 0 || num_workgroups < 1) return PA_ERR_SHAPE;
  if (num_ids == 0) return PA_OK;
  const hipError_t e = pa::launch_gather_read(
      buf, (int64_t)(bytes / (size_t)chunk_bytes), chunk_bytes, chunk_ids, num_ids,
      num_workgroups, sink, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status paged_attn_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (dst == nullptr || src == nullptr) return PA_ERR_NULL;
  if (bytes % 16 != 0) return PA_ERR_SHAPE;
  const hipError_t e = pa::launch_copy(dst, src, bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// Prepared decode (plans)
// ---------------------------------------------------------------------------------------------
struct pa_plan {
  int32_t schedule;
  int32_t kv_dtype;
  int32_t head_dim;
  int32_t group;          // kernel columns: Hq/Hkv, or (q_len > 1) q_len*Hq/Hkv rounded up to 2^k
  int32_t waves, num_workers;
  int32_t q_len;          // query tokens per sequence
  int32_t pass_tokens;    // tokens per launch pair (all of them unless q_len * Hq/Hkv > 16)
  pa::QkPath path;
  pa::DecodeParams dec;   // sizes; pointers are filled per run
  pa::ReduceParams red;   // partitioned schedule: sizes
  size_t part_bytes;      // partitioned: partials, then their LSEs
  size_t counter_off;     // fused: merge counters [B][Hkv] after the LSEs
  WsLayout bal;           // balanced workspace layout
  pa::QBlockParams qb;    // query-block grid: geometry (pointers filled per run)
  int64_t workspace_bytes;
  char name[128];
};

namespace {

// (query token, head) pairs per KV head one kernel holds: 32 (two 16-column halves sharing the
// tile) at head_dim <= 128, 16 at 256
int32_t max_columns(int32_t head_dim) { return head_dim <= 128 ? 32 : 16; }
constexpr int32_t kMaxQueryTokens = 4096;

// Largest row stride in bytes: 16 rows of a tile stay within 32-bit lane offsets.
constexpr int64_t kMaxRowStrideBytes = int64_t(1) << 26;

// The pool layout's byte strides in p: the default [num_blocks][Hkv][bs][D] for a NULL layout,
// else the given strides (elements of `elem` bytes), each row 16-byte aligned and rows of a block
// at least a row apart.
pa_status apply_kv_layout(pa::DecodeParams& p, const pa_kv_layout* kv_layout,
                          int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                          int64_t elem) {
  set_default_layout(p, num_kv_heads, block_size, elem * head_dim);
  if (kv_layout == nullptr) return PA_OK;
  const int64_t bsb = kv_layout->block_stride * elem, hsb = kv_layout->head_stride * elem,
                rsb = kv_layout->token_stride * elem;
  if (kv_layout->block_stride <= 0 || kv_layout->head_stride <= 0 ||
      kv_layout->token_stride < head_dim || rsb > kMaxRowStrideBytes ||
      kv_layout->block_stride > (int64_t(1) << 40) || kv_layout->head_stride > (int64_t(1) << 40))
    return PA_ERR_SHAPE;
  if (bsb % 16 != 0 || hsb % 16 != 0 || rsb % 16 != 0) return PA_ERR_SHAPE;
  p.kv_block_stride = bsb;
  p.kv_head_stride = hsb;
  p.kv_row_stride = rsb;
  return PA_OK;
}

pa_status plan_build(const pa_shape* shape, int32_t head_dim, int32_t block_size, int32_t window,
                     int32_t schedule, int32_t kv_dtype, const pa_kv_layout* kv_layout,
                     int32_t q_len, int32_t max_seq_len, int32_t num_workers, int32_t flags,
                     pa_plan* pl) {
  const pa_status st = check_shape(shape);
  if (st != PA_OK) return st;
  if ((flags & ~PA_PLAN_P_ONE_BF16) != 0) return PA_ERR_UNSUPPORTED;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  const int group = shape->num_q_heads / shape->num_kv_heads;
  if (!pa::decode_supported(head_dim, group)) return PA_ERR_UNSUPPORTED;
  if (window < 0 || max_seq_len < 0) return PA_ERR_SHAPE;
  if (schedule == PA_SCHEDULE_UNSPLIT && shape->partition_size != 0) return PA_ERR_SHAPE;
  const bool parted =
      schedule == PA_SCHEDULE_PARTITIONED || schedule == PA_SCHEDULE_PARTITIONED_FUSED;
  if (parted && shape->partition_size <= 0) return PA_ERR_SHAPE;
  const bool qblocks = schedule == PA_SCHEDULE_QUERY_BLOCKS;
  if (!parted && !qblocks && schedule != PA_SCHEDULE_UNSPLIT && schedule != PA_SCHEDULE_BALANCED)
    return PA_ERR_SHAPE;
  if (qblocks && shape->partition_size != 0) return PA_ERR_SHAPE;
  if (parted && shape->num_q_heads > kMaxGridYZ * 32) return PA_ERR_SHAPE;
  if (schedule == PA_SCHEDULE_BALANCED &&
      ((int64_t)shape->num_seqs * shape->num_q_heads > 0x7FFFFFFF || num_workers < 0 ||
       num_workers > kMaxWorkers))
    return PA_ERR_SHAPE;
  if (kv_dtype != PA_KV_BF16 && kv_dtype != PA_KV_FP8_E4M3) return PA_ERR_UNSUPPORTED;
  if (q_len < 1 || q_len > kMaxQueryTokens) return PA_ERR_SHAPE;
  int32_t columns = group;
  int32_t pass_tokens = q_len;
  if (qblocks) {
    // query blocks: one wave per (sequence, KV head, max_columns / group tokens)
    if (group > max_columns(head_dim)) return PA_ERR_UNSUPPORTED;
    if ((int64_t)shape->num_seqs * q_len * shape->num_q_heads > 0x7FFFFFFF) return PA_ERR_SHAPE;
    if (window > 0x7FFFFFFF - max_columns(head_dim)) return PA_ERR_SHAPE;
  } else if (q_len > 1) {
    // several query tokens: the balanced schedule, (token, head) columns on the matrix cores;
    // more tokens than 16 columns hold run in passes of 16 / group tokens, each reading the KV
    if (schedule != PA_SCHEDULE_BALANCED) return PA_ERR_UNSUPPORTED;
    if ((int64_t)shape->num_seqs * q_len * shape->num_q_heads > 0x7FFFFFFF) return PA_ERR_SHAPE;
    if ((int64_t)q_len * group > max_columns(head_dim))
      pass_tokens = max_columns(head_dim) / group;
    if (window > 0x7FFFFFFF - pass_tokens) return PA_ERR_SHAPE;
    columns = 1;
    while (columns < pass_tokens * group) columns *= 2;
  }
  pa::QkPath path;
  if (kv_dtype == PA_KV_FP8_E4M3)
    path = pa::QkPath::kMfmaPvFp8;   // the one path that reads FP8 rows
  else if (q_len > 1 || qblocks)
    path = pa::QkPath::kMfmaPv;      // the one path with column-wise query tokens
  else if (decode_path(head_dim, group, &path) != 0)
    return PA_ERR_UNSUPPORTED;
  const int waves = decode_waves(head_dim, group, parted ? shape->partition_size : 0);
  if (waves < 0) return PA_ERR_UNSUPPORTED;

  pl->schedule = schedule;
  pl->kv_dtype = kv_dtype;
  pl->head_dim = head_dim;
  pl->group = columns;
  pl->q_len = q_len;
  pl->pass_tokens = pass_tokens;
  pl->waves = waves;
  pl->path = path;
  pl->num_workers = 0;
  pl->part_bytes = 0;
  pl->counter_off = 0;
  pl->workspace_bytes = 0;
  pa::DecodeParams& p = pl->dec;
  p = pa::DecodeParams{};
  p.num_seqs = shape->num_seqs;
  p.num_q_heads = shape->num_q_heads;
  p.num_kv_heads = shape->num_kv_heads;
  p.num_blocks = shape->num_blocks;
  p.stride = shape->block_table_stride;
  p.bs_log2 = log2_exact(block_size);
  p.window = window;
  p.psize = parted ? shape->partition_size : 0;
  p.max_parts = parted ? shape->max_partitions : 1;
  p.q_len = pass_tokens;
  p.q_total = q_len;
  p.q_first = 0;
  p.group = group;
  const int64_t elem = kv_dtype == PA_KV_FP8_E4M3 ? 1 : 2;
  if (apply_kv_layout(p, kv_layout, shape->num_kv_heads, block_size, head_dim, elem) != PA_OK)
    return PA_ERR_SHAPE;
  pl->red = pa::ReduceParams{};
  const char* dname = pa::decode_variant_name(head_dim, group, waves, parted, path);
  if (schedule == PA_SCHEDULE_UNSPLIT) {
    std::snprintf(pl->name, sizeof(pl->name), "%s", dname);
  } else if (qblocks) {
    pl->qb = pa::QBlockParams{};
    pl->qb.d = p;
    pa::qblock_geometry(pl->qb, head_dim, max_seq_len);
    // one bf16 term of P where the 32-key workgroup form runs (bf16 caches, head_dim <= 128)
    pl->qb.p_one_term = (flags & PA_PLAN_P_ONE_BF16) != 0 && pl->qb.waves > 1 &&
                                path != pa::QkPath::kMfmaPvFp8 && head_dim <= 128
                            ? 1
                            : 0;
    pl->group = pa::qblock_columns(head_dim);
    if (pl->qb.splits > 1) {
      // key splits: normalised partial outputs, then their LSEs
      const size_t slots = (size_t)shape->num_seqs * q_len * shape->num_q_heads * pl->qb.splits;
      pl->part_bytes = align256(slots * head_dim * sizeof(float));
      pl->workspace_bytes = (int64_t)(pl->part_bytes + align256(slots * sizeof(float)));
    }
    char splits[16] = "";
    if (pl->qb.splits > 1) std::snprintf(splits, sizeof(splits), "_s%d", pl->qb.splits);
    std::snprintf(pl->name, sizeof(pl->name), "pa_qblock_%s_d%d_g%d_q%d_t%d_w%d%s%s%s",
                  pa::qk_path_name(path), head_dim, group, q_len, pl->qb.tokens_per_block,
                  pl->qb.waves, splits, pl->qb.xcd_pinned ? "_xcd" : "",
                  pl->qb.p_one_term ? "_p1" : "");
  } else if (schedule == PA_SCHEDULE_PARTITIONED) {
    const size_t rows = (size_t)shape->num_seqs * shape->num_q_heads * shape->max_partitions;
    pl->part_bytes = align256(rows * head_dim * sizeof(float));
    pl->workspace_bytes = (int64_t)(pl->part_bytes + align256(rows * sizeof(float)));
    pl->red.num_q_heads = shape->num_q_heads;
    pl->red.psize = shape->partition_size;
    pl->red.max_parts = shape->max_partitions;
    std::snprintf(pl->name, sizeof(pl->name), "%s + pa_reduce_d%d", dname, head_dim);
  } else if (schedule == PA_SCHEDULE_PARTITIONED_FUSED) {
    const size_t rows = (size_t)shape->num_seqs * shape->num_q_heads * shape->max_partitions;
    pl->part_bytes = align256(rows * head_dim * sizeof(float));
    pl->counter_off = pl->part_bytes + align256(rows * sizeof(float));
    pl->workspace_bytes = (int64_t)(pl->counter_off +
                                    align256((size_t)shape->num_seqs * shape->num_kv_heads * 4));
    std::snprintf(pl->name, sizeof(pl->name), "%s + merge by the last partition", dname);
  } else {
    // KV-head pairs: with one query token, an even number of KV heads and 2 or 4 query heads
    // per KV head, a unit is two adjacent KV heads (the kernels see half the KV heads, twice
    // the group, a doubled head stride and the pair's second head one head stride after its
    // first), so that each step streams both heads' 16-token tiles (4 KiB of K per head pair
    // at head_dim 64 instead of 2).  Measured (decode µs, pairs against single heads): head_dim
    // 64 on the B32 L8192 sweep point, bf16 91.3 against 97.3, FP8 50.9 against 52.9; at
    // head_dim 128 no gain on the Llama-8B-shaped step (bf16 110.0 / 110.5, FP8 62.9 / 62.6)
    // and a loss on the mixed batch (bf16 208 / 202, FP8 111.4 / 109.7), so pairs only at 64.
    const bool pair_bf16 = kHeadPairs && path == pa::QkPath::kMfmaPv;
    const bool pair_fp8 = kHeadPairsFp8 && path == pa::QkPath::kMfmaPvFp8;
    if ((pair_bf16 || pair_fp8) && q_len == 1 && shape->num_kv_heads % 2 == 0 && group >= 2 &&
        group <= 4 && head_dim == 64) {
      path = pair_fp8 ? pa::QkPath::kMfmaPvFp8Heads2 : pa::QkPath::kMfmaPvHeads2;
      pl->path = path;
      columns = 2 * group;
      pl->group = columns;
      p.num_kv_heads = shape->num_kv_heads / 2;
      p.group = columns;
      p.kv_pair_off = p.kv_head_stride;
      p.kv_head_stride *= 2;
    }
    if (num_workers == 0) {
      num_workers = pa::balanced_default_workers(head_dim, columns, path, q_len > 1,
                                                  (int64_t)shape->num_seqs * p.num_kv_heads);
      if (num_workers <= 0) return PA_ERR_LAUNCH;
    }
    if (max_seq_len > 0) {
      // at most this many 16-token tiles (a window start may add one), four per worker; the
      // query tokens' windows together span window + q_len - 1 keys
      const int64_t wspan = window > 0 ? (int64_t)window + pass_tokens - 1 : 0;
      const int64_t span = wspan > 0 && wspan < max_seq_len ? wspan : max_seq_len;
      const int64_t tiles = (int64_t)shape->num_seqs * p.num_kv_heads * ((span + 15) / 16 + 1);
      const int64_t cap = (tiles + 3) / 4;
      if (cap < num_workers) num_workers = (int32_t)(cap < 1 ? 1 : cap);
    }
    pl->num_workers = num_workers;
    pl->bal = ws_layout(shape->num_seqs, columns, head_dim, num_workers);
    pl->workspace_bytes = (int64_t)pl->bal.total;
    char qtag[48] = "";
    const int32_t passes = (q_len + pass_tokens - 1) / pass_tokens;
    if (passes > 1)
      std::snprintf(qtag, sizeof(qtag), "_q%d_c%d_passes%d", q_len, columns, passes);
    else if (q_len > 1)
      std::snprintf(qtag, sizeof(qtag), "_q%d_c%d", q_len, columns);
    std::snprintf(pl->name, sizeof(pl->name), "pa_balanced_%s_d%d_g%d%s_workers%d + fixup",
                  pa::qk_path_name(path), head_dim, group, qtag, num_workers);
  }
  return PA_OK;
}

}  // namespace

extern "C" {

int32_t paged_attn_suggest_schedule(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t window,
                                    int32_t q_len, int32_t max_seq_len, int32_t num_cus,
                                    int32_t* partition_size) {
  if (partition_size == nullptr) return PA_ERR_NULL;
  *partition_size = 0;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      window < 0 || q_len < 1 || max_seq_len < 0 || num_cus < 0)
    return PA_ERR_SHAPE;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (num_cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess ||
        num_cus <= 0)
      return PA_ERR_LAUNCH;
  }
  const int64_t group = num_q_heads / num_kv_heads;
  // no plan exists for a group size the kernels do not take, so suggest none
  if (!pa::decode_supported(head_dim, (int)group)) return PA_ERR_UNSUPPORTED;
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  if (q_len > 1) {
    // Query blocks from a full block of (token, head) pairs up; below half a block the balanced
    // schedule's one pass reads each tile once for all pairs at less cost, and up to a block it
    // still wins while the batch is small.
    const int64_t cols = max_columns(head_dim), pairs = (int64_t)q_len * group;
    if (group > cols || pairs <= cols / 2 || (pairs <= cols && units <= 32))
      return PA_SCHEDULE_BALANCED;
    return PA_SCHEDULE_QUERY_BLOCKS;
  }
  if (max_seq_len == 0) return PA_SCHEDULE_BALANCED;   // nothing known: the robust choice
  const int64_t keys = window > 0 ? std::min<int64_t>(max_seq_len, window) : max_seq_len;
  // one workgroup per (sequence, KV head) when every range is short and the units cover the
  // CUs (or there is a single 256-token range anyway)
  if (keys <= 256 || (keys <= 1024 && units >= num_cus)) return PA_SCHEDULE_UNSPLIT;
  // little work in all (at most 1024 keys per CU): fixed 256-token partitions start fastest
  if (units * keys <= (int64_t)1024 * num_cus) {
    *partition_size = std::max<int32_t>(256, block_size);
    return PA_SCHEDULE_PARTITIONED;
  }
  return PA_SCHEDULE_BALANCED;   // the rest, and any spread of lengths
}

pa_status paged_attn_plan_create(const pa_shape* shape, int32_t head_dim, int32_t block_size,
                                 int32_t window, int32_t schedule, int32_t kv_dtype,
                                 const pa_kv_layout* kv_layout, int32_t q_len,
                                 int32_t max_seq_len, int32_t num_workers, pa_plan** plan) {
  return paged_attn_plan_create_flags(shape, head_dim, block_size, window, schedule, kv_dtype,
                                      kv_layout, q_len, max_seq_len, num_workers, 0, plan);
}

pa_status paged_attn_plan_create_flags(const pa_shape* shape, int32_t head_dim,
                                       int32_t block_size, int32_t window, int32_t schedule,
                                       int32_t kv_dtype, const pa_kv_layout* kv_layout,
                                       int32_t q_len, int32_t max_seq_len, int32_t num_workers,
                                       int32_t flags, pa_plan** plan) {
  if (plan == nullptr) return PA_ERR_NULL;
  *plan = nullptr;
  pa_plan* pl = new (std::nothrow) pa_plan;
  if (pl == nullptr) return PA_ERR_LAUNCH;
  const pa_status st =
      plan_build(shape, head_dim, block_size, window, schedule, kv_dtype, kv_layout, q_len,
                 max_seq_len, num_workers, flags, pl);
  if (st != PA_OK) {
    delete pl;
    return st;
  }
  *plan = pl;
  return PA_OK;
}

int64_t paged_attn_plan_workspace_size(const pa_plan* plan) {
  return plan == nullptr ? PA_ERR_NULL : plan->workspace_bytes;
}

const char* paged_attn_plan_name(const pa_plan* plan) {
  return plan == nullptr ? nullptr : plan->name;
}

void paged_attn_plan_destroy(pa_plan* plan) { delete plan; }

}  // extern "C"

namespace {

// A plan's step; ev0 / ev1 (optional) recorded right before and after the decode launch (the
// first pass's, with several passes).
pa_status plan_run(const pa_plan* plan, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_table, const int32_t* seq_lens, float scale,
                   float k_scale, float v_scale, const float* sinks, float* out, float* lse,
                   void* workspace, void* stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (plan == nullptr) return PA_ERR_NULL;
  if (!std::isfinite(scale) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return PA_ERR_SHAPE;
  if (plan->kv_dtype == PA_KV_BF16 && (k_scale != 1.f || v_scale != 1.f)) return PA_ERR_SHAPE;
  if (plan->dec.num_seqs == 0) return PA_OK;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || block_table == nullptr ||
      seq_lens == nullptr || out == nullptr)
    return PA_ERR_NULL;
  if (plan->workspace_bytes > 0) {
    if (workspace == nullptr) return PA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return PA_ERR_SHAPE;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  pa::DecodeParams p = plan->dec;
  p.q = static_cast<const uint16_t*>(q);
  p.k_cache = static_cast<const char*>(k_cache);
  p.v_cache = static_cast<const char*>(v_cache);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.sinks = sinks;
  // an FP8 cache's K scale multiplies every score: folded into the score scale
  p.qk_scale_log2 = (float)((double)scale * (double)k_scale * 1.4426950408889634);
  p.v_scale = v_scale;
  hipError_t e = hipSuccess;
  // the events around the decode launch (each records only once)
  auto before = [&]() {
    if (ev0 != nullptr && e == hipSuccess) e = hipEventRecord(ev0, s);
    ev0 = nullptr;
    return e;
  };
  auto after = [&]() {
    if (ev1 != nullptr && e == hipSuccess) e = hipEventRecord(ev1, s);
    ev1 = nullptr;
  };
  if (plan->schedule == PA_SCHEDULE_UNSPLIT) {
    p.out = out;
    p.lse = lse;
    if (before() == hipSuccess)
      e = pa::launch_decode(p, plan->head_dim, plan->group, plan->waves, plan->path, s);
    after();
  } else if (plan->schedule == PA_SCHEDULE_QUERY_BLOCKS) {
    pa::QBlockParams qp = plan->qb;
    qp.d = p;
    qp.d.out = out;
    qp.d.lse = lse;
    if (qp.splits > 1) {
      char* ws = static_cast<char*>(workspace);
      qp.part_out = reinterpret_cast<float*>(ws);
      qp.part_lse = reinterpret_cast<float*>(ws + plan->part_bytes);
    }
    // the query-block kernel, and its key-split merge when the plan has splits
    if (before() == hipSuccess) e = pa::launch_qblock(qp, plan->head_dim, plan->path, s);
    after();
    if (e == hipSuccess) e = pa::launch_qblock_merge(qp, plan->head_dim, s);
  } else if (plan->schedule == PA_SCHEDULE_PARTITIONED_FUSED) {
    char* ws = static_cast<char*>(workspace);
    p.out = reinterpret_cast<float*>(ws);
    p.lse = reinterpret_cast<float*>(ws + plan->part_bytes);
    p.merge_counters = reinterpret_cast<uint32_t*>(ws + plan->counter_off);
    p.final_out = out;
    p.final_lse = lse;
    if (before() == hipSuccess)
      e = pa::launch_decode(p, plan->head_dim, plan->group, plan->waves, plan->path, s);
    after();
  } else if (plan->schedule == PA_SCHEDULE_PARTITIONED) {
    char* ws = static_cast<char*>(workspace);
    p.out = reinterpret_cast<float*>(ws);
    p.lse = reinterpret_cast<float*>(ws + plan->part_bytes);
    if (before() == hipSuccess)
      e = pa::launch_decode(p, plan->head_dim, plan->group, plan->waves, plan->path, s);
    after();
    if (e == hipSuccess) {
      pa::ReduceParams r = plan->red;
      r.partials = p.out;
      r.lse_partials = p.lse;
      r.seq_lens = seq_lens;
      r.out = out;
      r.lse = lse;
      e = pa::launch_reduce(r, plan->head_dim, plan->dec.num_seqs, s);
    }
  } else {
    char* ws = static_cast<char*>(workspace);
    pa::BalancedParams bp{};
    bp.d = p;
    bp.d.out = out;
    bp.d.lse = lse;
    bp.prefix = reinterpret_cast<int64_t*>(ws + plan->bal.prefix);
    bp.ws_lse = reinterpret_cast<float*>(ws + plan->bal.lse);
    bp.ws_o = reinterpret_cast<float*>(ws + plan->bal.o);
    bp.num_workers = plan->num_workers;
    // one decode + fix-up per pass of query tokens (a single pass unless there are more
    // (token, head) columns than a kernel holds); the passes share the workspace in order
    for (int32_t first = 0; first < plan->q_len && e == hipSuccess;
         first += plan->pass_tokens) {
      bp.d.q_first = first;
      bp.d.q_len = plan->q_len - first < plan->pass_tokens ? plan->q_len - first
                                                           : plan->pass_tokens;
      if (before() == hipSuccess)
        e = pa::launch_balanced(bp, plan->head_dim, plan->group, plan->path, plan->q_len > 1,
                                s);
      after();
      if (e == hipSuccess) e = pa::launch_balanced_fixup(bp, plan->head_dim, plan->group, s);
    }
  }
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

pa_status paged_attn_plan_run(const pa_plan* plan, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, float scale, float k_scale,
                              float v_scale, const float* sinks, float* out, float* lse,
                              void* workspace, void* stream) {
  return plan_run(plan, q, k_cache, v_cache, block_table, seq_lens, scale, k_scale, v_scale,
                  sinks, out, lse, workspace, stream, nullptr, nullptr);
}

pa_status paged_attn_plan_run_timed(const pa_plan* plan, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* block_table,
                                    const int32_t* seq_lens, float scale, float k_scale,
                                    float v_scale, const float* sinks, float* out, float* lse,
                                    void* workspace, void* stream, void* ev_before,
                                    void* ev_after) {
  return plan_run(plan, q, k_cache, v_cache, block_table, seq_lens, scale, k_scale, v_scale,
                  sinks, out, lse, workspace, stream, static_cast<hipEvent_t>(ev_before),
                  static_cast<hipEvent_t>(ev_after));
}

}  // extern "C"

extern "C" {

pa_status paged_attn_gather_witness_balanced(const pa_shape* shape, const void* k_cache,
                                             const void* v_cache, const int32_t* block_table,
                                             const int32_t* seq_lens, int32_t head_dim,
                                             int32_t block_size, int32_t window,
                                             int32_t kv_dtype, const pa_kv_layout* kv_layout,
                                             int32_t num_workers, int32_t max_rows, void* k_rows,
                                             void* v_rows, void* stream) {
  const pa_status st = check_shape(shape);
  if (st != PA_OK) return st;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (kv_dtype != PA_KV_BF16 && kv_dtype != PA_KV_FP8_E4M3) return PA_ERR_UNSUPPORTED;
  if (window < 0 || max_rows < 1 || num_workers < 1 || num_workers > kMaxWorkers)
    return PA_ERR_SHAPE;
  const int64_t elem = kv_dtype == PA_KV_FP8_E4M3 ? 1 : 2;
  pa::BalancedParams bp{};
  pa::DecodeParams& p = bp.d;
  if (apply_kv_layout(p, kv_layout, shape->num_kv_heads, block_size, head_dim, elem) != PA_OK)
    return PA_ERR_SHAPE;
  if (shape->num_seqs == 0) return PA_OK;
  if (k_cache == nullptr || v_cache == nullptr || block_table == nullptr ||
      seq_lens == nullptr || k_rows == nullptr || v_rows == nullptr)
    return PA_ERR_NULL;
  p.k_cache = static_cast<const char*>(k_cache);
  p.v_cache = static_cast<const char*>(v_cache);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.num_seqs = shape->num_seqs;
  p.num_q_heads = shape->num_q_heads;
  p.num_kv_heads = shape->num_kv_heads;
  p.num_blocks = shape->num_blocks;
  p.stride = shape->block_table_stride;
  p.bs_log2 = log2_exact(block_size);
  p.window = window;
  p.max_parts = 1;
  p.q_len = 1;
  p.q_total = 1;
  p.group = shape->num_q_heads / shape->num_kv_heads;
  bp.num_workers = num_workers;
  const hipError_t e = pa::launch_balanced_witness(
      bp, static_cast<char*>(k_rows), static_cast<char*>(v_rows), (int)(elem * head_dim),
      max_rows, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // extern "C"
