// Test and measurement kernels: the gather witness, a streaming-read probe and a plain copy.
//
// The witness walks a sequence's attended tiles with the decode kernels' own TileAddr and
// part_range code and the same per-lane row loads, and stores the rows it would read into a
// contiguous buffer, so a test can compare the integer path (block-table walk, head and slot
// offsets, window start, tail) byte for byte with the oracle's gather.  Witnesses that prove
// which code ran from inside the kernel: vllm.cpp PR #2472 "cooperate across Q8_K activation
// blocks", "Evidence"; window skip: randomvariable/vllm issue #23, table "Current state".
#include "pa_device.hpp"
#include "pa_kernels.hpp"

namespace pa {

template <int D>
__global__ __launch_bounds__(kWave) void witness_kernel(const WitnessParams p) {
  using RG = RowGeom<D>;
  constexpr int W = RG::kWords;
  const int lane = threadIdx.x;
  const int r = lane >> 4;
  const int c = lane & (kRowLanes - 1);
  const int kvh = blockIdx.x;
  const int b = blockIdx.y;
  const int L = p.seq_lens[b];
  if (L <= 0 || (int64_t)L > ((int64_t)p.stride << p.bs_log2)) return;
  const PartRange pr = part_range(L, p.window, 0, 0);
  // the default pool layout [num_blocks][Hkv][bs][D]
  const int64_t head_bytes = (int64_t)RG::kRowBytes << p.bs_log2;
  const TileAddr ta{p.num_blocks, p.bs_log2, head_bytes * p.num_kv_heads, kvh * head_bytes,
                    RG::kRowBytes};
  const int32_t* bt_row = p.block_table + (size_t)b * p.stride;
  const size_t base = ((size_t)b * p.num_kv_heads + kvh) * p.max_rows;
  const int t0 = pr.lo / kTileTokens;
  const int t1 = (pr.hi + kTileTokens - 1) / kTileTokens;
  for (int t = t0; t < t1; ++t) {
    const int64_t off = ta.offset(__builtin_amdgcn_readfirstlane(bt_row[ta.logical_block(t)]), t);
#pragma unroll
    for (int j = 0; j < kTileSteps; ++j) {
      const int tk = t * kTileTokens + kRows * j + r;
      const int i = tk - pr.lo;
      if (tk < pr.lo || tk >= pr.hi || i >= p.max_rows) continue;
      uint32_t kw[W], vw[W];
      if (off < 0) {
#pragma unroll
        for (int w = 0; w < W; ++w) kw[w] = vw[w] = 0x7FC07FC0u;
      } else {
        load_row<D>(p.k_cache + off + (kRows * j + r) * RG::kRowBytes, c, kw);
        load_row<D>(p.v_cache + off + (kRows * j + r) * RG::kRowBytes, c, vw);
      }
      store_row<D>(p.k_rows + (base + i) * RG::kRowBytes, c, kw);
      store_row<D>(p.v_rows + (base + i) * RG::kRowBytes, c, vw);
    }
  }
}

hipError_t launch_witness(const WitnessParams& p, int head_dim, int num_seqs, hipStream_t stream) {
  const dim3 grid(p.num_kv_heads, num_seqs);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(witness_kernel<64>, grid, dim3(kWave), 0, stream, p); break;
    case 128: hipLaunchKernelGGL(witness_kernel<128>, grid, dim3(kWave), 0, stream, p); break;
    case 256: hipLaunchKernelGGL(witness_kernel<256>, grid, dim3(kWave), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// streaming read: each thread reads 16 B per step, 4 steps unrolled, grid-strided
// ---------------------------------------------------------------------------------------------
constexpr int kStreamThreads = 256;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint4* __restrict__ buf,
                                                                    size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kStreamThreads;
  size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
  // non-temporal loads, as the decode kernels stream K/V
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(buf);
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t a = __builtin_nontemporal_load(src + i);
    const u32x4_t b = __builtin_nontemporal_load(src + i + stride);
    const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * stride);
    const u32x4_t e = a ^ b ^ c ^ d;
    x ^= e.x ^ e.y ^ e.z ^ e.w;
  }
  for (; i < n16; i += stride) {
    const u32x4_t a = __builtin_nontemporal_load(src + i);
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red[kStreamThreads];
  red[threadIdx.x] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int k = 0; k < kStreamThreads; ++k) y ^= red[k];
    sink[blockIdx.x] = y;
  }
}

hipError_t launch_stream_read(const void* buf, size_t bytes, int num_wg, uint32_t* sink,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(num_wg), dim3(kStreamThreads), 0, stream,
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// gather read: the access pattern of the decode kernels without their arithmetic.  Chunks of
// 1024 * P bytes (a 16-token tile of one KV head: 4 KiB at head_dim 128) are read in the order of
// a caller-given id list, each by one wave with P 16-byte non-temporal loads per lane; wave w of
// the grid takes the contiguous share [w n / N, (w+1) n / N) of the list and keeps two chunks in
// flight.  An id outside [0, num_chunks) is skipped, never read.
// ---------------------------------------------------------------------------------------------
constexpr int kGatherThreads = 256;

template <int P>
__global__ __launch_bounds__(kGatherThreads) void gather_read_kernel(
    const char* __restrict__ buf, int64_t num_chunks, const int32_t* __restrict__ ids,
    int64_t n_ids, uint32_t* sink) {
  constexpr int kChunk = 1024 * P;
  const int lane = threadIdx.x % kWave;
  const int64_t nw = (int64_t)gridDim.x * (kGatherThreads / kWave);
  const int64_t w = (int64_t)blockIdx.x * (kGatherThreads / kWave) + threadIdx.x / kWave;
  const int64_t q = n_ids / nw, r = n_ids - q * nw;
  const int64_t lo = w * q + (w * r) / nw, hi = (w + 1) * q + ((w + 1) * r) / nw;
  uint32_t x = 0;
  auto load = [&](int64_t k, u32x4_t (&v)[P]) {
    const int64_t id = __builtin_amdgcn_readfirstlane(ids[k]);
    if (id < 0 || id >= num_chunks) {
#pragma unroll
      for (int j = 0; j < P; ++j) v[j] = u32x4_t{0u, 0u, 0u, 0u};
      return;
    }
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(buf + id * kChunk) + lane;
#pragma unroll
    for (int j = 0; j < P; ++j) v[j] = __builtin_nontemporal_load(src + j * kWave);
  };
  u32x4_t a[P], b[P];
  int64_t k = lo;
  for (; k + 1 < hi; k += 2) {
    load(k, a);
    load(k + 1, b);
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const u32x4_t e = a[j] ^ b[j];
      x ^= e.x ^ e.y ^ e.z ^ e.w;
    }
  }
  if (k < hi) {
    load(k, a);
#pragma unroll
    for (int j = 0; j < P; ++j) x ^= a[j].x ^ a[j].y ^ a[j].z ^ a[j].w;
  }
  __shared__ uint32_t red[kGatherThreads];
  red[threadIdx.x] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int i = 0; i < kGatherThreads; ++i) y ^= red[i];
    sink[blockIdx.x] = y;
  }
}

hipError_t launch_gather_read(const void* buf, int64_t num_chunks, int chunk_bytes,
                              const int32_t* ids, int64_t n_ids, int num_wg, uint32_t* sink,
                              hipStream_t stream) {
  const char* b = static_cast<const char*>(buf);
  switch (chunk_bytes) {
    case 2048:
      hipLaunchKernelGGL(gather_read_kernel<2>, dim3(num_wg), dim3(kGatherThreads), 0, stream, b,
                         num_chunks, ids, n_ids, sink);
      break;
    case 4096:
      hipLaunchKernelGGL(gather_read_kernel<4>, dim3(num_wg), dim3(kGatherThreads), 0, stream, b,
                         num_chunks, ids, n_ids, sink);
      break;
    case 8192:
      hipLaunchKernelGGL(gather_read_kernel<8>, dim3(num_wg), dim3(kGatherThreads), 0, stream, b,
                         num_chunks, ids, n_ids, sink);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void copy_kernel(uint4* __restrict__ dst,
                                                  const uint4* __restrict__ src, size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<uint4*>(dst), static_cast<const uint4*>(src), n16);
  return hipGetLastError();
}

}  // namespace pa
