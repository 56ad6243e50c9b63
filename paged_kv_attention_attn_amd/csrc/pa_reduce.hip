// Split-KV reduce for gfx950: merges the per-partition partial outputs and log-sum-exps of
// paged_attn_decode into the final output (and LSE).
//
// Per (sequence b, query head h) over its n = max(1, ceil(L/P)) partitions:
//   M = max_p lse_p,  w_p = exp(lse_p - M),  out = sum_p w_p o_p / sum_p w_p,
//   lse = M + ln sum_p w_p;  partitions with lse = -inf carry no weight.
// The reducer consumes the partial outputs, the sequence lengths and the LSE buffer:
// ROCm/rocm-libraries PR #13700 "prepare saved paged decode bindings once", review finding N1
// (the reduce kernel's output, seq_lens and lse pointers).
//
// One 256-thread workgroup per (h, b).  Pass 1 finds M over the partition LSEs.  Pass 2 reads
// the partial rows with 16-byte loads: D/4 threads cover one row, 1024/D rows per step, so a
// workgroup keeps several rows in flight; the per-row-slot sums meet in LDS.
#include "pa_device.hpp"
#include "pa_kernels.hpp"

namespace pa {

constexpr int kReduceThreads = 256;

__device__ __forceinline__ float block_max(float x, float* red) {
  x = wave_max(x);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  float y = red[0];
#pragma unroll
  for (int w = 1; w < kReduceThreads / kWave; ++w) y = fmaxf(y, red[w]);
  __syncthreads();
  return y;
}

template <int D>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(const ReduceParams p) {
  constexpr int TPR = D / 4;                  // threads per partial row
  constexpr int RPS = kReduceThreads / TPR;   // partial rows per step
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;

  const int L = p.seq_lens[b];
  int n = L > 0 ? (int)(((int64_t)L + p.psize - 1) / p.psize) : 1;
  bool bad = L < 0 || n > p.max_parts;
  if (n > p.max_parts) n = p.max_parts;

  const size_t row = (size_t)b * p.num_q_heads + h;
  const float* lr = p.lse_partials + row * p.max_parts;
  const float* orow = p.partials + row * p.max_parts * D;

  __shared__ float red[kReduceThreads / kWave];
  __shared__ float s_acc[RPS][D];
  __shared__ float s_sum[RPS];
  __shared__ int s_nan;
  if (tid == 0) s_nan = 0;

  float mx = -INFINITY;
  bool nan = false;
  for (int i = tid; i < n; i += kReduceThreads) {
    const float v = lr[i];
    nan |= v != v;
    mx = fmaxf(mx, v);
  }
  __syncthreads();
  if (nan) s_nan = 1;
  const float M = block_max(mx, red);
  const float Mu = M == -INFINITY ? 0.f : M;

  const int pr = tid / TPR;
  const int dq = tid - pr * TPR;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  float ssum = 0.f;
#pragma unroll 4
  for (int i = pr; i < n; i += RPS) {
    const float li = lr[i];
    const float4 o = *reinterpret_cast<const float4*>(orow + (size_t)i * D + 4 * dq);
    const bool live = li != -INFINITY;
    const float w = fast_exp2((li - Mu) * kLog2e);
    // select, not multiply: an empty partition's row is never mixed in, whatever it holds
    a.x = live ? fmaf(w, o.x, a.x) : a.x;
    a.y = live ? fmaf(w, o.y, a.y) : a.y;
    a.z = live ? fmaf(w, o.z, a.z) : a.z;
    a.w = live ? fmaf(w, o.w, a.w) : a.w;
    ssum += live ? w : 0.f;
  }
  *reinterpret_cast<float4*>(&s_acc[pr][4 * dq]) = a;
  if (dq == 0) s_sum[pr] = ssum;
  __syncthreads();

  if (tid < D) {
    float o = 0.f, S = 0.f;
#pragma unroll
    for (int k = 0; k < RPS; ++k) {
      o += s_acc[k][tid];
      S += s_sum[k];
    }
    float ov = S > 0.f ? o / S : 0.f;
    float lv = S > 0.f ? Mu + fast_log2(S) * kLn2 : -INFINITY;
    if (bad || s_nan) {
      ov = __builtin_nanf("");
      lv = __builtin_nanf("");
    }
    p.out[row * D + tid] = ov;
    if (tid == 0 && p.lse != nullptr) p.lse[row] = lv;
  }
}

hipError_t launch_reduce(const ReduceParams& p, int head_dim, int num_seqs, hipStream_t stream) {
  const dim3 grid(p.num_q_heads, num_seqs);
  switch (head_dim) {
    case 64:
      hipLaunchKernelGGL(reduce_kernel<64>, grid, dim3(kReduceThreads), 0, stream, p);
      break;
    case 128:
      hipLaunchKernelGGL(reduce_kernel<128>, grid, dim3(kReduceThreads), 0, stream, p);
      break;
    case 256:
      hipLaunchKernelGGL(reduce_kernel<256>, grid, dim3(kReduceThreads), 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
