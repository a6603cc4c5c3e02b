// reduce.hip -- merge the split path's per-partition partials.
//
// "Inside vLLM CUDA Kernels", Part 3, "How Each K/V Tile Contributes to the
// Output": partial states are rescaled to a common maximum before merging.  For
// (s, h) over the n = ceil(seq_len / partition) partitions that hold tokens:
// M = max m_p, w_p = l_p * exp(m_p - M), out = sum w_p o_p / sum w_p.
//
// One 256-thread workgroup per (sequence, query head).  The n (m_p, l_p) pairs are
// read once, cooperatively: a block-wide max gives M, and each weight w_p is formed
// once and kept in LDS (in chunks of kChunk partitions).  The lanes then split into
// 256 / (head_size/4) partition groups; each lane accumulates four output dimensions
// (one 16-byte load per partition) over its group's partitions, with up to eight
// loads in flight, and the groups' sums meet in LDS.
#include <cmath>

#include "device_common.h"
#include "launch.h"

namespace pcache {
namespace {

constexpr int kReduceThreads = 256;
constexpr int kChunk = 1024;  // partitions whose weights sit in LDS at once (512K tokens)

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kReduceThreads / kWave; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

template <class ST>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(ReduceArgs a) {
  __shared__ float w_lds[kChunk];
  __shared__ float red[kReduceThreads / kWave];
  __shared__ __align__(16) float4 part_o[kReduceThreads];
  __shared__ float part_w[kReduceThreads];

  const int h = blockIdx.x % a.num_q_heads;
  const int s = blockIdx.x / a.num_q_heads;
  const int D = a.head_size;
  const int D4 = D / 4;                      // float4 columns of a partial row
  const int groups = kReduceThreads / D4;    // partitions summed side by side
  const int d4 = threadIdx.x % D4;
  const int grp = threadIdx.x / D4;
  const int L = a.seq_lens[s];
  const int64_t n64 = L <= 0 ? 0 : ((int64_t)L + a.partition_size - 1) / a.partition_size;
  const bool bad = L < 0 || n64 > a.max_partitions;
  const int n = bad ? 0 : (int)n64;
  const int64_t sh = (int64_t)s * a.num_q_heads + h;
  const float* ml = a.max_logits + sh * a.max_partitions;
  const float* es = a.exp_sums + sh * a.max_partitions;
  const float* tmp = a.tmp_out + sh * a.max_partitions * D;

  float M = -INFINITY;
  for (int p = threadIdx.x; p < n; p += kReduceThreads) M = fmaxf(M, ml[p]);
  M = block_max(M, red);

  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float ws = 0.f;
  for (int c0 = 0; c0 < n; c0 += kChunk) {
    const int cn = min(kChunk, n - c0);
    for (int p = threadIdx.x; p < cn; p += kReduceThreads)
      w_lds[p] = es[c0 + p] * __builtin_amdgcn_exp2f((ml[c0 + p] - M) * kLog2e);
    __syncthreads();
    const float4* rows = reinterpret_cast<const float4*>(tmp + (int64_t)c0 * D) + d4;
#pragma unroll 8
    for (int p = grp; p < cn; p += groups) {
      const float wp = w_lds[p];
      const float4 t = rows[(int64_t)p * D4];
      ws += wp;
      o.x = fmaf(wp, t.x, o.x);
      o.y = fmaf(wp, t.y, o.y);
      o.z = fmaf(wp, t.z, o.z);
      o.w = fmaf(wp, t.w, o.w);
    }
    __syncthreads();
  }
  part_o[threadIdx.x] = o;
  part_w[threadIdx.x] = ws;
  __syncthreads();
  if (threadIdx.x < D4) {
    float4 to = make_float4(0.f, 0.f, 0.f, 0.f);
    float tw = 0.f;
    for (int g = 0; g < groups; ++g) {
      const float4 v = part_o[g * D4 + threadIdx.x];
      to.x += v.x;
      to.y += v.y;
      to.z += v.z;
      to.w += v.w;
      tw += part_w[g * D4 + threadIdx.x];
    }
    const float inv = 1.f / tw;
    float r[4] = {to.x * inv, to.y * inv, to.z * inv, to.w * inv};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = bad ? NAN : (n == 0 ? 0.f : r[e]);
      const uint32_t bits = to_storage<ST>(r[e]);
      if constexpr (ST::kBytes == 4)
        static_cast<uint32_t*>(a.out)[sh * D + 4 * threadIdx.x + e] = bits;
      else
        static_cast<uint16_t*>(a.out)[sh * D + 4 * threadIdx.x + e] = (uint16_t)bits;
    }
  }
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, int dtype, hipStream_t stream) {
  const int64_t n = (int64_t)a.num_seqs * a.num_q_heads;
  if (n == 0) return hipSuccess;
  if (!reduce_supported(a.head_size)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)n), block(kReduceThreads);
  switch (dtype) {
    case 0: hipLaunchKernelGGL((reduce_kernel<F32>), grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL((reduce_kernel<F16>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((reduce_kernel<BF16>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool reduce_supported(int head_size) {
  return head_size >= 4 && head_size % 4 == 0 && head_size / 4 <= kReduceThreads &&
         kReduceThreads % (head_size / 4) == 0;
}

}  // namespace pcache
