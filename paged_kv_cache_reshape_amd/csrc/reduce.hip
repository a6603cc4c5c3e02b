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
// 256 / head_size partition groups; each lane accumulates one output dimension over
// its group's partitions with independent, coalesced loads of the partial rows, and
// the groups' sums meet in LDS.
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
  __shared__ float part_o[kReduceThreads];
  __shared__ float part_w[kReduceThreads];

  const int h = blockIdx.x % a.num_q_heads;
  const int s = blockIdx.x / a.num_q_heads;
  const int D = a.head_size;
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

  // lanes t: dimension d = t % D of partition group t / D (D divides 256 for 64/128)
  const int groups = kReduceThreads / D;
  const int d = threadIdx.x % D;
  const int grp = threadIdx.x / D;
  float o = 0.f, ws = 0.f;
  for (int c0 = 0; c0 < n; c0 += kChunk) {
    const int cn = min(kChunk, n - c0);
    for (int p = threadIdx.x; p < cn; p += kReduceThreads)
      w_lds[p] = es[c0 + p] * __builtin_amdgcn_exp2f((ml[c0 + p] - M) * kLog2e);
    __syncthreads();
    if (grp < groups) {
      const float* row = tmp + (int64_t)c0 * D + d;
      int p = grp;
#pragma unroll 4
      for (; p < cn; p += groups) {
        const float wp = w_lds[p];
        ws += wp;
        o = fmaf(wp, row[(int64_t)p * D], o);
      }
    }
    __syncthreads();
  }
  part_o[threadIdx.x] = o;
  part_w[threadIdx.x] = ws;
  __syncthreads();
  if (threadIdx.x < D) {
    float to = 0.f, tw = 0.f;
    for (int g = 0; g < groups; ++g) {
      to += part_o[g * D + threadIdx.x];
      tw += part_w[g * D + threadIdx.x];
    }
    const float r = bad ? NAN : (n == 0 ? 0.f : to / tw);
    const uint32_t bits = to_storage<ST>(r);
    if constexpr (ST::kBytes == 4)
      static_cast<uint32_t*>(a.out)[sh * D + threadIdx.x] = bits;
    else
      static_cast<uint16_t*>(a.out)[sh * D + threadIdx.x] = (uint16_t)bits;
  }
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, int dtype, hipStream_t stream) {
  const int64_t n = (int64_t)a.num_seqs * a.num_q_heads;
  if (n == 0) return hipSuccess;
  if (a.head_size <= 0 || a.head_size > kReduceThreads || kReduceThreads % a.head_size != 0)
    return hipErrorInvalidValue;
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
  return head_size > 0 && head_size <= kReduceThreads && kReduceThreads % head_size == 0;
}

}  // namespace pcache
