// reduce.hip -- merge the split path's per-partition partials.
//
// "Inside vLLM CUDA Kernels", Part 3, "How Each K/V Tile Contributes to the
// Output": partial states are rescaled to a common maximum before merging.  For
// (s, h) over the n = ceil(seq_len / partition) partitions that hold tokens:
// M = max m_p, w_p = l_p * exp(m_p - M), out = sum w_p o_p / sum w_p.
//
// The work is tiny (4 MiB of partials for 4 sequences of 32768 tokens) and latency
// bound, so the kernel is built around one round trip to memory: a 256-thread
// workgroup per (sequence, query head, 32-dim slice of the output); once the
// sequence's length is known (one scalar load) each thread issues, at once, every
// load it needs -- m_p, l_p and one 16-byte piece of o_p for each of its partitions
// p = g, g + 32, ... -- then a block-wide max, the weights, the weighted sums and one
// LDS reduction over the 32 partition groups.
#include <cmath>

#include "device_common.h"
#include "launch.h"

namespace pcache {
namespace {

constexpr int kReduceThreads = 256;
constexpr int kSlice = 32;                        // output dims per workgroup
constexpr int kCols = kSlice / 4;                 // float4 columns of a slice
constexpr int kGroups = kReduceThreads / kCols;   // partitions summed side by side
constexpr int kPerThread = 8;                     // partitions a thread keeps in flight at once

template <class ST>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(ReduceArgs a) {
  __shared__ float red[kReduceThreads / kWave];
  __shared__ __align__(16) float4 part_o[kGroups][kCols];
  __shared__ float part_w[kGroups];

  const int D = a.head_size;
  const int slices = D / kSlice;
  const int slice = blockIdx.x % slices;
  const int64_t sh = blockIdx.x / slices;  // s * num_q_heads + h
  const int s = (int)(sh / a.num_q_heads);
  const int c = threadIdx.x % kCols;
  const int grp = threadIdx.x / kCols;
  const int L = a.seq_lens[s];
  const int64_t n64 = L <= 0 ? 0 : ((int64_t)L + a.partition_size - 1) / a.partition_size;
  const bool bad = L < 0 || n64 > a.max_partitions;
  const int n = bad ? 0 : (int)n64;
  const float* ml = a.max_logits + sh * a.max_partitions;
  const float* es = a.exp_sums + sh * a.max_partitions;
  const float4* rows = reinterpret_cast<const float4*>(a.tmp_out + sh * a.max_partitions * D + slice * kSlice) + c;
  const int row4 = D / 4;

  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  float M = -INFINITY;
  // partitions grp, grp + kGroups, ... in batches of kPerThread (one batch covers
  // 256 partitions = 131072 tokens)
  for (int p0 = 0; p0 < n; p0 += kGroups * kPerThread) {
    float m[kPerThread], l[kPerThread];
    float4 t[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int p = p0 + grp + i * kGroups;
      const bool in = p < n;
      m[i] = in ? ml[p] : -INFINITY;
      l[i] = in ? es[p] : 0.f;
      t[i] = in ? rows[(int64_t)p * row4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // the batch's max over every thread's partitions
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) bm = fmaxf(bm, m[i]);
    for (int off = 32; off > 0; off >>= 1) bm = fmaxf(bm, __shfl_xor(bm, off));
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = bm;
    __syncthreads();
    float nm = M;
#pragma unroll
    for (int i = 0; i < kReduceThreads / kWave; ++i) nm = fmaxf(nm, red[i]);
    __syncthreads();
    // rescale what earlier batches summed to the new maximum, then add this batch
    const float f = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((M - nm) * kLog2e);
    o.x *= f;
    o.y *= f;
    o.z *= f;
    o.w *= f;
    wsum *= f;
    M = nm;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const float wp = m[i] == -INFINITY ? 0.f : l[i] * __builtin_amdgcn_exp2f((m[i] - M) * kLog2e);
      wsum += wp;
      o.x = fmaf(wp, t[i].x, o.x);
      o.y = fmaf(wp, t[i].y, o.y);
      o.z = fmaf(wp, t[i].z, o.z);
      o.w = fmaf(wp, t[i].w, o.w);
    }
  }
  part_o[grp][c] = o;
  if (c == 0) part_w[grp] = wsum;
  __syncthreads();
  if (threadIdx.x < kCols) {
    float4 to = make_float4(0.f, 0.f, 0.f, 0.f);
    float tw = 0.f;
#pragma unroll 8
    for (int g = 0; g < kGroups; ++g) {
      const float4 v = part_o[g][threadIdx.x];
      to.x += v.x;
      to.y += v.y;
      to.z += v.z;
      to.w += v.w;
      tw += part_w[g];
    }
    const float inv = 1.f / tw;
    float r[4] = {to.x * inv, to.y * inv, to.z * inv, to.w * inv};
    const int64_t base = sh * D + slice * kSlice + 4 * threadIdx.x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = bad ? NAN : (n == 0 ? 0.f : r[e]);
      const uint32_t bits = to_storage<ST>(r[e]);
      if constexpr (ST::kBytes == 4)
        static_cast<uint32_t*>(a.out)[base + e] = bits;
      else
        static_cast<uint16_t*>(a.out)[base + e] = (uint16_t)bits;
    }
  }
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, int dtype, hipStream_t stream) {
  const int64_t n = (int64_t)a.num_seqs * a.num_q_heads * (a.head_size / kSlice);
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

bool reduce_supported(int head_size) { return head_size >= kSlice && head_size % kSlice == 0; }

}  // namespace pcache
