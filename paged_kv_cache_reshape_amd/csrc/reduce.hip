// reduce.hip -- merge the split path's per-partition partials.
//
// "Inside vLLM CUDA Kernels", Part 3, "How Each K/V Tile Contributes to the
// Output": partial states are rescaled to a common maximum before merging.  For
// (s, h) over the n = ceil(seq_len / partition) partitions that hold tokens:
// M = max m_p, w_p = l_p * exp(m_p - M), out = sum w_p o_p / sum w_p.
//
// One workgroup per (sequence, query head), one lane per output dimension: the
// partials of consecutive dimensions are contiguous, so each partition's row is a
// coalesced read; the n (m_p, l_p) pairs are read by every lane from cache.
#include <cmath>

#include "device_common.h"
#include "launch.h"

namespace pcache {
namespace {

constexpr int kReduceThreads = 128;

template <class ST>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(ReduceArgs a) {
  const int h = blockIdx.x % a.num_q_heads;
  const int s = blockIdx.x / a.num_q_heads;
  const int L = a.seq_lens[s];
  const int64_t n = L <= 0 ? 0 : ((int64_t)L + a.partition_size - 1) / a.partition_size;
  const bool bad = L < 0 || n > a.max_partitions;
  const int64_t sh = (int64_t)s * a.num_q_heads + h;
  const float* ml = a.max_logits + sh * a.max_partitions;
  const float* es = a.exp_sums + sh * a.max_partitions;
  const float* tmp = a.tmp_out + sh * a.max_partitions * a.head_size;

  float M = -INFINITY;
  if (!bad)
    for (int64_t p = 0; p < n; ++p) M = fmaxf(M, ml[p]);

  for (int d = threadIdx.x; d < a.head_size; d += kReduceThreads) {
    float o = 0.f, ws = 0.f;
    if (!bad)
      for (int64_t p = 0; p < n; ++p) {
        const float wp = es[p] * __builtin_amdgcn_exp2f((ml[p] - M) * kLog2e);
        ws += wp;
        o = fmaf(wp, tmp[p * a.head_size + d], o);
      }
    const float r = bad ? NAN : (n == 0 ? 0.f : o / ws);
    const uint32_t bits = to_storage<ST>(r);
    if constexpr (ST::kBytes == 4)
      static_cast<uint32_t*>(a.out)[sh * a.head_size + d] = bits;
    else
      static_cast<uint16_t*>(a.out)[sh * a.head_size + d] = (uint16_t)bits;
  }
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, int dtype, hipStream_t stream) {
  const int64_t n = (int64_t)a.num_seqs * a.num_q_heads;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)n), block(kReduceThreads);
  switch (dtype) {
    case 0: hipLaunchKernelGGL((reduce_kernel<F32>), grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL((reduce_kernel<F16>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((reduce_kernel<BF16>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pcache
