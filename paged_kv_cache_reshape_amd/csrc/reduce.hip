// reduce.hip -- merge the split path's per-partition partials.
//
// "Inside vLLM CUDA Kernels", Part 3, "How Each K/V Tile Contributes to the
// Output": partial states are rescaled to a common maximum before merging.  For
// (s, h) over the n = ceil(seq_len / partition) partitions that hold tokens:
// M = max m_p, w_p = l_p * exp(m_p - M), out = sum w_p o_p / sum w_p.
//
// The work is small and latency bound, so both kernels are built around one round
// trip to memory: once a row's sequence length is known, every load the row needs --
// m_p, l_p and 16-byte pieces of o_p for each partition p < n -- is issued at once.
// * Many partitions per row (long sequences, few rows): reduce_kernel, a 256-thread
//   workgroup per (sequence, query head, 32-dim slice of the output); its threads
//   take partitions g, g + 32, ... side by side.  Each wave keeps its own running
//   maximum and sums (folded across its 8 partition groups with lane shuffles); the
//   four wave states are rescaled to the common maximum once, through LDS, behind a
//   single barrier.
// * Few partitions per row (at most kRowsMaxParts, i.e. sequences up to 8192 tokens,
//   typically many rows): reduce_rows_kernel, one wave per (sequence, query head).
//   The wave's lanes form 64 / (D/4) partition groups of D/4 lanes (a float4 of the
//   row each); the max and the sums fold across the groups with lane shuffles, so no
//   barrier and no LDS are involved.  (The slice kernel would leave most of its 32
//   groups idle there and pay two barriers per workgroup.)
#include <cmath>

#include "device_common.h"
#include "launch.h"

namespace pcache {
namespace {

constexpr int kReduceThreads = 256;
constexpr int kSlice = 32;                        // output dims per workgroup
constexpr int kCols = kSlice / 4;                 // float4 columns of a slice
constexpr int kGroups = kReduceThreads / kCols;   // partitions summed side by side
constexpr int kWaves = kReduceThreads / kWave;
constexpr int kPerThread = 8;                     // partitions a thread keeps in flight at once

template <class ST>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(ReduceArgs a) {
  __shared__ __align__(16) float4 wave_o[kWaves][kCols];
  __shared__ float wave_m[kWaves];
  __shared__ float wave_w[kWaves];

  const int D = a.head_size;
  const int slices = D / kSlice;
  const int slice = blockIdx.x % slices;
  const int64_t sh = blockIdx.x / slices;  // s * num_q_heads + h
  const int s = (int)(sh / a.num_q_heads);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
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

  // this wave's state: M over its partitions so far (the same in every lane), and the
  // lane's weighted sums relative to M
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
    // the batch's max over the wave's partition groups (lanes of one group hold the same m)
    float bm = M;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) bm = fmaxf(bm, m[i]);
#pragma unroll
    for (int off = kCols; off < kWave; off <<= 1) bm = fmaxf(bm, __shfl_xor(bm, off));
    // rescale what earlier batches summed to the new maximum, then add this batch
    const float f = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((M - bm) * kLog2e);
    o.x *= f;
    o.y *= f;
    o.z *= f;
    o.w *= f;
    wsum *= f;
    M = bm;
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
  // fold the wave's partition groups (all relative to the wave's M)
#pragma unroll
  for (int off = kCols; off < kWave; off <<= 1) {
    wsum += __shfl_xor(wsum, off);
    o.x += __shfl_xor(o.x, off);
    o.y += __shfl_xor(o.y, off);
    o.z += __shfl_xor(o.z, off);
    o.w += __shfl_xor(o.w, off);
  }
  if (lane < kCols) wave_o[wave][lane] = o;
  if (lane == 0) {
    wave_m[wave] = M;
    wave_w[wave] = wsum;
  }
  __syncthreads();
  if (threadIdx.x < kCols) {
    float gm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) gm = fmaxf(gm, wave_m[w]);
    float4 to = make_float4(0.f, 0.f, 0.f, 0.f);
    float tw = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      // a wave that saw no partition (or only -inf maxima) holds zeros, or NaN sums
      // that must still reach the output
      const float wm = wave_m[w];
      const float f = wm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((wm - gm) * kLog2e);
      const float4 v = wave_o[w][threadIdx.x];
      to.x = fmaf(f, v.x, to.x);
      to.y = fmaf(f, v.y, to.y);
      to.z = fmaf(f, v.z, to.z);
      to.w = fmaf(f, v.w, to.w);
      tw = fmaf(f, wave_w[w], tw);
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

// ---- few partitions per row: one wave per (sequence, query head) --------------------
constexpr int kRowsMaxParts = 16;  // partitions a row may have on this kernel
constexpr int kRowsPerBlock = 4;   // waves (rows) per workgroup

template <class ST, int D>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void reduce_rows_kernel(ReduceArgs a) {
  constexpr int kLanes = D / 4;               // lanes covering one partition's row (a float4 each)
  constexpr int kGroupsW = kWave / kLanes;    // partition groups in the wave
  constexpr int kPer = kRowsMaxParts / kGroupsW;  // partitions per lane, all loads in flight
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t sh = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;  // s * num_q_heads + h
  if (sh >= (int64_t)a.num_seqs * a.num_q_heads) return;
  const int s = (int)(sh / a.num_q_heads);
  const int c = lane % kLanes;
  const int grp = lane / kLanes;
  const int L = a.seq_lens[s];  // wave-uniform
  const int64_t n64 = L <= 0 ? 0 : ((int64_t)L + a.partition_size - 1) / a.partition_size;
  const bool bad = L < 0 || n64 > a.max_partitions;
  const int n = bad ? 0 : (int)n64;  // <= max_partitions <= kRowsMaxParts
  const float* ml = a.max_logits + sh * a.max_partitions;
  const float* es = a.exp_sums + sh * a.max_partitions;
  const float4* rows = reinterpret_cast<const float4*>(a.tmp_out + sh * a.max_partitions * D) + c;

  float m[kPer], l[kPer];
  float4 t[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int p = grp + i * kGroupsW;
    const bool in = p < n;
    m[i] = in ? ml[p] : -INFINITY;
    l[i] = in ? es[p] : 0.f;
    t[i] = in ? rows[(int64_t)p * (D / 4)] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPer; ++i) M = fmaxf(M, m[i]);
#pragma unroll
  for (int off = kLanes; off < kWave; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float w = 0.f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const float wp = m[i] == -INFINITY ? 0.f : l[i] * __builtin_amdgcn_exp2f((m[i] - M) * kLog2e);
    w += wp;
    o.x = fmaf(wp, t[i].x, o.x);
    o.y = fmaf(wp, t[i].y, o.y);
    o.z = fmaf(wp, t[i].z, o.z);
    o.w = fmaf(wp, t[i].w, o.w);
  }
#pragma unroll
  for (int off = kLanes; off < kWave; off <<= 1) {
    w += __shfl_xor(w, off);
    o.x += __shfl_xor(o.x, off);
    o.y += __shfl_xor(o.y, off);
    o.z += __shfl_xor(o.z, off);
    o.w += __shfl_xor(o.w, off);
  }
  if (grp != 0) return;
  const float inv = 1.f / w;
  float r[4] = {o.x * inv, o.y * inv, o.z * inv, o.w * inv};
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = bad ? NAN : (n == 0 ? 0.f : r[e]);
  const int64_t base = sh * D + 4 * c;
  if constexpr (ST::kBytes == 4) {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + base) = make_float4(r[0], r[1], r[2], r[3]);
  } else {
    const uint32_t lo = to_storage<ST>(r[0]) | (to_storage<ST>(r[1]) << 16);
    const uint32_t hi = to_storage<ST>(r[2]) | (to_storage<ST>(r[3]) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + base) = make_uint2(lo, hi);
  }
}

}  // namespace

template <class ST>
hipError_t launch_rows(const ReduceArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.num_seqs * a.num_q_heads;
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(kRowsPerBlock * kWave);
  if (a.head_size == 128)
    hipLaunchKernelGGL((reduce_rows_kernel<ST, 128>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((reduce_rows_kernel<ST, 64>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& a, int dtype, hipStream_t stream) {
  const int64_t n = (int64_t)a.num_seqs * a.num_q_heads * (a.head_size / kSlice);
  if (n == 0) return hipSuccess;
  if (!reduce_supported(a.head_size)) return hipErrorInvalidValue;
  // the rows kernel stores 4 output elements at once: out must be aligned to that
  const uintptr_t out_align = (dtype == 0 ? 16u : 8u) - 1u;
  if (a.max_partitions <= kRowsMaxParts && (a.head_size == 64 || a.head_size == 128) &&
      (reinterpret_cast<uintptr_t>(a.out) & out_align) == 0) {
    switch (dtype) {
      case 0: return launch_rows<F32>(a, stream);
      case 1: return launch_rows<F16>(a, stream);
      case 2: return launch_rows<BF16>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
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
