// stream.hip -- a plain streaming read of device memory, the yardstick for the decode's
// HBM rate.
//
// The decode reads each K/V byte once from HBM; "vLLM 源码完全拆解（七）: PagedAttention
// Kernel", section 性能模型, names that stream as the bound of the whole path.  What a
// kernel can reach on one chip is below the 8 TB/s the part is rated for, so the
// benchmark also reports the decode's rate against this kernel's: every byte of the
// buffer read once, 16-byte buffer loads, eight in flight per lane, each workgroup a
// contiguous chunk, with the cache-policy operand the decode uses for K (0) or for V
// (non-temporal, 2).  The loaded words are folded with XOR into one word per workgroup
// so that no load is dead.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "device_common.h"
#include "mfma_common.h"
#include "pc.h"

namespace pcache {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;  // 16-byte loads in flight per lane
constexpr int64_t kStreamStep = (int64_t)kStreamThreads * kStreamUnroll * 16;  // bytes per workgroup iteration

template <int CPOL>
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const char* src, int64_t chunk, int64_t bytes,
                                                                     uint32_t* sink) {
  const int64_t begin = (int64_t)blockIdx.x * chunk;
  const int64_t len = begin >= bytes ? 0 : (bytes - begin < chunk ? bytes - begin : chunk);  // < 2^31
  const __amdgpu_buffer_rsrc_t r = tile_rsrc(src + begin, (uint32_t)len);
  uint32_t acc = 0;
  for (int64_t o = 0; o < len; o += kStreamStep) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u)  // past len the buffer resource returns zeros
      v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           r, (int)(o + ((int64_t)u * kStreamThreads + threadIdx.x) * 16), 0, CPOL));
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  if ((threadIdx.x & (kWave - 1)) == 0) atomicXor(sink + blockIdx.x, acc);
}

}  // namespace
}  // namespace pcache

extern "C" int pc_stream_read(const void* src, int64_t bytes, uint32_t* sink, int num_workgroups, int cache_policy,
                              void* stream) {
  using namespace pcache;
  if (!src || !sink || bytes <= 0 || num_workgroups <= 0 || (cache_policy != 0 && cache_policy != 2))
    return PC_ERR_INVALID_ARG;
  if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0) return PC_ERR_UNSUPPORTED;
  // each workgroup's chunk: whole iterations, addressed with 32-bit buffer offsets
  int64_t chunk = (bytes + num_workgroups - 1) / num_workgroups;
  chunk = (chunk + kStreamStep - 1) / kStreamStep * kStreamStep;
  if (chunk > INT_MAX - kStreamStep) return PC_ERR_UNSUPPORTED;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (cache_policy == 2)
    hipLaunchKernelGGL((stream_read_kernel<2>), dim3(num_workgroups), dim3(kStreamThreads), 0, st,
                       static_cast<const char*>(src), chunk, bytes, sink);
  else
    hipLaunchKernelGGL((stream_read_kernel<0>), dim3(num_workgroups), dim3(kStreamThreads), 0, st,
                       static_cast<const char*>(src), chunk, bytes, sink);
  return hipGetLastError() == hipSuccess ? PC_OK : PC_ERR_LAUNCH;
}
