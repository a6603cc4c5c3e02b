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
//
// A second yardstick, pc_gather_read, reads exactly the K and V tiles a decode of a
// batch reads -- 16 token rows of one kv head per block, through the block table, in
// the split decode's order -- and does nothing else with them: what a plain gather of
// the decode's bytes reaches, against which the decode's own rate can be set.
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

// ---- the decode's tiles, loads only ---------------------------------------------------

constexpr int kGatherWaves = 4;
constexpr int kGatherTiles = 2;     // tiles in flight per wave
constexpr int kGatherSink = 4096;   // words of the caller's sink
constexpr int kTileRows = 16;       // token rows of a tile (16-token blocks)
constexpr int kPartTiles = 32;      // tiles of a 512-token partition

struct GatherArgs {
  const char* k_pool;
  const char* v_pool;
  int64_t num_blocks;
  int64_t block_bytes;  // strides in bytes
  int64_t token_bytes;
  int64_t head_bytes;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* seq_lens;
  int num_seqs;
  int num_kv_heads;
  int parts;  // 512-token partitions of max_seq_len
  uint32_t* sink;
};

// Workgroup = (kv head, sequence, partition), kv head fastest and the last partitions
// first, as the split decode deals them; wave w reads tiles w, w + 4, ... of the
// partition, kGatherTiles at a time.  RB = bytes of one kv head's token row.
template <int RB, int VCPOL>
__global__ __launch_bounds__(kGatherWaves * kWave) void gather_read_kernel(GatherArgs a) {
  constexpr int CPL = kTileRows * RB / 16 / kWave;  // 16-byte pieces of a tile per lane
  static_assert(CPL >= 1 && CPL * kWave * 16 == kTileRows * RB, "a tile is whole 16-byte pieces per lane");
  int64_t id = blockIdx.x;
  const int kvh = (int)(id % a.num_kv_heads);
  id /= a.num_kv_heads;
  const int s = (int)(id % a.num_seqs);
  const int part = a.parts - 1 - (int)(id / a.num_seqs);
  const int L = uniform_load(a.seq_lens, s);
  // a length the table row or max_seq_len cannot hold reads nothing (the decode's NaN case)
  if (L <= 0 || (int64_t)L > (int64_t)a.max_blocks_per_seq * kTileRows || (int64_t)L > (int64_t)a.parts * 512 ||
      part * 512 >= L)
    return;
  const int t0 = part * kPartTiles;
  const int nt = (L + kTileRows - 1) / kTileRows;
  const int t1 = nt < t0 + kPartTiles ? nt : t0 + kPartTiles;
  const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const uint32_t span = (uint32_t)((kTileRows - 1) * a.token_bytes + RB);  // a tile's bytes from its first row
  uint32_t acc = 0;
  for (int t = t0 + w; t < t1; t += kGatherWaves * kGatherTiles) {
    uint4 x[kGatherTiles][2 * CPL];
#pragma unroll
    for (int j = 0; j < kGatherTiles; ++j) {
      const int tj = t + kGatherWaves * j;
      const int b = tj < t1 ? uniform_load(table, tj) : -1;
      const bool ok = b >= 0 && (int64_t)b < a.num_blocks;  // an invalid id or a step past t1: extent 0
      const int64_t off = ok ? (int64_t)b * a.block_bytes + (int64_t)kvh * a.head_bytes : 0;
      const __amdgpu_buffer_rsrc_t kr = tile_rsrc(a.k_pool + off, ok ? span : 0u);
      const __amdgpu_buffer_rsrc_t vr = tile_rsrc(a.v_pool + off, ok ? span : 0u);
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int e = lane + kWave * u;  // piece e: row e / (RB / 16), 16-byte column e % (RB / 16)
        const int o = (int)((e / (RB / 16)) * a.token_bytes) + 16 * (e % (RB / 16));
        x[j][u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, o, 0, 0));
        x[j][CPL + u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, o, 0, VCPOL));
      }
    }
#pragma unroll
    for (int j = 0; j < kGatherTiles; ++j)
#pragma unroll
      for (int u = 0; u < 2 * CPL; ++u) acc ^= x[j][u].x ^ x[j][u].y ^ x[j][u].z ^ x[j][u].w;
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  if (lane == 0) atomicXor(a.sink + (blockIdx.x & (kGatherSink - 1)), acc);
}

template <int RB>
hipError_t launch_gather(const GatherArgs& a, int64_t wgs, int cache_policy, hipStream_t st) {
  if (cache_policy == 2)
    hipLaunchKernelGGL((gather_read_kernel<RB, 2>), dim3((unsigned)wgs), dim3(kGatherWaves * kWave), 0, st, a);
  else
    hipLaunchKernelGGL((gather_read_kernel<RB, 0>), dim3((unsigned)wgs), dim3(kGatherWaves * kWave), 0, st, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace pcache

extern "C" int pc_gather_read(const void* k_pool, const void* v_pool, int64_t num_blocks, int64_t block_stride,
                              int64_t token_stride, int64_t head_stride, const int32_t* block_tables,
                              int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs, int max_seq_len,
                              int num_kv_heads, int head_size, int element_bytes, uint32_t* sink, int v_cache_policy,
                              void* stream) {
  using namespace pcache;
  if (num_seqs < 0 || max_seq_len < 0 || max_blocks_per_seq < 0 || num_kv_heads <= 0 || head_size <= 0 ||
      (element_bytes != 1 && element_bytes != 2 && element_bytes != 4) || (v_cache_policy != 0 && v_cache_policy != 2))
    return PC_ERR_INVALID_ARG;
  if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * kTileRows) return PC_ERR_INVALID_ARG;
  if (num_seqs == 0 || max_seq_len == 0) return PC_OK;
  if (!k_pool || !v_pool || !block_tables || !seq_lens || !sink) return PC_ERR_INVALID_ARG;
  if (num_blocks <= 0 || block_stride <= 0 || token_stride <= 0 || head_stride <= 0) return PC_ERR_INVALID_ARG;
  const int64_t rb = (int64_t)head_size * element_bytes;
  if (rb != 128 && rb != 256 && rb != 512) return PC_ERR_UNSUPPORTED;
  const int64_t eb = element_bytes;
  if ((reinterpret_cast<uintptr_t>(k_pool) & 15u) || (reinterpret_cast<uintptr_t>(v_pool) & 15u) ||
      (block_stride * eb) % 16 || (token_stride * eb) % 16 || (head_stride * eb) % 16)
    return PC_ERR_UNSUPPORTED;
  if (token_stride * eb > INT_MAX / kTileRows) return PC_ERR_UNSUPPORTED;  // tile offsets are 32-bit
  const int parts = (max_seq_len + 511) / 512;
  const int64_t wgs = (int64_t)num_kv_heads * num_seqs * parts;
  if (wgs > INT_MAX) return PC_ERR_UNSUPPORTED;
  GatherArgs a{static_cast<const char*>(k_pool), static_cast<const char*>(v_pool), num_blocks, block_stride * eb,
               token_stride * eb, head_stride * eb, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
               num_kv_heads, parts, sink};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (rb) {
    case 128: e = launch_gather<128>(a, wgs, v_cache_policy, st); break;
    case 256: e = launch_gather<256>(a, wgs, v_cache_policy, st); break;
    default: e = launch_gather<512>(a, wgs, v_cache_policy, st); break;
  }
  return e == hipSuccess ? PC_OK : PC_ERR_LAUNCH;
}

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
