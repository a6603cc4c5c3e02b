// write.hip -- the KV-cache write: scatter new K/V rows into the paged pool.
//
// Follows "Inside vLLM CUDA Kernels: KV-Cache Writes and Paged Attention", Part 2:
// one token's destination is slot_mapping[t]; a negative slot has no destination;
// block = slot / block_size and offset = slot % block_size select the row, and the
// block/token/head strides form the address.  The copy moves raw bits.
//
// MI355X mapping: one 256-thread workgroup per token; its K row and V row are cut
// into 16-byte vectors spread over the 256 lanes, so a wave's 64 lanes touch 1 KiB
// of contiguous source and, per head, contiguous destination bytes.  The pages'
// two copy paths (whole-row span vs one warp per head) collapse into one: every
// 16-byte vector computes its own head offset, which costs a divide per vector and
// coalesces the same way for NHD and HND.  A pool or stride that is not 16-byte
// aligned falls back to element-sized copies.
//
// 8-bit cache (same page, "Why Layout and Quantization Scale Produce Two Copy
// Paths": the conversion applies the head's scale -- k_scale[h * kv_scale_stride],
// one shared scale when the stride is 0): each element x becomes the OCP E4M3 code
// of x / scale, computed in fp32 with IEEE division, clamped to +-448 (the largest
// finite code; NaN stays NaN) and rounded to nearest-even by v_cvt_pk_fp8_f32, four
// elements to one 32-bit store.
#include "device_common.h"
#include "launch.h"

namespace pcache {
namespace {

constexpr int kWriteThreads = 256;

template <int ES, bool VEC>
__global__ __launch_bounds__(kWriteThreads) void write_kernel(WriteArgs a) {
  using Vec = typename std::conditional<VEC, uint4, typename std::conditional<ES == 4, uint32_t, uint16_t>::type>::type;
  constexpr int kElems = VEC ? 16 / ES : 1;  // elements per moved vector

  const int64_t t = blockIdx.x;
  const int64_t slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.num_blocks * a.block_size) return;  // padding (or outside the pool): no destination
  const int64_t blk = slot / a.block_size;
  const int64_t off = slot - blk * a.block_size;
  const int64_t dst_row = blk * a.block_stride + off * a.token_stride;  // elements

  const int per_head = a.head_size / kElems;
  const int per_row = a.num_kv_heads * per_head;
  const char* ksrc = static_cast<const char*>(a.key) + t * a.key_row_stride * ES;
  const char* vsrc = static_cast<const char*>(a.value) + t * a.value_row_stride * ES;
  char* kdst = static_cast<char*>(a.k_pool) + dst_row * ES;
  char* vdst = static_cast<char*>(a.v_pool) + dst_row * ES;

  for (int c = threadIdx.x; c < 2 * per_row; c += kWriteThreads) {
    const bool is_v = c >= per_row;
    const int cc = is_v ? c - per_row : c;
    const int h = cc / per_head;
    const int e = (cc - h * per_head) * kElems;
    const int64_t src_off = ((int64_t)h * a.head_size + e) * ES;
    const int64_t dst_off = ((int64_t)h * a.head_stride + e) * ES;
    const Vec v = *reinterpret_cast<const Vec*>((is_v ? vsrc : ksrc) + src_off);
    *reinterpret_cast<Vec*>((is_v ? vdst : kdst) + dst_off) = v;
  }
}

template <class SRC>
__device__ __forceinline__ float src_elem(const void* base, int64_t i);
template <>
__device__ __forceinline__ float src_elem<F32>(const void* base, int64_t i) {
  return static_cast<const float*>(base)[i];
}
template <>
__device__ __forceinline__ float src_elem<F16>(const void* base, int64_t i) {
  return (float)static_cast<const _Float16*>(base)[i];
}
template <>
__device__ __forceinline__ float src_elem<BF16>(const void* base, int64_t i) {
  return __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[i] << 16);
}

// x / scale clamped into the finite E4M3 range (NaN passes through)
__device__ __forceinline__ float fp8_arg(float x, float scale) {
  const float y = x / scale;
  return __builtin_isnan(y) ? y : fminf(fmaxf(y, -448.f), 448.f);
}

template <class SRC>
__global__ __launch_bounds__(kWriteThreads) void write_fp8_kernel(WriteArgs a) {
  const int64_t t = blockIdx.x;
  const int64_t slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.num_blocks * a.block_size) return;  // padding (or outside the pool): no destination
  const int64_t blk = slot / a.block_size;
  const int64_t off = slot - blk * a.block_size;
  const int64_t dst_row = blk * a.block_stride + off * a.token_stride;  // bytes
  const int quads = a.head_size / 4;  // 4 codes per 32-bit store
  const int per_row = a.num_kv_heads * quads;
  for (int c = threadIdx.x; c < 2 * per_row; c += kWriteThreads) {
    const bool is_v = c >= per_row;
    const int cc = is_v ? c - per_row : c;
    const int h = cc / quads;
    const int e = (cc - h * quads) * 4;
    const float sc = (is_v ? a.v_scale : a.k_scale)[(int64_t)h * a.scale_stride];
    const void* src = is_v ? a.value : a.key;
    const int64_t si = t * (is_v ? a.value_row_stride : a.key_row_stride) + (int64_t)h * a.head_size + e;
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_arg(src_elem<SRC>(src, si), sc),
                                                fp8_arg(src_elem<SRC>(src, si + 1), sc), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_arg(src_elem<SRC>(src, si + 2), sc),
                                       fp8_arg(src_elem<SRC>(src, si + 3), sc), w, true);
    uint8_t* dst = static_cast<uint8_t*>(is_v ? a.v_pool : a.k_pool) + dst_row + (int64_t)h * a.head_stride + e;
    *reinterpret_cast<uint32_t*>(dst) = w;
  }
}

}  // namespace

hipError_t launch_write_fp8(const WriteArgs& a, int dtype, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const dim3 grid((unsigned)a.num_tokens), block(kWriteThreads);
  switch (dtype) {
    case 0: hipLaunchKernelGGL((write_fp8_kernel<F32>), grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL((write_fp8_kernel<F16>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((write_fp8_kernel<BF16>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_write(const WriteArgs& a, int dtype, bool vec16, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const dim3 grid((unsigned)a.num_tokens), block(kWriteThreads);
  const int es = dtype == 0 ? 4 : 2;
  if (vec16) {
    if (es == 4)
      hipLaunchKernelGGL((write_kernel<4, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((write_kernel<2, true>), grid, block, 0, stream, a);
  } else {
    if (es == 4)
      hipLaunchKernelGGL((write_kernel<4, false>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((write_kernel<2, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pcache
