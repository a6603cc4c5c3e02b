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

}  // namespace

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
