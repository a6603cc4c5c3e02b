// noalloc.hip -- the split decode and its reduce with the partial results in a buffer
// the library holds, for callers that cannot allocate device memory (code under HIP
// graph capture, serving loops that forbid allocation).
//
// The buffer is a file-scope device array; each GPU the library runs on holds its own
// copy, at its own address, from the first use until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is only a stand-in): the
// device address comes from hipGetSymbolAddress, once per device, with that device
// current, and is kept per device.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <mutex>

#include "launch.h"
#include "pc.h"

namespace {

constexpr int64_t kScratchFloats = PC_NOALLOC_SCRATCH_BYTES / sizeof(float);
static_assert(PC_NOALLOC_SCRATCH_BYTES % 256 == 0, "the partials are carved in 256-byte multiples");

// tmp_out, then exp_sums, then max_logits of the split path.  Nothing in it has to
// start at zero: the decode writes every partition that holds tokens and the reduce
// reads only those.
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device (looked up on its first call
// there), or nullptr with the HIP error cleared.
float* scratch_on_current_device() {
  static std::mutex mu;
  static float* addr[kMaxDevices] = {nullptr};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[dev] = static_cast<float*>(p);
  }
  return addr[dev];
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

extern "C" int pc_paged_attention_split_noalloc(void* out, const void* q, const void* k_pool, const void* v_pool,
                                                int64_t num_blocks, int64_t block_stride, int64_t token_stride,
                                                int64_t head_stride, const int32_t* block_tables,
                                                int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs,
                                                int max_seq_len, int num_q_heads, int num_kv_heads, int head_size,
                                                int block_size, float scale, const float* alibi_slopes, int dtype,
                                                void* stream) {
  if (num_seqs < 0 || max_seq_len < 0 || num_q_heads <= 0 || head_size <= 0) return PC_ERR_INVALID_ARG;
  if (num_seqs == 0) return PC_OK;
  if (!out) return PC_ERR_INVALID_ARG;
  if (!pcache::reduce_supported(head_size)) return PC_ERR_UNSUPPORTED;
  const int64_t parts = (max_seq_len + PC_PARTITION_SIZE - 1) / PC_PARTITION_SIZE;
  const int64_t rows = (int64_t)num_seqs * num_q_heads * parts;  // (s, h, p) partials
  // each piece starts on a 256-byte boundary (64 floats)
  const int64_t tmp_floats = round_up(rows * head_size, 64);
  const int64_t stat_floats = round_up(rows, 64);
  if (tmp_floats + 2 * stat_floats > kScratchFloats) return PC_ERR_TOO_LARGE;
  float* base = scratch_on_current_device();
  if (!base) return PC_ERR_LAUNCH;
  float* tmp_out = base;
  float* exp_sums = base + tmp_floats;
  float* max_logits = exp_sums + stat_floats;
  const int rc = pc_paged_attention_decode(nullptr, q, k_pool, v_pool, num_blocks, block_stride, token_stride,
                                           head_stride, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                                           max_seq_len, num_q_heads, num_kv_heads, head_size, block_size, scale,
                                           PC_PARTITION_SIZE, exp_sums, max_logits, tmp_out, alibi_slopes, dtype,
                                           stream);
  if (rc != PC_OK) return rc;
  return pc_paged_attention_reduce(out, exp_sums, max_logits, tmp_out, seq_lens, num_seqs, num_q_heads, head_size,
                                   (int)parts, PC_PARTITION_SIZE, dtype, stream);
}
