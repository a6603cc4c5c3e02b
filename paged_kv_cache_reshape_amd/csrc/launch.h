// launch.h -- host-side launchers shared by the C entry points (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pcache {

struct WriteArgs {
  const void* key;
  const void* value;
  int64_t key_row_stride, value_row_stride;  // elements
  void* k_pool;
  void* v_pool;
  int64_t num_blocks, block_stride, token_stride, head_stride;  // elements
  const int64_t* slot_mapping;
  int64_t num_tokens;
  int num_kv_heads, head_size, block_size;
  // 8-bit cache only: head h of K divides by k_scale[h * scale_stride], V likewise
  const float* k_scale;
  const float* v_scale;
  int64_t scale_stride;
};

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  int64_t num_blocks, block_stride, token_stride, head_stride;  // elements
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* seq_lens;
  int num_seqs, num_q_heads, num_kv_heads;
  int block_size;      // tokens per pool block: 8, 16 or 32
  float scale_log2;    // scale * log2(e): scores are kept in the base-2 domain
  int max_partitions;  // split path only
  int max_seq_len;     // host-known bound of seq_lens (the one-pass path picks its kernel from it)
  int longest_first;   // one-pass path: workgroup i takes the i-th longest sequence's units
  float* exp_sums;
  float* max_logits;
  float* tmp_out;
  // 8-bit (OCP E4M3) pool: codes times k_scale / v_scale of the kv head
  int kv8;
  // ALiBi: score of token t for query head h gains alibi_slopes[h] * (t - p), p the query
  // token's position (L - 1 for one token per sequence); NULL: none
  const float* alibi_slopes;
  const float* k_scale;
  const float* v_scale;
  int64_t scale_stride;
  // several query tokens per sequence (one-pass path only): sequence s owns q/out rows
  // [query_start_loc[s], query_start_loc[s+1]) of total_q, its newest tokens; causal:
  // token i of n attends positions <= L - n + i.  NULL: one token per sequence, row s.
  const int32_t* query_start_loc;
  int64_t total_q;
  int causal;
  // the decode step's own K/V write, fused (16-bit pools, one token per sequence):
  // token s = sequence s's newest token, row s of step_key / step_value (elements;
  // [num_seqs, num_kv_heads, head_size] rows), destination step_slots[s].  NULL: none.
  const int64_t* step_slots;
  const void* step_key;
  const void* step_value;
  int64_t step_key_stride, step_value_stride;
  // head size 64 with the kv heads of a token next to each other (head_stride == 64): kv
  // heads 2p and 2p+1 are read as one head of 128 elements and computed together, G query
  // heads each; num_kv_heads and head_stride then count pairs, q / out / partials keep
  // head size 64 (decode_mfma.hip).  0: off.
  int pair;
  // split path with a common prefix (pc_paged_attention_decode_prefix): tokens [0,
  // shared_lens[s]) of sequence s lie in the blocks prefix_table[0 .. prefix_blocks).
  // The partitions those tokens cover completely are computed by the prefix kernel,
  // several sequences per read of each tile, and skipped by the split kernel.  NULL: none.
  const int32_t* prefix_table;
  int prefix_blocks;
  const int32_t* shared_lens;
};

struct VarlenArgs {
  void* out;
  const void* q;  // [total_q, num_q_heads, head_size]
  const void* k_pool;
  const void* v_pool;
  int64_t num_blocks, block_stride, token_stride, head_stride;  // elements
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* query_start_loc;  // [num_reqs + 1]
  const int32_t* seq_lens;         // [num_reqs]
  int num_reqs;
  int64_t total_q;
  int max_query_len;  // sizes the grid; longer requests are still covered
  int num_q_heads, num_kv_heads;
  float scale_log2;
  int causal;
  const float* alibi_slopes;
};

struct ReduceArgs {
  void* out;
  const float* exp_sums;
  const float* max_logits;
  const float* tmp_out;
  const int32_t* seq_lens;
  int num_seqs, num_q_heads, head_size, max_partitions, partition_size;
};

// Each returns hipSuccess or the launch error; `vec16` selects the 16-byte copy path.
hipError_t launch_write(const WriteArgs& a, int dtype, bool vec16, hipStream_t stream);
// The write into an 8-bit (OCP E4M3) pool; `dtype` is the type of key / value.
hipError_t launch_write_fp8(const WriteArgs& a, int dtype, hipStream_t stream);
// Returns hipErrorInvalidValue for a (dtype, head_size, group) the library has no kernel for.
hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_size, bool split, hipStream_t stream);
// The common-prefix units of pc_paged_attention_decode_prefix (fp16 / bf16, 16-token
// blocks).
hipError_t launch_decode_prefix(const DecodeArgs& a, int dtype, int head_size, hipStream_t stream);
// 16-bit storage: q.k on the matrix cores (decode_mfma.hip).
hipError_t launch_decode_mfma(const DecodeArgs& a, int dtype, int head_size, bool split, hipStream_t stream);
// the one-pass decode over several query tokens per request (at most 16 (token, head)
// columns per request and kv head in one pass): 16-bit storage, 16-token blocks
hipError_t launch_decode_multitoken(const VarlenArgs& a, int dtype, int head_size, hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, int dtype, hipStream_t stream);
// Multi-token queries (varlen.hip); 16-bit storage only.
hipError_t launch_varlen(const VarlenArgs& a, int dtype, int head_size, hipStream_t stream);
bool decode_supported(int dtype, int head_size, int group);
bool reduce_supported(int head_size);
// Compute units of the current device (cached per device; 256, MI355X's count, when
// no device can be queried).
int device_compute_units();
// The one-pass path's kernel for a batch of `units` (sequence, kv head) units whose
// longest holds max_seq_len tokens: true for one workgroup per unit (dealt by the
// hardware), false for the persistent, longest-first workgroups (api.hip).
bool onepass_grid(int64_t units, int max_seq_len, int compute_units);

}  // namespace pcache
