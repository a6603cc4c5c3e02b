/*
 * pc.h -- C ABI of the paged KV-cache library for AMD Instinct MI355X (gfx950).
 *
 * Three operations form the data-parallel hot path of a paged KV cache at decode
 * time, plus a host-only planner:
 *
 *   pc_reshape_and_cache       scatter each new token's K/V rows into a pool of
 *                              fixed-size physical blocks through slot_mapping;
 *   pc_paged_attention_decode  for every (sequence, query head): walk the block
 *                              table, gather K/V, scaled q.k scores, online softmax,
 *                              softmax . V -- either in one pass, or per 512-token
 *                              partition writing partial results;
 *   pc_paged_attention_reduce  merge the partitions' partial results (log-sum-exp);
 *   pc_paged_attention_decode_prefix  the split path for sequences sharing a prefix,
 *                              each shared tile read once for many sequences;
 *   pc_paged_attention_plan    choose between the one-pass and the split path;
 *   pc_paged_attention_varlen  several query tokens per request (chunked prefill,
 *                              speculative decode) over the same paged history;
 *   pc_reshape_and_cache_decode  a whole decode step -- the write and the decode
 *                              -- in one launch.
 *
 * The write and the decode also exist for an 8-bit cache (suffix _fp8): the pool
 * holds OCP E4M3 codes with one dequantisation scale per kv head for K and one
 * for V (see pc_reshape_and_cache_fp8).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every data pointer is a DEVICE pointer (hipMalloc'd or equivalent),
 *   except the out-parameters of pc_paged_attention_plan, which are host pointers.
 *   The caller owns every buffer, allocates the split workspace (sizes from
 *   pc_paged_attention_plan) and keeps it alive until the stream has executed the
 *   call.  The library allocates no memory and keeps no state beyond cached
 *   device-property and symbol-address queries; the one device buffer it holds is
 *   a static array of its code object (see pc_paged_attention_split_noalloc).
 * Streams.  `stream` is a hipStream_t (NULL = the legacy default stream).  All
 *   device work is enqueued on it and nothing waits for it; a write followed by a
 *   decode on the same stream sees the written tokens.
 * Storage types.  q, out, key/value rows and the pool share one storage type
 *   (pc_dtype); arithmetic is fp32 throughout (scores, softmax statistics and the
 *   value accumulator); out is rounded to nearest-even from fp32.
 * Pool layout.  A pool is described by ELEMENT strides (block_stride,
 *   token_stride, head_stride); the head_size dimension is contiguous.  Examples:
 *     HND  [num_blocks, num_kv_heads, block_size, head_size]:
 *          {Hkv*B*D, D, B*D}   (the layout this library is tuned for)
 *     NHD  [num_blocks, block_size, num_kv_heads, head_size]:
 *          {B*Hkv*D, Hkv*D, D}
 *     one buffer per block holding K for B tokens then V for B tokens
 *     ("Splitting the KV cache into 16-token blocks", section "What one block
 *     holds"): v_pool = k_pool + B*Hkv*D elements, strides {2*B*Hkv*D, Hkv*D, D}.
 *   K and V use the same strides.  Element addresses are formed in 64 bits; the
 *   decode additionally needs 16 * token_stride * element size < 2^31 (else
 *   PC_ERR_UNSUPPORTED).
 * Alignment.  The kernels move 16-byte vectors: pool bases, q, key/value rows,
 *   and every stride times the element size must be multiples of 16 bytes, and
 *   head_size * element size a multiple of 16 (else PC_ERR_UNSUPPORTED).
 * Errors.  Arguments are validated on the host before anything is enqueued; a
 *   failing check returns a negative status and launches nothing.  Data values
 *   (slots, block ids, lengths) live in device memory and are checked by the
 *   kernels: an out-of-range slot is skipped like a negative one; a sequence
 *   whose length exceeds its table row (or max_seq_len on the split path) or
 *   whose table names a block outside [0, num_blocks) gets NaN in every output
 *   element of its heads instead of an out-of-bounds read.
 * Concurrency.  Calls on different streams that write the same pool slots or
 *   outputs race; slot_mapping must not name one slot twice in a call.
 */
#ifndef PC_H
#define PC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type shared by q, out, key/value and the pool. */
typedef enum { PC_F32 = 0, PC_F16 = 1, PC_BF16 = 2 } pc_dtype;

/* Status codes. */
#define PC_OK 0
#define PC_ERR_INVALID_ARG (-1) /* a null pointer, negative size, or inconsistent sizes */
#define PC_ERR_UNSUPPORTED (-2) /* a valid request the library has no kernel for */
#define PC_ERR_LAUNCH (-3)      /* the HIP runtime refused the launch */
#define PC_ERR_TOO_LARGE (-4)   /* the request needs more than the library's fixed buffer holds */

/* Tokens per partition on the split path. */
#define PC_PARTITION_SIZE 512

/* Version of this ABI (bumped on any signature change). */
int pc_abi_version(void);

/* Short static description of a status code. */
const char *pc_status_string(int status);

/*
 * pc_reshape_and_cache -- write new K/V rows into the paged pool.
 *
 * Defined by "Inside vLLM CUDA Kernels: KV-Cache Writes and Paged Attention",
 * Part 2, sections "Decomposing a Slot into Block and Offset" and "Why Layout and
 * Quantization Scale Produce Two Copy Paths", and "How vLLM CUDA Kernels Write
 * and Read the Paged KV Cache", section "Writing K and V into the cache": token t
 * goes to slot = slot_mapping[t]; a negative slot means the token has no
 * destination (padding) and nothing is written; otherwise block = slot /
 * block_size, offset = slot % block_size, and for every kv head h and dimension d
 *     k_pool[block*block_stride + offset*token_stride + h*head_stride + d]
 *         = key[t*key_row_stride + h*head_size + d]
 * and the same for value into v_pool.  Bits are copied unchanged (no rounding,
 * NaN payloads survive).
 *
 *   key, value        device, rows of num_kv_heads*head_size elements, row t at
 *                     t*key_row_stride / t*value_row_stride elements
 *   k_pool, v_pool    device pool bases (may lie in one buffer, see Pool layout)
 *   num_blocks        physical blocks in the pool; slots >= num_blocks*block_size
 *                     are skipped
 *   slot_mapping      device int64 [num_tokens]
 *   block_size        tokens per physical block (any positive value)
 * Returns PC_OK, PC_ERR_INVALID_ARG, PC_ERR_UNSUPPORTED or PC_ERR_LAUNCH.
 * num_tokens == 0 is a valid no-op.
 */
int pc_reshape_and_cache(const void *key, const void *value, int64_t key_row_stride, int64_t value_row_stride,
                         void *k_pool, void *v_pool, int64_t num_blocks, int64_t block_stride,
                         int64_t token_stride, int64_t head_stride, const int64_t *slot_mapping,
                         int64_t num_tokens, int num_kv_heads, int head_size, int block_size, int dtype,
                         void *stream);

/*
 * pc_paged_attention_decode -- one query token per sequence against its paged
 * history.
 *
 * Defined by "vLLM 源码完全拆解（七）: PagedAttention Kernel", sections
 * 先明确问题 (decode attention of query head h of sequence s over its L_s visible
 * tokens), 线程组织 (query head h reads kv head h / (num_q_heads/num_kv_heads)),
 * 第一步 (positions >= seq_len take no part), V1与V2 (512-token partitions, a
 * partition past seq_len does nothing), and "Inside vLLM CUDA Kernels", Part 3,
 * section "How Each K/V Tile Contributes to the Output" (scores = q.k * scale,
 * online softmax with running max, sum and accumulator, output acc / l).  Logical
 * token t of sequence s lives in physical block block_tables[s*max_blocks_per_seq
 * + t/block_size] at offset t%block_size ("How vLLM CUDA Kernels Write and Read
 * the Paged KV Cache", section "Reading logical blocks during attention").
 *
 *   out               device [num_seqs, num_q_heads, head_size] (one-pass path only)
 *   q                 device [num_seqs, num_q_heads, head_size], contiguous
 *   k_pool, v_pool    device pool bases; num_blocks and strides as for the write
 *   block_tables      device int32 [num_seqs, max_blocks_per_seq]; entries past
 *                     ceil(seq_len/16) are never read (padding, e.g. -1)
 *   seq_lens          device int32 [num_seqs]; must include this step's token
 *   max_seq_len       host-known upper bound of seq_lens (sizes the split grid)
 *   num_q_heads       multiple of num_kv_heads; num_q_heads/num_kv_heads in {1,2,4,8}
 *                     for fp16/bf16, {1,2,4} for fp32
 *   head_size         64 or 128
 *   block_size        8, 16 or 32 for fp16/bf16 (and the 8-bit cache); 16 for fp32
 *                     ("vLLM 源码完全拆解（七）", section GQA、向量化加载与 Block Size
 *                     的联动: the block size trades fragmentation against table reads)
 *   scale             multiplies q.k (typically 1/sqrt(head_size)); positive, finite
 *   partition_size    0: one pass, writes out.  PC_PARTITION_SIZE: split path,
 *                     writes only exp_sums, max_logits and tmp_out; follow with
 *                     pc_paged_attention_reduce on the same stream.
 *   exp_sums          device fp32 [num_seqs, num_q_heads, P] with
 *   max_logits        P = ceil(max_seq_len / partition_size): per partition, the
 *   tmp_out           sum of exp(score - max), the max score (natural-log domain)
 *                     and the normalised partial output [.., P, head_size].
 *                     Partitions past a sequence's length are not written.
 *                     All three must be NULL when partition_size == 0.
 *   alibi_slopes      NULL (no positional bias) or device fp32 [num_q_heads]: the
 *                     ALiBi bias of "vLLM 源码完全拆解（七）", section 第一步 -- the
 *                     score of token t of query head h becomes scale * q.k_t +
 *                     alibi_slopes[h] * (t - (seq_len - 1)) before the softmax (zero
 *                     at the newest token, the negative distance times the slope
 *                     before it).  The split partials' max_logits include the bias.
 * A sequence with seq_len 0 gets zeros (one pass) or no partials (split).
 * Returns PC_OK, PC_ERR_INVALID_ARG, PC_ERR_UNSUPPORTED or PC_ERR_LAUNCH.
 */
int pc_paged_attention_decode(void *out, const void *q, const void *k_pool, const void *v_pool,
                              int64_t num_blocks, int64_t block_stride, int64_t token_stride,
                              int64_t head_stride, const int32_t *block_tables, int max_blocks_per_seq,
                              const int32_t *seq_lens, int num_seqs, int max_seq_len, int num_q_heads,
                              int num_kv_heads, int head_size, int block_size, float scale, int partition_size,
                              float *exp_sums, float *max_logits, float *tmp_out, const float *alibi_slopes,
                              int dtype, void *stream);

/*
 * pc_paged_attention_decode_prefix -- the split path's decode for a batch whose
 * sequences share a common prefix: the same partials as pc_paged_attention_decode with
 * partition_size = PC_PARTITION_SIZE, computed with one read of each prefix tile for
 * many sequences at once.
 *
 * Sequences that share a prefix point their first table entries at the same physical
 * blocks ("PagedAttention kernel: paged KV cache & block tables", section Interviewer
 * follow-ups).  Each such block is then read by every sharing sequence.  Here the
 * caller names the shared blocks.  For every partition that a sequence's shared tokens
 * cover completely, one workgroup per kv head computes that partition's partials for
 * 16 / G sequences at once (G query heads per kv head): each K/V tile is read once and
 * scored against all their queries.  The remaining partitions run as on the split path.
 * Follow with pc_paged_attention_reduce as usual.  The results are the split path's, up
 * to rounding.
 *
 *   all arguments but the three below: as for pc_paged_attention_decode with
 *                       partition_size = PC_PARTITION_SIZE (exp_sums, max_logits and
 *                       tmp_out required, [num_seqs, num_q_heads, P(, head_size)])
 *   prefix_table        device int32 [prefix_blocks]: the shared blocks, in token order
 *   prefix_blocks       >= 0; 0: no prefix (exactly the split decode)
 *   shared_lens         device int32 [num_seqs]: sequence s's tokens [0, shared_lens[s])
 *                       lie in prefix_table's blocks, i.e. its table's first
 *                       ceil(shared_lens[s] / 16) entries equal prefix_table's; 0 for a
 *                       sequence that shares nothing.  Must not exceed seq_lens[s] or
 *                       prefix_blocks * 16.
 * fp16 / bf16 pools of 16-token blocks with a prefix (else PC_ERR_UNSUPPORTED).  A
 * sequence whose shared_lens entry exceeds its length or the prefix, or whose table
 * differs from prefix_table over a partition its shared tokens cover, gets NaN
 * partials there (so NaN outputs after the reduce) instead of a wrong value.
 * Returns PC_OK, PC_ERR_INVALID_ARG, PC_ERR_UNSUPPORTED or PC_ERR_LAUNCH.
 */
int pc_paged_attention_decode_prefix(const void *q, const void *k_pool, const void *v_pool, int64_t num_blocks,
                                     int64_t block_stride, int64_t token_stride, int64_t head_stride,
                                     const int32_t *block_tables, int max_blocks_per_seq, const int32_t *seq_lens,
                                     int num_seqs, int max_seq_len, int num_q_heads, int num_kv_heads, int head_size,
                                     int block_size, float scale, float *exp_sums, float *max_logits, float *tmp_out,
                                     const float *alibi_slopes, const int32_t *prefix_table, int prefix_blocks,
                                     const int32_t *shared_lens, int dtype, void *stream);

/*
 * pc_reshape_and_cache_fp8 -- write new K/V rows into an 8-bit (OCP E4M3) pool.
 *
 * Defined by "Inside vLLM CUDA Kernels", Part 2, "Why Layout and Quantization
 * Scale Produce Two Copy Paths" (an 8-bit cache stores each element converted with
 * a scale; the per-head form reads the scale of head h at h * kv_scale_stride, the
 * shared form passes stride 0) and the slot rules of pc_reshape_and_cache.  For
 * every written element x of kv head h the pool byte becomes the E4M3 code of
 * y = x / k_scale[h * kv_scale_stride] (V: v_scale), where the division is fp32
 * (correctly rounded), y is clamped to [-448, 448] (the largest finite E4M3
 * magnitude; E4M3 has no infinity), and the code is y rounded to nearest-even.
 * NaN becomes the NaN code 0xFF.  A code c stands for E4M3(c) * scale.
 *
 *   key, value          device, storage dtype (fp32, fp16 or bf16), rows as for
 *                       pc_reshape_and_cache (element strides)
 *   k_pool, v_pool      device uint8 pools; strides in bytes (= elements)
 *   k_scale, v_scale    device fp32, read at h * kv_scale_stride for h < num_kv_heads
 *   kv_scale_stride     >= 0 (0: one scale for every head)
 * Pools, block_stride, token_stride and head_stride must be multiples of 4 bytes
 * and head_size a multiple of 4 (four codes per store; else PC_ERR_UNSUPPORTED).
 * Returns PC_OK, PC_ERR_INVALID_ARG, PC_ERR_UNSUPPORTED or PC_ERR_LAUNCH.
 */
int pc_reshape_and_cache_fp8(const void *key, const void *value, int64_t key_row_stride, int64_t value_row_stride,
                             uint8_t *k_pool, uint8_t *v_pool, int64_t num_blocks, int64_t block_stride,
                             int64_t token_stride, int64_t head_stride, const int64_t *slot_mapping,
                             int64_t num_tokens, int num_kv_heads, int head_size, int block_size,
                             const float *k_scale, const float *v_scale, int64_t kv_scale_stride, int dtype,
                             void *stream);

/*
 * pc_paged_attention_decode_fp8 -- pc_paged_attention_decode over an 8-bit pool.
 *
 * Same operation and arguments as pc_paged_attention_decode, with K and V the
 * dequantised pool values: token row element d of kv head h is E4M3(code) *
 * k_scale[h * kv_scale_stride] for K and E4M3(code) * v_scale[...] for V (the
 * scaled conversion of "Why Layout and Quantization Scale Produce Two Copy Paths"
 * read back).  q and out are fp16 or bf16 (fp32 gives PC_ERR_UNSUPPORTED); the
 * split path's partials and pc_paged_attention_reduce are unchanged.
 *
 *   k_pool, v_pool    device uint8 pools written by pc_reshape_and_cache_fp8;
 *                     strides in bytes, multiples of 16; pool bases 16-byte aligned
 *   k_scale, v_scale  device fp32 as for the write; each used scale must be
 *                     positive and finite with scale * k_scale * log2(e) in
 *                     [2^-120, 2^120], else that kv head's outputs are NaN
 * Returns PC_OK, PC_ERR_INVALID_ARG, PC_ERR_UNSUPPORTED or PC_ERR_LAUNCH.
 */
int pc_paged_attention_decode_fp8(void *out, const void *q, const uint8_t *k_pool, const uint8_t *v_pool,
                                  int64_t num_blocks, int64_t block_stride, int64_t token_stride,
                                  int64_t head_stride, const int32_t *block_tables, int max_blocks_per_seq,
                                  const int32_t *seq_lens, int num_seqs, int max_seq_len, int num_q_heads,
                                  int num_kv_heads, int head_size, int block_size, float scale,
                                  int partition_size, float *exp_sums, float *max_logits, float *tmp_out,
                                  const float *alibi_slopes, const float *k_scale, const float *v_scale,
                                  int64_t kv_scale_stride, int dtype, void *stream);

/*
 * pc_reshape_and_cache_decode -- one decode step in one launch: the write of
 * pc_reshape_and_cache for this step's tokens, then pc_paged_attention_decode,
 * with the result of running the two in that order on one stream.
 *
 * The operations are the two defined above (same passages).  Token s of the step
 * is sequence s's newest token (num_tokens == num_seqs): its K/V row goes to
 * slot_mapping[s], which must be the slot of position seq_lens[s] - 1 of sequence s
 * (its block block_tables[s*max_blocks_per_seq + (seq_lens[s]-1)/block_size], offset
 * (seq_lens[s]-1) % block_size), or outside the pool (negative: padding, nothing is
 * written, and the decode reads whatever the pool holds there).  The workgroup that
 * decodes the tile holding that position stores the row, waits for the stores to
 * complete, and only then reads the tile, so the decode sees the new row.  A slot
 * inside the pool that is not that position is an invalid step for the sequence:
 * nothing is written for it and its outputs (or split partials) are NaN; a sequence
 * of length 0 has no such position, writes nothing and decodes as empty.  No other
 * sequence may read the written slots in this step (true of a decode step: every
 * sequence appends to its own last block), since only the writer's reads are ordered
 * after the write.
 *
 *   out, q, k_pool ... partition_size, exp_sums, max_logits, tmp_out, alibi_slopes:
 *                     as for pc_paged_attention_decode (16-bit storage: fp16 or bf16;
 *                     fp32, and block_size 8 with num_q_heads == 8 * num_kv_heads at
 *                     head_size 128, give PC_ERR_UNSUPPORTED); the pools are written
 *   key, value        device [num_seqs, num_kv_heads, head_size] rows at
 *   key_row_stride,   key_row_stride / value_row_stride elements, q's type,
 *   value_row_stride  16-byte aligned rows (else PC_ERR_UNSUPPORTED)
 *   slot_mapping      device int64 [num_seqs]
 * Returns PC_OK, PC_ERR_INVALID_ARG, PC_ERR_UNSUPPORTED or PC_ERR_LAUNCH.
 */
int pc_reshape_and_cache_decode(void *out, const void *q, const void *key, const void *value, int64_t key_row_stride,
                                int64_t value_row_stride, const int64_t *slot_mapping, void *k_pool, void *v_pool,
                                int64_t num_blocks, int64_t block_stride, int64_t token_stride, int64_t head_stride,
                                const int32_t *block_tables, int max_blocks_per_seq, const int32_t *seq_lens,
                                int num_seqs, int max_seq_len, int num_q_heads, int num_kv_heads, int head_size,
                                int block_size, float scale, int partition_size, float *exp_sums, float *max_logits,
                                float *tmp_out, const float *alibi_slopes, int dtype, void *stream);

/*
 * pc_paged_attention_varlen -- attention of several new query tokens per request
 * over the paged history.
 *
 * Defined by "Inside vLLM CUDA Kernels", Part 3, sections "How Metadata Connects a Q
 * Tile to Paged K/V" (query_start_loc delimits each request's rows of the packed
 * query, seq_lens its visible KV length, block_table its pages; the kernel resolves
 * pages as it scans the K dimension) and "How Each K/V Tile Contributes to the
 * Output" (online softmax over the K/V tiles).  Request r owns rows
 * [query_start_loc[r], query_start_loc[r+1]) of q and out: its newest n_r tokens,
 * whose K/V must already be in the cache, so query token i sits at position
 * p = seq_lens[r] - n_r + i.  causal = 1: it attends positions t <= p; causal = 0:
 * all of [0, seq_lens[r]).  Scores scale * q.k_t (+ alibi_slopes[h] * (t - p) when
 * given), softmax, times V, as for the decode; n_r = 1 with causal = 1 is the decode.
 *
 *   out, q            device [total_q, num_q_heads, head_size], fp16 or bf16,
 *                     16-byte aligned (fp32 gives PC_ERR_UNSUPPORTED)
 *   k_pool ... block_tables, block_size, head_size, groups: as for the decode
 *   query_start_loc   device int32 [num_reqs + 1], non-decreasing, from 0 to total_q
 *   seq_lens          device int32 [num_reqs], seq_lens[r] >= n_r
 *   max_query_len     host upper bound of n_r (sizes the grid; a longer request is
 *                     still computed, more slowly)
 *   causal            0 or 1
 *   alibi_slopes      NULL or device fp32 [num_q_heads]
 * A request whose row range leaves [0, total_q] or is decreasing has its rows left
 * unwritten; one with seq_len < n_r, a length past its table row or a block id
 * outside the pool gets NaN in its rows.
 * Returns PC_OK, PC_ERR_INVALID_ARG, PC_ERR_UNSUPPORTED or PC_ERR_LAUNCH.
 */
int pc_paged_attention_varlen(void *out, const void *q, const void *k_pool, const void *v_pool, int64_t num_blocks,
                              int64_t block_stride, int64_t token_stride, int64_t head_stride,
                              const int32_t *block_tables, int max_blocks_per_seq, const int32_t *query_start_loc,
                              const int32_t *seq_lens, int num_reqs, int64_t total_q, int max_query_len,
                              int num_q_heads, int num_kv_heads, int head_size, int block_size, float scale,
                              int causal, const float *alibi_slopes, int dtype, void *stream);

/*
 * pc_paged_attention_reduce -- merge the split path's partials.
 *
 * Defined by "Inside vLLM CUDA Kernels", Part 3, section "How Each K/V Tile
 * Contributes to the Output" (partial states rescaled to a common maximum before
 * merging) and "vLLM 源码完全拆解（七）", section V1与V2 (a second kernel merges
 * the partitions).  For each (s, h), over the n = ceil(seq_len/partition_size)
 * partitions that hold tokens: M = max max_logits, w_p = exp_sums_p *
 * exp(max_logits_p - M), out = sum_p w_p tmp_out_p / sum_p w_p.  Only those n
 * partitions are read.  seq_len 0 gives zeros; n > max_num_partitions gives NaN.
 *
 *   out                device [num_seqs, num_q_heads, head_size], storage dtype
 *   exp_sums ...       device fp32, as written by pc_paged_attention_decode
 *   max_num_partitions P of the decode call; partition_size PC_PARTITION_SIZE;
 *                      tmp_out 16-byte aligned (as for the decode)
 * Returns PC_OK, PC_ERR_INVALID_ARG, PC_ERR_UNSUPPORTED or PC_ERR_LAUNCH.
 */
int pc_paged_attention_reduce(void *out, const float *exp_sums, const float *max_logits, const float *tmp_out,
                              const int32_t *seq_lens, int num_seqs, int num_q_heads, int head_size,
                              int max_num_partitions, int partition_size, int dtype, void *stream);

/*
 * pc_paged_attention_plan -- pick the decode path for a batch (host only, no
 * device work).
 *
 * The pages' rule of thumb trades the one-pass path's idle compute units when
 * sequences are few and long against the split path's extra launch and partial
 * traffic ("vLLM 源码完全拆解（七）", section V1与V2).  This planner estimates both
 * paths' times from a model of the library's kernels fitted to measurements on
 * MI355X (see pc_paged_attention_plan_lens), taking every sequence to be max_seq_len
 * long; work units are (sequence, kv head) -- every query head of a group is computed
 * from one read of its K/V.  A caller that knows the lengths should use
 * pc_paged_attention_plan_lens: a skewed batch can favour the other path.
 *
 *   partition_size      out: 0 (one pass) or PC_PARTITION_SIZE (split)
 *   max_num_partitions  out: P for the split path (1 for one pass)
 *   workspace_bytes     out: bytes of exp_sums + max_logits + tmp_out the split
 *                       path needs (0 for one pass)
 * Any out-pointer may be NULL.  Returns PC_OK or PC_ERR_INVALID_ARG.
 */
int pc_paged_attention_plan(int num_seqs, int num_q_heads, int num_kv_heads, int head_size, int max_seq_len,
                            int dtype, int *partition_size, int *max_num_partitions, size_t *workspace_bytes);

/*
 * pc_paged_attention_plan_lens -- pc_paged_attention_plan for a batch whose sequence
 * lengths the host knows (a serving scheduler does: it builds slot_mapping from them).
 *
 * The same choice as pc_paged_attention_plan ("vLLM 源码完全拆解（七）", section
 * V1与V2: idle compute units with few long sequences against the split path's second
 * launch and partial traffic), made from the lengths themselves rather than from their
 * maximum: how the lengths are spread decides how evenly the one-pass workgroups are
 * loaded, and with it which path is faster.  The library estimates both paths' launch
 * times from a model of its kernels fitted to measurements on MI355X and returns the
 * faster.  With partition_size 0 the decode itself picks its one-pass kernel from the
 * unit count (num_seqs * num_kv_heads) and max_seq_len: one workgroup per unit when
 * max_seq_len <= 512, or for at least 32 units per compute unit with max_seq_len <=
 * 2048 (16-bit pools); persistent, longest-first workgroups otherwise.  pc_paged_attention_plan applies the same model with every sequence taken
 * to be max_seq_len long.
 *
 *   seq_lens            HOST int32 [num_seqs], each >= 0 (the decode's seq_lens)
 *   shared_lens         NULL, or HOST int32 [num_seqs]: how many leading tokens of each
 *                       sequence sit in blocks that other sequences of the batch also read
 *                       (a shared prefix, "PagedAttention kernel: paged KV cache & block
 *                       tables", section Interviewer follow-ups: sequences sharing a
 *                       prefix point at the same physical blocks); 0 <= shared_lens[s] <=
 *                       seq_lens[s].  Shared tokens come partly from cache on the one-pass
 *                       path; given them, the split estimate is for
 *                       pc_paged_attention_decode_prefix (the partitions they cover
 *                       completely read once for many sequences), the path a caller that
 *                       knows its sharing runs.
 *   head_stride         the pool's head_stride in elements (the decode computes pairs of
 *                       kv heads together when head_size is 64 and the heads of a token
 *                       are adjacent; the plan accounts for it)
 *   kv_fp8              1 for an 8-bit pool (pc_paged_attention_decode_fp8), else 0
 *   partition_size ...  out, as for pc_paged_attention_plan (max_seq_len = the largest
 *                       seq_lens entry)
 * Host only: no device work, no allocation visible to the caller.  Returns PC_OK or
 * PC_ERR_INVALID_ARG (a negative length, a shared count outside [0, seq_len], a NULL
 * seq_lens with num_seqs > 0, bad sizes).
 */
int pc_paged_attention_plan_lens(const int32_t *seq_lens, const int32_t *shared_lens, int num_seqs, int num_q_heads,
                                 int num_kv_heads, int head_size, int64_t head_stride, int kv_fp8, int dtype,
                                 int *partition_size, int *max_num_partitions, size_t *workspace_bytes);

/*
 * pc_stream_read -- measurement aid: read `bytes` of device memory once.
 *
 * Not a step of the path.  The decode is bound by one read of every K/V byte from HBM
 * ("vLLM 源码完全拆解（七）", section 性能模型), and this plain streaming read -- each
 * workgroup a contiguous chunk, 16-byte loads, eight in flight per lane -- measures how
 * fast one GPU can do that, so a decode's rate can be quoted against it beside the
 * rated peak.  The words read are folded with XOR into sink[w] (w < num_workgroups)
 * so the loads are not dead; sink's contents mean nothing.
 *
 *   src             device, 16-byte aligned; bytes a positive multiple of 16
 *   sink            device uint32 [num_workgroups]
 *   cache_policy    0 (default) or 2 (non-temporal hint, as the decode's V loads)
 * A chunk of more than 2^31 - 32768 bytes per workgroup gives PC_ERR_UNSUPPORTED.
 * Returns PC_OK, PC_ERR_INVALID_ARG, PC_ERR_UNSUPPORTED or PC_ERR_LAUNCH.
 */
int pc_stream_read(const void *src, int64_t bytes, uint32_t *sink, int num_workgroups, int cache_policy,
                   void *stream);

/*
 * pc_gather_read -- measurement aid: read the K and V tiles a decode of this batch reads,
 * and nothing else.
 *
 * Not a step of the path.  The decode's HBM stream ("vLLM 源码完全拆解（七）", section
 * 性能模型) is not one contiguous read but a gather through the block table ("How vLLM
 * CUDA Kernels Write and Read the Paged KV Cache", section "Reading logical blocks
 * during attention"): for every sequence s, kv head h and block j < ceil(seq_lens[s] /
 * 16), the 16 token rows of head h in block block_tables[s, j], from the K pool and from
 * the V pool.  This call loads exactly those tiles (16-byte loads, workgroups dealt as
 * the split decode deals its partitions) and folds the words with XOR, so a decode's
 * rate can be set against a plain gather of its own bytes.  With sink zeroed first,
 * the XOR of sink's 4096 entries afterwards is the XOR of every 32-bit word read.
 *
 *   k_pool, v_pool, num_blocks, block_stride, token_stride, head_stride, block_tables,
 *   max_blocks_per_seq, seq_lens, num_seqs, max_seq_len, num_kv_heads, head_size:
 *                   as for pc_paged_attention_decode (16-token blocks; element strides)
 *   element_bytes   1, 2 or 4 (the pool's element size); head_size * element_bytes must
 *                   be 128, 256 or 512
 *   sink            device uint32 [4096]
 *   v_cache_policy  0 (default) or 2 (non-temporal hint on the V loads, as the decode's)
 * A sequence whose length exceeds its table row or max_seq_len, and a block id outside
 * [0, num_blocks), read nothing.  Returns PC_OK, PC_ERR_INVALID_ARG, PC_ERR_UNSUPPORTED
 * or PC_ERR_LAUNCH.
 */
int pc_gather_read(const void *k_pool, const void *v_pool, int64_t num_blocks, int64_t block_stride,
                   int64_t token_stride, int64_t head_stride, const int32_t *block_tables, int max_blocks_per_seq,
                   const int32_t *seq_lens, int num_seqs, int max_seq_len, int num_kv_heads, int head_size,
                   int element_bytes, uint32_t *sink, int v_cache_policy, void *stream);

/* Bytes of the device buffer behind pc_paged_attention_split_noalloc, per GPU. */
#define PC_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * pc_paged_attention_split_noalloc -- the split decode and its reduce in one call
 * that allocates nothing, for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops or harnesses that forbid hipMalloc).
 *
 * Computes what pc_paged_attention_decode with partition_size = PC_PARTITION_SIZE
 * followed by pc_paged_attention_reduce computes -- the same kernels, so the same
 * bits in out -- but keeps exp_sums, max_logits and tmp_out in a device buffer of
 * PC_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on (from the
 * first call on that GPU until the process ends).  Arguments as for
 * pc_paged_attention_decode, without the partition size and the partials; out is
 * [num_seqs, num_q_heads, head_size] in the storage dtype.
 *
 * Limit: with P = ceil(max_seq_len / PC_PARTITION_SIZE) and R = num_seqs *
 * num_q_heads * P, the partials take 4 * (R * head_size + 2 * R) bytes (each piece
 * rounded up to 256); more than PC_NOALLOC_SCRATCH_BYTES gives PC_ERR_TOO_LARGE
 * before anything is enqueued (use pc_paged_attention_decode with a workspace then).
 * The call makes no hipMalloc, hipFree or other allocating call; on its first call on
 * a GPU it looks up the buffer's device address (hipGetSymbolAddress).
 * Concurrency: every call on one GPU uses that GPU's one buffer, which keeps the last
 * call's contents.  Calls on one GPU whose executions overlap (different streams, or
 * other threads' streams) race on it; calls in one stream are ordered.
 * Returns PC_OK, PC_ERR_INVALID_ARG, PC_ERR_UNSUPPORTED, PC_ERR_TOO_LARGE or
 * PC_ERR_LAUNCH.
 */
int pc_paged_attention_split_noalloc(void *out, const void *q, const void *k_pool, const void *v_pool,
                                     int64_t num_blocks, int64_t block_stride, int64_t token_stride,
                                     int64_t head_stride, const int32_t *block_tables, int max_blocks_per_seq,
                                     const int32_t *seq_lens, int num_seqs, int max_seq_len, int num_q_heads,
                                     int num_kv_heads, int head_size, int block_size, float scale,
                                     const float *alibi_slopes, int dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PC_H */
