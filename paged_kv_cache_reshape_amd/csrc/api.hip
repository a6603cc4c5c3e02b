// api.hip -- the C entry points declared in include/pc.h: argument validation on
// the host (nothing is enqueued when a check fails), then one or two launches on
// the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <numeric>
#include <vector>

#include "launch.h"
#include "pc.h"

namespace {

constexpr int kAbiVersion = 10;
constexpr int kBlockTokens = 16;

int esize(int dtype) { return dtype == PC_F32 ? 4 : (dtype == PC_F16 || dtype == PC_BF16) ? 2 : 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool strides16(int es, std::initializer_list<int64_t> strides) {
  for (int64_t s : strides)
    if ((s * es) % 16 != 0) return false;
  return true;
}

int status_of(hipError_t e) { return e == hipSuccess ? PC_OK : PC_ERR_LAUNCH; }

// Checks shared by both writes; es = element size of key / value.
int check_write(const void* key, const void* value, int64_t key_row_stride, int64_t value_row_stride,
                const void* k_pool, const void* v_pool, int64_t num_blocks, int64_t block_stride,
                int64_t token_stride, int64_t head_stride, const int64_t* slot_mapping, int64_t num_tokens,
                int num_kv_heads, int head_size, int block_size, int es) {
  if (!es || num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 || num_blocks <= 0 ||
      block_stride <= 0 || token_stride <= 0 || head_stride <= 0 || key_row_stride < 0 || value_row_stride < 0)
    return PC_ERR_INVALID_ARG;
  if (num_tokens == 0) return PC_OK;
  if (!key || !value || !k_pool || !v_pool || !slot_mapping) return PC_ERR_INVALID_ARG;
  if ((int64_t)num_kv_heads * head_size > key_row_stride && num_tokens > 1) return PC_ERR_INVALID_ARG;
  if ((int64_t)num_kv_heads * head_size > value_row_stride && num_tokens > 1) return PC_ERR_INVALID_ARG;
  if (num_tokens > INT_MAX || num_blocks > INT64_MAX / block_size) return PC_ERR_UNSUPPORTED;
  return PC_OK;
}

// Both decodes; kv8 = the pool holds E4M3 codes (1 byte per element) with per-head
// scales, else the pool has q's storage type.
int decode_impl(void* out, const void* q, const void* k_pool, const void* v_pool, int64_t num_blocks,
                int64_t block_stride, int64_t token_stride, int64_t head_stride, const int32_t* block_tables,
                int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs, int max_seq_len, int num_q_heads,
                int num_kv_heads, int head_size, int block_size, float scale, int partition_size, float* exp_sums,
                float* max_logits, float* tmp_out, const float* alibi_slopes, const float* k_scale,
                const float* v_scale, int64_t kv_scale_stride, int dtype, bool kv8, void* stream,
                const int64_t* step_slots = nullptr, const void* step_key = nullptr,
                const void* step_value = nullptr, int64_t step_key_stride = 0, int64_t step_value_stride = 0,
                const int32_t* prefix_table = nullptr, int prefix_blocks = 0, const int32_t* shared_lens = nullptr) {
  const int es = esize(dtype);
  if (!es || num_seqs < 0 || max_seq_len < 0 || max_blocks_per_seq < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_size <= 0 || block_size <= 0 || num_q_heads % num_kv_heads != 0 || (kv8 && kv_scale_stride < 0))
    return PC_ERR_INVALID_ARG;
  const bool split = partition_size != 0;
  if (split && partition_size != PC_PARTITION_SIZE) return partition_size < 0 ? PC_ERR_INVALID_ARG : PC_ERR_UNSUPPORTED;
  if (split) {
    if (!exp_sums || !max_logits || !tmp_out) return PC_ERR_INVALID_ARG;
  } else if (exp_sums || max_logits || tmp_out) {
    return PC_ERR_INVALID_ARG;
  }
  if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * block_size) return PC_ERR_INVALID_ARG;
  if (num_seqs == 0) return PC_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || (!split && !out)) return PC_ERR_INVALID_ARG;
  if (kv8 && (!k_scale || !v_scale)) return PC_ERR_INVALID_ARG;
  if (num_blocks <= 0 || block_stride <= 0 || token_stride <= 0 || head_stride <= 0) return PC_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !std::isfinite(scale)) return PC_ERR_INVALID_ARG;
  // 16-bit and 8-bit pools: blocks of 8, 16 or 32 tokens; fp32 storage: 16
  if (block_size != 8 && block_size != 16 && block_size != 32) return PC_ERR_UNSUPPORTED;
  if (dtype == PC_F32 && block_size != kBlockTokens) return PC_ERR_UNSUPPORTED;
  if (kv8 && dtype == PC_F32) return PC_ERR_UNSUPPORTED;
  if (!pcache::decode_supported(dtype, head_size, num_q_heads / num_kv_heads)) return PC_ERR_UNSUPPORTED;
  const int pes = kv8 ? 1 : es;  // pool bytes per element
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !strides16(pes, {block_stride, token_stride, head_stride, (int64_t)head_size}))
    return PC_ERR_UNSUPPORTED;
  // a block's 16 token rows of one head are addressed with 32-bit byte offsets
  if (token_stride > INT_MAX / (kBlockTokens * pes)) return PC_ERR_UNSUPPORTED;
  const int parts = split ? (max_seq_len + PC_PARTITION_SIZE - 1) / PC_PARTITION_SIZE : 1;
  if ((int64_t)num_seqs * num_kv_heads * parts > INT_MAX) return PC_ERR_UNSUPPORTED;
  if (split && parts == 0) return PC_OK;  // every sequence is empty: no partials exist
  // a common prefix (split path): fp16 / bf16 pools of 16-token blocks
  if (shared_lens && (dtype == PC_F32 || kv8 || block_size != kBlockTokens)) return PC_ERR_UNSUPPORTED;
  pcache::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.num_blocks = num_blocks;
  a.block_stride = block_stride;
  a.token_stride = token_stride;
  a.head_stride = head_stride;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.seq_lens = seq_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.max_partitions = parts;
  a.max_seq_len = max_seq_len;
  a.exp_sums = exp_sums;
  a.max_logits = max_logits;
  a.tmp_out = tmp_out;
  a.kv8 = kv8;
  a.alibi_slopes = alibi_slopes;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.scale_stride = kv_scale_stride;
  a.step_slots = step_slots;
  a.step_key = step_key;
  a.step_value = step_value;
  a.step_key_stride = step_key_stride;
  a.step_value_stride = step_value_stride;
  a.prefix_table = prefix_table;
  a.prefix_blocks = prefix_blocks;
  a.shared_lens = shared_lens;
  // Head size 64 with a token's kv heads next to each other (NHD, or K then V per block):
  // one kv head's token rows are 128-byte pieces a whole token row apart.  Kv heads 2p
  // and 2p+1 are then read together as 256-byte pieces and computed as one head of 128
  // with twice the query heads (16-bit pools, at most 8 query columns).
  const int group = num_q_heads / num_kv_heads;
  const bool pair = !kv8 && dtype != PC_F32 && head_size == 64 && head_stride == head_size && num_kv_heads % 2 == 0 &&
                    group <= 4 && step_slots == nullptr && shared_lens == nullptr &&
                    pcache::decode_supported(dtype, 128, 2 * group);
  if (pair) {
    a.pair = 1;
    a.num_kv_heads = num_kv_heads / 2;
    a.head_stride = 2 * head_stride;
  }
  hipError_t e = pcache::launch_decode(a, dtype, pair ? 2 * head_size : head_size, split,
                                       static_cast<hipStream_t>(stream));
  if (e == hipSuccess && shared_lens) e = pcache::launch_decode_prefix(a, dtype, head_size, static_cast<hipStream_t>(stream));
  return status_of(e);
}

}  // namespace

namespace pcache {

// Compute units of the current device, cached per device; MI355X's 256 when no
// device can be queried (the planner is usable without a GPU).
int device_compute_units() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cached[dev] = n;
  }
  return cached[dev];
}

// The one-pass path has two kernels.  The persistent one (one workgroup of 12 waves per
// CU, units dealt longest first) keeps long units streaming but pays each unit's start
// and merge in series; the grid one (a 4-wave workgroup per unit, three per CU, dealt by
// the hardware) overlaps those costs across workgroups but leaves the longest units to
// whichever workgroup draws them.  Of the rules of this form tried against measurements
// of both kernels and the split path on MI355X (194 batch shapes: 1/8 to 32 units per
// CU, longest sequences of 512 to 32768 tokens, fixed, uniform and log-uniform mixes),
// this one left the planner's choice within 5% of the fastest of the three on the most
// shapes: the grid kernel when the longest sequence fits one 512-token partition, or for
// at least 32 units per CU with sequences up to 2048 tokens.
bool onepass_grid(int64_t units, int max_seq_len, int compute_units) {
  return max_seq_len <= 512 || (units >= 32LL * compute_units && max_seq_len <= 2048);
}

namespace {

// Estimated launch time (us) of each decode path for a batch, from a model fitted to
// measurements of the three kernels on MI355X: 218 batch shapes (24 of them with a
// shared 1024-token prefix), GQA 32/8 and MHA 32/32, head size 128, bf16, 16-token
// blocks; the split path's constants apart for MHA (its 2-wave workgroups) and GQA.
//   * persistent one pass: each workgroup's units under the kernel's own deal (turn 0
//     in index order, then sequences ranked longest first and dealt in snake order),
//     each unit costing its bytes plus a fixed equivalent; the workgroups stream
//     concurrently, each at 1 / (1/R0 + n/B) with n of them still busy (a shared memory
//     system: a lone CU streams near R0, a full chip near B in total);
//   * grid one pass and split: one workgroup per unit (per 512-token partition), three
//     per CU; the larger of the whole batch at a chip rate, the workgroup slots' total
//     occupancy, and the longest unit alone at a per-workgroup rate that falls with the
//     number of busy workgroups; the split path adds its reduce.
// Tokens in blocks that several sequences of the batch read (a shared prefix) come
// partly from cache: each counts as a fraction of a token read from HBM, fitted per
// kernel on batches with a shared 1024-token prefix (24 more measured shapes, each
// kernel's on the shapes it runs): 0.60 persistent, 0.54 grid.  Given the sharing, the
// split path runs pc_paged_attention_decode_prefix; its model is in
// est_per_unit_workgroups.
struct Batch {
  const int32_t* lens;
  const int32_t* shared;     // per sequence: leading tokens in blocks other sequences also read (or NULL)
  int S, Hq, units_per_seq;  // units_per_seq: kv heads (or kv head pairs)
  double tok_bytes;          // K and V bytes per token of one unit
  int cus, wgs_per_cu;       // persistent workgroups: cus * wgs_per_cu
};

double unit_bytes(const Batch& b, int s, int t0, int t1, double lam) {  // tokens [t0, t1) of sequence s
  const int sh = b.shared ? std::max(0, std::min(b.shared[s], t1) - t0) : 0;
  return ((t1 - t0) - sh + lam * sh) * b.tok_bytes;
}

double est_persistent(const Batch& b) {
  constexpr double R0 = 54.75e3, Bw = 12557e3, o1 = 69.2e3, c1 = 3.39;  // bytes/us, bytes, us
  const int H = b.units_per_seq, S = b.S;
  const int64_t U = (int64_t)S * H, W = (int64_t)b.cus * b.wgs_per_cu;
  std::vector<double> load((size_t)W, 0.0);
  std::vector<int> cnt((size_t)W, 0);
  constexpr double lam = 0.60;
  for (int64_t k = 0; k < std::min(U, W); ++k) {
    load[k] += unit_bytes(b, (int)(k / H), 0, b.lens[k / H], lam);
    ++cnt[k];
  }
  if (U > W) {
    const bool ranked = S <= 512 && W % H == 0;  // as the kernel decides (longest first on)
    const int S0 = (int)(W / H);
    std::vector<int> order, rank0;
    if (ranked) {
      auto longer = [&](int x, int y) { return b.lens[x] > b.lens[y] || (b.lens[x] == b.lens[y] && x < y); };
      order.resize(S - S0);
      std::iota(order.begin(), order.end(), S0);
      std::sort(order.begin(), order.end(), longer);
      std::vector<int> first(S0);
      std::iota(first.begin(), first.end(), 0);
      std::sort(first.begin(), first.end(), longer);
      rank0.resize(S0);
      for (int i = 0; i < S0; ++i) rank0[first[i]] = i;
    }
    const int64_t rest = U - W;
    for (int64_t k = 0; k < W; ++k) {
      const int64_t r0 = ranked ? (int64_t)rank0[k / H] * H + k % H : k;
      for (int64_t t = 1; (t - 1) * W < rest; ++t) {
        const int64_t q = (t - 1) * W + ((t & 1) ? W - 1 - r0 : r0);
        if (q >= rest) continue;
        const int s = ranked ? order[q / H] : (int)((W + q) / H);
        load[k] += unit_bytes(b, s, 0, b.lens[s], lam);
        ++cnt[k];
      }
    }
  }
  for (int64_t k = 0; k < W; ++k) load[k] += cnt[k] * o1;
  std::sort(load.begin(), load.end());
  double t = 0.0, prev = 0.0;
  int64_t busy = 0;
  for (double x : load) busy += x > 0.0;
  for (double x : load) {
    if (x <= 0.0) continue;
    t += (x - prev) * (1.0 / R0 + busy / Bw);
    prev = x;
    --busy;
  }
  return t + c1;
}

// grid one pass (split = false) or split (split = true).  On the split path a batch with
// shared prefix tokens is taken to run pc_paged_attention_decode_prefix: the partitions
// its shared tokens cover completely leave the split kernel for the prefix kernel.
double est_per_unit_workgroups(const Batch& b, bool split) {
  const bool mha = b.Hq == b.units_per_seq;  // one query head per kv head: 2-wave split workgroups
  struct K { double BW, R, t0, c, R1, B1, rr; };
  constexpr K kGrid{5792e3, 764.2e3, 0.0, 4.10, 50.98e3, 43898e3, 0.0};
  constexpr K kSplitMha{6233e3, 5734e3, 4.87, 9.75, 117.3e3, 1e13, 0.557e-3};
  constexpr K kSplitGqa{6235e3, 5883e3, 3.25, 11.16, 100.1e3, 1e13, 0.416e-3};
  const K& k = !split ? kGrid : mha ? kSplitMha : kSplitGqa;
  const bool pfx = split && b.shared != nullptr;
  // shared tokens: in a partition they cover completely, the prefix kernel's (pfx);
  // elsewhere a fraction of an HBM token
  const double lam = !split ? 0.54 : !pfx ? 0.46 : mha ? 0.55 : 1.0;
  double total = 0.0, bmax = 0.0;
  int64_t n = 0;
  int lmax = 0, shmax = 0;
  for (int s = 0; s < b.S; ++s) {
    const int L = std::max(b.lens[s], 0);
    const int sh = b.shared ? b.shared[s] : 0;
    const int step = split ? PC_PARTITION_SIZE : std::max(L, 1);
    for (int t0 = 0; t0 < L; t0 += step) {  // the sequence's units (its partitions on the split path)
      if (pfx && sh >= t0 + PC_PARTITION_SIZE) continue;
      const double x = unit_bytes(b, s, t0, std::min(L, t0 + step), lam);
      total += x * b.units_per_seq;
      bmax = std::max(bmax, x);
      n += b.units_per_seq;
    }
    if (!split && L == 0) n += b.units_per_seq;
    lmax = std::max(lmax, L);
    shmax = std::max(shmax, sh);
  }
  const double slots = (split && mha ? 6.0 : 3.0) * b.cus;
  const double r1 = 1.0 / (1.0 / k.R1 + std::min((double)n, slots) / k.B1);
  double t = std::max({total / k.BW, (n * k.t0 + total / k.R) / slots, bmax / r1 + k.t0}) + k.c;
  const int parts = (lmax + PC_PARTITION_SIZE - 1) / PC_PARTITION_SIZE;
  if (split) t += k.rr * b.S * b.Hq * parts;
  if (pfx) {  // the prefix kernel: one workgroup per (kv head, 16 / G sequences, covered partition)
    const int G = b.Hq / b.units_per_seq;
    const int64_t units = (int64_t)b.units_per_seq * ((b.S + 16 / G - 1) / (16 / G)) *
                          std::min(shmax / PC_PARTITION_SIZE, parts);
    if (units > 0) t += (mha ? 0.0 : 0.287) * units * PC_PARTITION_SIZE * b.tok_bytes / k.BW + (mha ? 15.2 : 3.91);
  }
  return t;
}

// 1: split, 0: one pass
int plan_choice(const int32_t* lens, const int32_t* shared, int S, int Hq, int Hkv, int D, bool paired, bool kv8,
                int dtype) {
  int lmax = 0;
  for (int s = 0; s < S; ++s) lmax = std::max(lmax, lens[s]);
  if (lmax <= PC_PARTITION_SIZE) return 0;  // one partition: the split path only adds its reduce
  const int cus = device_compute_units();
  Batch b{};
  b.lens = lens;
  b.shared = shared;
  b.S = S;
  b.Hq = Hq;
  b.units_per_seq = paired ? Hkv / 2 : Hkv;
  const int Deff = paired ? 2 * D : D;
  b.tok_bytes = 2.0 * Deff * (kv8 ? 1 : esize(dtype));
  b.cus = cus;
  b.wgs_per_cu = (Deff == 64 && !kv8) ? 2 : 1;  // the persistent kernel's workgroups per CU
  const int64_t units = (int64_t)S * b.units_per_seq;
  const bool grid = dtype == PC_F32 || (!kv8 && onepass_grid(units, lmax, cus));
  const double one = grid ? est_per_unit_workgroups(b, false) : est_persistent(b);
  return est_per_unit_workgroups(b, true) < one ? 1 : 0;
}

}  // namespace
}  // namespace pcache

extern "C" {

int pc_abi_version(void) { return kAbiVersion; }

const char* pc_status_string(int status) {
  switch (status) {
    case PC_OK: return "ok";
    case PC_ERR_INVALID_ARG: return "invalid argument";
    case PC_ERR_UNSUPPORTED: return "unsupported configuration";
    case PC_ERR_LAUNCH: return "kernel launch failed";
    case PC_ERR_TOO_LARGE: return "request exceeds the library's fixed device buffer";
    default: return "unknown status";
  }
}

int pc_reshape_and_cache(const void* key, const void* value, int64_t key_row_stride, int64_t value_row_stride,
                         void* k_pool, void* v_pool, int64_t num_blocks, int64_t block_stride, int64_t token_stride,
                         int64_t head_stride, const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads,
                         int head_size, int block_size, int dtype, void* stream) {
  const int es = esize(dtype);
  const int rc = check_write(key, value, key_row_stride, value_row_stride, k_pool, v_pool, num_blocks, block_stride,
                             token_stride, head_stride, slot_mapping, num_tokens, num_kv_heads, head_size, block_size,
                             es);
  if (rc != PC_OK || num_tokens == 0) return rc;
  const bool vec16 = aligned16(key) && aligned16(value) && aligned16(k_pool) && aligned16(v_pool) &&
                     strides16(es, {key_row_stride, value_row_stride, block_stride, token_stride, head_stride,
                                    (int64_t)head_size});
  pcache::WriteArgs a{key,        value,        key_row_stride, value_row_stride, k_pool,     v_pool,
                      num_blocks, block_stride, token_stride,   head_stride,      slot_mapping, num_tokens,
                      num_kv_heads, head_size,  block_size,     nullptr,          nullptr,      0};
  return status_of(pcache::launch_write(a, dtype, vec16, static_cast<hipStream_t>(stream)));
}

int pc_reshape_and_cache_fp8(const void* key, const void* value, int64_t key_row_stride, int64_t value_row_stride,
                             uint8_t* k_pool, uint8_t* v_pool, int64_t num_blocks, int64_t block_stride,
                             int64_t token_stride, int64_t head_stride, const int64_t* slot_mapping,
                             int64_t num_tokens, int num_kv_heads, int head_size, int block_size,
                             const float* k_scale, const float* v_scale, int64_t kv_scale_stride, int dtype,
                             void* stream) {
  const int es = esize(dtype);
  const int rc = check_write(key, value, key_row_stride, value_row_stride, k_pool, v_pool, num_blocks, block_stride,
                             token_stride, head_stride, slot_mapping, num_tokens, num_kv_heads, head_size, block_size,
                             es);
  if (rc != PC_OK) return rc;
  if (kv_scale_stride < 0) return PC_ERR_INVALID_ARG;
  if (num_tokens == 0) return PC_OK;
  if (!k_scale || !v_scale) return PC_ERR_INVALID_ARG;
  // four codes per 32-bit store
  if (head_size % 4 != 0 || ((uintptr_t)k_pool | (uintptr_t)v_pool) % 4 != 0 ||
      (block_stride | token_stride | head_stride) % 4 != 0)
    return PC_ERR_UNSUPPORTED;
  pcache::WriteArgs a{key,        value,        key_row_stride, value_row_stride, k_pool,     v_pool,
                      num_blocks, block_stride, token_stride,   head_stride,      slot_mapping, num_tokens,
                      num_kv_heads, head_size,  block_size,     k_scale,          v_scale,      kv_scale_stride};
  return status_of(pcache::launch_write_fp8(a, dtype, static_cast<hipStream_t>(stream)));
}

int pc_paged_attention_decode(void* out, const void* q, const void* k_pool, const void* v_pool, int64_t num_blocks,
                              int64_t block_stride, int64_t token_stride, int64_t head_stride,
                              const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_lens,
                              int num_seqs, int max_seq_len, int num_q_heads, int num_kv_heads, int head_size,
                              int block_size, float scale, int partition_size, float* exp_sums, float* max_logits,
                              float* tmp_out, const float* alibi_slopes, int dtype, void* stream) {
  return decode_impl(out, q, k_pool, v_pool, num_blocks, block_stride, token_stride, head_stride, block_tables,
                     max_blocks_per_seq, seq_lens, num_seqs, max_seq_len, num_q_heads, num_kv_heads, head_size,
                     block_size, scale, partition_size, exp_sums, max_logits, tmp_out, alibi_slopes, nullptr,
                     nullptr, 0, dtype, false, stream);
}

int pc_paged_attention_decode_prefix(const void* q, const void* k_pool, const void* v_pool, int64_t num_blocks,
                                     int64_t block_stride, int64_t token_stride, int64_t head_stride,
                                     const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_lens,
                                     int num_seqs, int max_seq_len, int num_q_heads, int num_kv_heads, int head_size,
                                     int block_size, float scale, float* exp_sums, float* max_logits, float* tmp_out,
                                     const float* alibi_slopes, const int32_t* prefix_table, int prefix_blocks,
                                     const int32_t* shared_lens, int dtype, void* stream) {
  if (prefix_blocks < 0 || (prefix_blocks > 0 && (!prefix_table || !shared_lens))) return PC_ERR_INVALID_ARG;
  const bool pfx = prefix_blocks > 0;
  return decode_impl(nullptr, q, k_pool, v_pool, num_blocks, block_stride, token_stride, head_stride, block_tables,
                     max_blocks_per_seq, seq_lens, num_seqs, max_seq_len, num_q_heads, num_kv_heads, head_size,
                     block_size, scale, PC_PARTITION_SIZE, exp_sums, max_logits, tmp_out, alibi_slopes, nullptr,
                     nullptr, 0, dtype, false, stream, nullptr, nullptr, nullptr, 0, 0, pfx ? prefix_table : nullptr,
                     pfx ? prefix_blocks : 0, pfx ? shared_lens : nullptr);
}

int pc_paged_attention_decode_fp8(void* out, const void* q, const uint8_t* k_pool, const uint8_t* v_pool,
                                  int64_t num_blocks, int64_t block_stride, int64_t token_stride, int64_t head_stride,
                                  const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_lens,
                                  int num_seqs, int max_seq_len, int num_q_heads, int num_kv_heads, int head_size,
                                  int block_size, float scale, int partition_size, float* exp_sums,
                                  float* max_logits, float* tmp_out, const float* alibi_slopes,
                                  const float* k_scale, const float* v_scale, int64_t kv_scale_stride, int dtype,
                                  void* stream) {
  return decode_impl(out, q, k_pool, v_pool, num_blocks, block_stride, token_stride, head_stride, block_tables,
                     max_blocks_per_seq, seq_lens, num_seqs, max_seq_len, num_q_heads, num_kv_heads, head_size,
                     block_size, scale, partition_size, exp_sums, max_logits, tmp_out, alibi_slopes, k_scale,
                     v_scale, kv_scale_stride, dtype, true, stream);
}

int pc_reshape_and_cache_decode(void* out, const void* q, const void* key, const void* value, int64_t key_row_stride,
                                int64_t value_row_stride, const int64_t* slot_mapping, void* k_pool, void* v_pool,
                                int64_t num_blocks, int64_t block_stride, int64_t token_stride, int64_t head_stride,
                                const int32_t* block_tables, int max_blocks_per_seq, const int32_t* seq_lens,
                                int num_seqs, int max_seq_len, int num_q_heads, int num_kv_heads, int head_size,
                                int block_size, float scale, int partition_size, float* exp_sums, float* max_logits,
                                float* tmp_out, const float* alibi_slopes, int dtype, void* stream) {
  const int es = esize(dtype);
  if (num_seqs < 0) return PC_ERR_INVALID_ARG;
  const int wrc = check_write(key, value, key_row_stride, value_row_stride, k_pool, v_pool, num_blocks, block_stride,
                              token_stride, head_stride, slot_mapping, num_seqs, num_kv_heads, head_size,
                              block_size, es);
  if (wrc != PC_OK) return wrc;
  if (dtype == PC_F32) return PC_ERR_UNSUPPORTED;  // the fused write lives in the matrix-core decode
  // 8-token blocks, 8 query heads per kv head, head size 128: the fused one-pass kernel
  // would not keep its state in registers, so the library has no fused kernel for it
  if (block_size == 8 && num_kv_heads > 0 && num_q_heads == 8 * num_kv_heads && head_size == 128)
    return PC_ERR_UNSUPPORTED;
  // the row is moved in 16-byte pieces
  if (num_seqs > 0 && (!aligned16(key) || !aligned16(value) || !strides16(es, {key_row_stride, value_row_stride})))
    return PC_ERR_UNSUPPORTED;
  return decode_impl(out, q, k_pool, v_pool, num_blocks, block_stride, token_stride, head_stride, block_tables,
                     max_blocks_per_seq, seq_lens, num_seqs, max_seq_len, num_q_heads, num_kv_heads, head_size,
                     block_size, scale, partition_size, exp_sums, max_logits, tmp_out, alibi_slopes, nullptr,
                     nullptr, 0, dtype, false, stream, slot_mapping, key, value, key_row_stride, value_row_stride);
}

int pc_paged_attention_varlen(void* out, const void* q, const void* k_pool, const void* v_pool, int64_t num_blocks,
                              int64_t block_stride, int64_t token_stride, int64_t head_stride,
                              const int32_t* block_tables, int max_blocks_per_seq, const int32_t* query_start_loc,
                              const int32_t* seq_lens, int num_reqs, int64_t total_q, int max_query_len,
                              int num_q_heads, int num_kv_heads, int head_size, int block_size, float scale,
                              int causal, const float* alibi_slopes, int dtype, void* stream) {
  const int es = esize(dtype);
  if (!es || num_reqs < 0 || total_q < 0 || max_query_len < 0 || max_blocks_per_seq < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 || num_q_heads % num_kv_heads != 0 ||
      (causal != 0 && causal != 1))
    return PC_ERR_INVALID_ARG;
  if (num_reqs == 0 || total_q == 0) return PC_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !query_start_loc || !seq_lens) return PC_ERR_INVALID_ARG;
  if (num_blocks <= 0 || block_stride <= 0 || token_stride <= 0 || head_stride <= 0) return PC_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !std::isfinite(scale)) return PC_ERR_INVALID_ARG;
  if (block_size != kBlockTokens || dtype == PC_F32) return PC_ERR_UNSUPPORTED;
  const int group = num_q_heads / num_kv_heads;
  if ((head_size != 64 && head_size != 128) || (group != 1 && group != 2 && group != 4 && group != 8))
    return PC_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !strides16(es, {block_stride, token_stride, head_stride, (int64_t)head_size}))
    return PC_ERR_UNSUPPORTED;
  if (token_stride > INT_MAX / (kBlockTokens * es)) return PC_ERR_UNSUPPORTED;
  if (total_q > INT_MAX) return PC_ERR_UNSUPPORTED;
  pcache::VarlenArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.num_blocks = num_blocks;
  a.block_stride = block_stride;
  a.token_stride = token_stride;
  a.head_stride = head_stride;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.query_start_loc = query_start_loc;
  a.seq_lens = seq_lens;
  a.num_reqs = num_reqs;
  a.total_q = total_q;
  a.max_query_len = max_query_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.causal = causal;
  a.alibi_slopes = alibi_slopes;
  return status_of(pcache::launch_varlen(a, dtype, head_size, static_cast<hipStream_t>(stream)));
}

int pc_paged_attention_reduce(void* out, const float* exp_sums, const float* max_logits, const float* tmp_out,
                              const int32_t* seq_lens, int num_seqs, int num_q_heads, int head_size,
                              int max_num_partitions, int partition_size, int dtype, void* stream) {
  if (!esize(dtype) || num_seqs < 0 || num_q_heads <= 0 || head_size <= 0 || max_num_partitions < 0 ||
      partition_size <= 0)
    return PC_ERR_INVALID_ARG;
  if (partition_size != PC_PARTITION_SIZE || !pcache::reduce_supported(head_size)) return PC_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PC_OK;
  if (!out || !seq_lens || (max_num_partitions > 0 && (!exp_sums || !max_logits || !tmp_out)))
    return PC_ERR_INVALID_ARG;
  if (!aligned16(tmp_out)) return PC_ERR_UNSUPPORTED;
  if ((int64_t)num_seqs * num_q_heads > INT_MAX) return PC_ERR_UNSUPPORTED;
  pcache::ReduceArgs a{out, exp_sums, max_logits, tmp_out, seq_lens, num_seqs, num_q_heads, head_size,
                       max_num_partitions, partition_size};
  return status_of(pcache::launch_reduce(a, dtype, static_cast<hipStream_t>(stream)));
}

namespace {
int plan_common(const int32_t* lens, const int32_t* shared, int num_seqs, int num_q_heads, int num_kv_heads,
                int head_size, int max_seq_len, bool paired, bool kv8, int dtype, int* partition_size,
                int* max_num_partitions, size_t* workspace_bytes) {
  const int parts = (max_seq_len + PC_PARTITION_SIZE - 1) / PC_PARTITION_SIZE;
  const bool split = num_seqs > 0 && parts > 1 &&
                     pcache::plan_choice(lens, shared, num_seqs, num_q_heads, num_kv_heads, head_size, paired, kv8,
                                         dtype);
  const int mp = split ? parts : 1;
  if (partition_size) *partition_size = split ? PC_PARTITION_SIZE : 0;
  if (max_num_partitions) *max_num_partitions = mp;
  if (workspace_bytes)
    *workspace_bytes = split ? (size_t)num_seqs * num_q_heads * mp * ((size_t)head_size + 2) * sizeof(float) : 0;
  return PC_OK;
}
}  // namespace

int pc_paged_attention_plan(int num_seqs, int num_q_heads, int num_kv_heads, int head_size, int max_seq_len,
                            int dtype, int* partition_size, int* max_num_partitions, size_t* workspace_bytes) {
  if (!esize(dtype) || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 || max_seq_len < 0 ||
      num_q_heads % num_kv_heads != 0)
    return PC_ERR_INVALID_ARG;
  // lengths unknown: every sequence is taken to be max_seq_len long
  std::vector<int32_t> lens((size_t)num_seqs, max_seq_len);
  return plan_common(lens.data(), nullptr, num_seqs, num_q_heads, num_kv_heads, head_size, max_seq_len, false, false,
                     dtype, partition_size, max_num_partitions, workspace_bytes);
}

int pc_paged_attention_plan_lens(const int32_t* seq_lens, const int32_t* shared_lens, int num_seqs, int num_q_heads,
                                 int num_kv_heads, int head_size, int64_t head_stride, int kv_fp8, int dtype,
                                 int* partition_size, int* max_num_partitions, size_t* workspace_bytes) {
  if (!esize(dtype) || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
      num_q_heads % num_kv_heads != 0 || (kv_fp8 != 0 && kv_fp8 != 1) || (num_seqs > 0 && !seq_lens))
    return PC_ERR_INVALID_ARG;
  int max_seq_len = 0;
  for (int s = 0; s < num_seqs; ++s) {
    if (seq_lens[s] < 0 || (shared_lens && (shared_lens[s] < 0 || shared_lens[s] > seq_lens[s])))
      return PC_ERR_INVALID_ARG;
    max_seq_len = std::max(max_seq_len, seq_lens[s]);
  }
  // the decode's own pairing rule (16-bit pools, head size 64, heads side by side)
  const int group = num_q_heads / num_kv_heads;
  const bool paired = !kv_fp8 && dtype != PC_F32 && head_size == 64 && head_stride == head_size &&
                      num_kv_heads % 2 == 0 && group <= 4;
  return plan_common(seq_lens, shared_lens, num_seqs, num_q_heads, num_kv_heads, head_size, max_seq_len, paired,
                     kv_fp8 != 0, dtype, partition_size, max_num_partitions, workspace_bytes);
}

}  // extern "C"
