// decode.hip -- paged decode attention: one query token per (sequence, head)
// against the sequence's paged K/V, in one pass or per 512-token partition.  This
// VALU kernel serves fp32 storage; fp16 / bf16 storage runs decode_mfma.hip.
//
// What is computed ("vLLM 源码完全拆解（七）: PagedAttention Kernel", sections
// 先明确问题, 线程组织, 第一步 and V1与V2; "Inside vLLM CUDA Kernels", Part 3,
// "How Each K/V Tile Contributes to the Output"): for query head h of sequence s,
// kv head h / G, scores x_t = scale * q.k_t over the visible positions, an online
// softmax (running max m, sum l, accumulator acc rescaled by exp(m_old - m_new))
// and out = acc / l.  The split form stops at each 512-token partition and stores
// (acc / l, m, l) for the reduce kernel.
//
// MI355X mapping (prior art in the pages is a 32-lane-warp design; this is not it):
// * Work unit = (sequence, kv head[, partition]) -- one workgroup computes all G
//   query heads of a GQA group from a single read of each K/V tile, so every K/V
//   byte leaves HBM once.
// * Four waves per workgroup take the unit's 16-token blocks round-robin, each
//   keeping its own softmax state; the states meet once, in LDS, at the end.
// * Inside a wave a 16-token block is read with 16-byte loads: a token row
//   (head_size elements) is spread over LPR lanes, TPI = 64 / LPR rows per load, so
//   every load instruction moves 1 KiB of whole rows.  Each lane dot-products its
//   16-byte slice against the matching slice of each query head (v_dot2 for 16-bit
//   types) and the LPR-lane partial sums are folded with DPP row permutes.
// * Lanes holding the same token subset (rows r, r + TPI, ...) keep identical
//   softmax state, so the P.V update needs no cross-lane traffic: each lane scales
//   its 16-byte slice of V by the probabilities it already holds.
// * The next block's K/V loads are issued before the current block is consumed.
// * Scores live in the base-2 domain (scale folded with log2 e) so exp is a single
//   v_exp_f32; the split path stores max_logits back in the natural-log domain.
#include <cmath>

#include "device_common.h"
#include "launch.h"

namespace pcache {
namespace {

constexpr int kBlockTokens = 16;
constexpr int kPartition = 512;
constexpr int kWaves = 4;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <class ST, int D, int G, bool SPLIT>
__global__ __launch_bounds__(kWaves* kWave) void decode_kernel(DecodeArgs a) {
  constexpr int EB = ST::kBytes;
  constexpr int EPL = 16 / EB;                  // elements per 16-byte slice
  constexpr int LPR = D / EPL;                  // lanes per token row
  constexpr int TPI = kWave / LPR;              // token rows per wave-wide load
  constexpr int NI = kBlockTokens / TPI;        // wave-wide loads per block, for K and for V
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "unsupported row width");
  static_assert(NI * TPI == kBlockTokens, "block must split into whole loads");

  __shared__ float sm_acc[kWaves][TPI][G][D];
  __shared__ float sm_m[kWaves][TPI][G];
  __shared__ float sm_l[kWaves][TPI][G];
  __shared__ int sm_bad[kWaves];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int li = lane % LPR;  // 16-byte slice of the row
  const int lr = lane / LPR;  // row within a wave-wide load

  int64_t id = blockIdx.x;
  const int kvh = (int)(id % a.num_kv_heads);
  id /= a.num_kv_heads;
  const int s = (int)(id % a.num_seqs);
  const int part = SPLIT ? (int)(id / a.num_seqs) : 0;

  const int L = a.seq_lens[s];
  bool bad = L < 0 || (int64_t)L > (int64_t)a.max_blocks_per_seq * kBlockTokens ||
             (SPLIT && (int64_t)L > (int64_t)a.max_partitions * kPartition);
  const int t_begin = SPLIT ? part * kPartition : 0;
  if (SPLIT && !bad && t_begin >= L) return;  // a partition past the sequence writes nothing
  const int t_end = bad ? t_begin : (SPLIT ? min(L, t_begin + kPartition) : L);
  const int b_begin = t_begin / kBlockTokens;
  const int b_end = (t_end + kBlockTokens - 1) / kBlockTokens;

  const int h0 = kvh * G;
  uint4 qv[G];
  {
    const char* qb = static_cast<const char*>(a.q) + (((int64_t)s * a.num_q_heads + h0) * D + li * EPL) * EB;
#pragma unroll
    for (int g = 0; g < G; ++g) qv[g] = *reinterpret_cast<const uint4*>(qb + (int64_t)g * D * EB);
  }

  // ALiBi slopes of the group's query heads, in the base-2 score domain
  const bool alibi = a.alibi_slopes != nullptr;
  float ab[G];
#pragma unroll
  for (int g = 0; g < G; ++g) ab[g] = alibi ? a.alibi_slopes[h0 + g] * kLog2e : 0.f;

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int64_t head_off = (int64_t)kvh * a.head_stride * EB;
  const char* kbase = static_cast<const char*>(a.k_pool) + head_off;
  const char* vbase = static_cast<const char*>(a.v_pool) + head_off;
  const int64_t lane_off = ((int64_t)lr * a.token_stride + li * EPL) * EB;
  const int64_t load_step = (int64_t)TPI * a.token_stride * EB;
  const int64_t block_bytes = a.block_stride * EB;

  // This wave takes blocks b_begin + w, b_begin + w + kWaves, ...: nw of them.  Their
  // physical ids are fetched 64 at a time into one VGPR (lane k holds the k-th) and
  // read back with readlane, so no table load sits on the per-block path.
  const int first = b_begin + w;
  const int nw = first < b_end ? (b_end - first + kWaves - 1) / kWaves : 0;
  int tv = 0;
  auto fetch_table = [&](int chunk) {
    const int idx = chunk * kWave + lane;
    int v = 0;
    if (idx < nw) v = table[first + idx * kWaves];
    const bool out_of_pool = idx < nw && (v < 0 || (int64_t)v >= a.num_blocks);
    if (__builtin_amdgcn_ballot_w64(out_of_pool) != 0) bad = true;
    tv = v;
  };
  int n_iter = nw;
  if (n_iter > 0) {
    fetch_table(0);
    if (bad) n_iter = 0;  // a block id outside the pool: nothing is read, the outputs become NaN
  }

  uint4 kc[NI], vc[NI], kn[NI], vn[NI];
  if (n_iter > 0) {
    const int64_t boff = (int64_t)__builtin_amdgcn_readlane(tv, 0) * block_bytes + lane_off;
#pragma unroll
    for (int j = 0; j < NI; ++j) kc[j] = *reinterpret_cast<const uint4*>(kbase + boff + j * load_step);
#pragma unroll
    for (int j = 0; j < NI; ++j) vc[j] = *reinterpret_cast<const uint4*>(vbase + boff + j * load_step);
  }
  for (int it = 0; it < n_iter; ++it) {
    const int b = first + it * kWaves;
    const int nx = it + 1;
    if (nx < n_iter) {
      if ((nx & (kWave - 1)) == 0) {
        fetch_table(nx / kWave);
        if (bad) n_iter = nx;  // stop before the first chunk holding a bad id
      }
      if (nx < n_iter) {
        const int64_t boff = (int64_t)__builtin_amdgcn_readlane(tv, nx & (kWave - 1)) * block_bytes + lane_off;
#pragma unroll
        for (int j = 0; j < NI; ++j) kn[j] = *reinterpret_cast<const uint4*>(kbase + boff + j * load_step);
#pragma unroll
        for (int j = 0; j < NI; ++j) vn[j] = *reinterpret_cast<const uint4*>(vbase + boff + j * load_step);
      }
    }

    // scores of this block: sc[j][g] for token row j*TPI + lr, query head h0 + g
    float sc[NI][G];
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int g = 0; g < G; ++g) sc[j][g] = group_sum<LPR>(dot16<ST>(kc[j], qv[g], 0.f)) * a.scale_log2;
    if (alibi) {  // signed distance of the row's token to the newest position, times the slope
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const float dist = (float)(b * kBlockTokens + j * TPI + lr - (L - 1));
#pragma unroll
        for (int g = 0; g < G; ++g) sc[j][g] = fmaf(ab[g], dist, sc[j][g]);
      }
    }

    const int visible = t_end - b * kBlockTokens;
    if (visible < kBlockTokens) {  // last block: positions >= seq_len take no part
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const bool masked = j * TPI + lr >= visible;
#pragma unroll
        for (int g = 0; g < G; ++g) sc[j][g] = masked ? -INFINITY : sc[j][g];
        // stale V may be NaN, and 0 * NaN = NaN
        vc[j].x = masked ? 0u : vc[j].x;
        vc[j].y = masked ? 0u : vc[j].y;
        vc[j].z = masked ? 0u : vc[j].z;
        vc[j].w = masked ? 0u : vc[j].w;
      }
    }

#pragma unroll
    for (int g = 0; g < G; ++g) {
      float bm = sc[0][g];
#pragma unroll
      for (int j = 1; j < NI; ++j) bm = fmaxf(bm, sc[j][g]);
      const float mn = fmaxf(m[g], bm);
      // a lane row may not have seen a visible token yet (mn = -inf): use 0 as the
      // exponent reference so exp2(-inf - ref) gives 0 instead of NaN
      const float ref = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(m[g] - ref);
      m[g] = mn;
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const float p = fast_exp2(sc[j][g] - ref);
        l[g] += p;
        sc[j][g] = p;
      }
    }
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float v = elem<ST>(vc[j], e);
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g][e] = fmaf(sc[j][g], v, acc[g][e]);
      }

#pragma unroll
    for (int j = 0; j < NI; ++j) {
      kc[j] = kn[j];
      vc[j] = vn[j];
    }
  }

  // ---- merge the TPI x kWaves partial states of this unit -----------------------
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) sm_acc[w][lr][g][li * EPL + e] = acc[g][e];
  if (li == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sm_m[w][lr][g] = m[g];
      sm_l[w][lr][g] = l[g];
    }
  }
  if (lane == 0) sm_bad[w] = bad ? 1 : 0;
  __syncthreads();

  bool any_bad = false;
#pragma unroll
  for (int ww = 0; ww < kWaves; ++ww) any_bad |= sm_bad[ww] != 0;

  for (int o = threadIdx.x; o < G * D; o += kWaves * kWave) {
    const int g = o / D;
    const int d = o - g * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww)
#pragma unroll
      for (int r = 0; r < TPI; ++r) M = fmaxf(M, sm_m[ww][r][g]);
    float lsum = 0.f, osum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww)
#pragma unroll
        for (int r = 0; r < TPI; ++r) {
          const float f = fast_exp2(sm_m[ww][r][g] - M);
          lsum = fmaf(sm_l[ww][r][g], f, lsum);
          osum = fmaf(sm_acc[ww][r][g][d], f, osum);
        }
    }
    float res = M == -INFINITY ? 0.f : osum / lsum;
    if (any_bad) res = NAN;
    const int64_t sh = (int64_t)s * a.num_q_heads + h0 + g;
    if constexpr (SPLIT) {
      const int64_t sp = sh * a.max_partitions + part;
      a.tmp_out[sp * D + d] = res;
      if (d == 0) {
        a.max_logits[sp] = any_bad ? NAN : M * kLn2;
        a.exp_sums[sp] = any_bad ? NAN : lsum;
      }
    } else {
      const uint32_t bits = to_storage<ST>(res);
      if constexpr (EB == 4)
        static_cast<uint32_t*>(a.out)[sh * D + d] = bits;
      else
        static_cast<uint16_t*>(a.out)[sh * D + d] = (uint16_t)bits;
    }
  }
}

template <class ST, int D, int G>
hipError_t launch_typed(const DecodeArgs& a, bool split, hipStream_t stream) {
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * (split ? a.max_partitions : 1);
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)units), block(kWaves * kWave);
  if (split)
    hipLaunchKernelGGL((decode_kernel<ST, D, G, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<ST, D, G, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <class ST, int D>
hipError_t launch_group(const DecodeArgs& a, bool split, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_typed<ST, D, 1>(a, split, stream);
    case 2: return launch_typed<ST, D, 2>(a, split, stream);
    case 4: return launch_typed<ST, D, 4>(a, split, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class ST>
hipError_t launch_dim(const DecodeArgs& a, int head_size, bool split, hipStream_t stream) {
  switch (head_size) {
    case 64: return launch_group<ST, 64>(a, split, stream);
    case 128: return launch_group<ST, 128>(a, split, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_supported(int dtype, int head_size, int group) {
  if (head_size != 64 && head_size != 128) return false;
  if (dtype == 0) return group == 1 || group == 2 || group == 4;
  if (dtype == 1 || dtype == 2) return group == 1 || group == 2 || group == 4 || group == 8;
  return false;
}

// fp32 storage runs the VALU kernel above; fp16 / bf16 take the matrix-core kernel.
hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_size, bool split, hipStream_t stream) {
  if (a.kv8 && dtype != 1 && dtype != 2) return hipErrorInvalidValue;  // 8-bit pools: 16-bit queries only
  switch (dtype) {
    case 0: return launch_dim<F32>(a, head_size, split, stream);
    case 1:
    case 2: return launch_decode_mfma(a, dtype, head_size, split, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pcache
