// decode_mfma.hip -- paged decode attention for 16-bit storage (fp16 / bf16) with the
// q.k products on the matrix cores.
//
// What is computed is the same as decode.hip ("vLLM 源码完全拆解（七）: PagedAttention
// Kernel", sections 先明确问题, 线程组织, 第一步, 第三步 and V1与V2; "Inside vLLM CUDA
// Kernels", Part 3, "How Each K/V Tile Contributes to the Output"): per (sequence,
// query head) a softmax over the visible positions of scale * q.k, times V; or, on
// the split path, the same over one 512-token partition with (out, max, sum) stored.
//
// gfx950 mapping of one wave's work on one 16-token block of one kv head:
// * q.k as one 16x16 tile: v_mfma_f32_16x16x32_{bf16,f16} with A = the block's K
//   (16 token rows x 32 dims per instruction) and B = the group's query heads
//   (G <= 8 of the 16 columns, the rest zero), head_size/32 instructions per block.
//   Lane l receives the scores of tokens 4*(l/16) + i (i < 4) for head l % 16, so a
//   lane (row group r = l/16, head g = l%16 < G) owns the softmax of its 4 tokens
//   and computes each probability exactly once.
// * Online softmax with a lazy reference: the exponent reference m_ref of a (row
//   group, head) stream moves only when a block's max exceeds it by more than
//   2^8 (log2 domain), so most blocks skip the accumulator rescale entirely (a
//   wave-uniform branch); the true running max is tracked alongside and the final
//   state is expressed relative to it.
// * The 16 probabilities of a row group and the rescale factors go through a few
//   LDS words to the lanes that hold the row group's V slices; P.V then runs on
//   the VALU in fp32: lane (r, i) holds 16 bytes of each of its tokens' V rows and
//   all G heads' accumulators for those 8 (or, for head_size 64, 8 of 64) dims.
// * A ring of STAGES register sets keeps the next STAGES-1 blocks' K/V loads in
//   flight while one block is consumed; each wave reads its block ids 64 at a time
//   into one VGPR.  A unit's waves merge their states once, at the end.
//
// Work distribution:
// * Split path: one workgroup per (sequence, kv head, 512-token partition); the
//   partitions are equal-sized, so the grid balances itself.
// * One-pass path: a unit is a whole (sequence, kv head) and unit lengths can differ
//   several-fold, so a grid of one unit per workgroup ends with a few long units
//   running alone.  Instead the kernel is persistent: one workgroup per resident
//   slot; units are ordered longest first and dealt in snake order (workgroup k of
//   W takes positions k, 2W-1-k, 2W+k, ...), so every workgroup receives about the
//   same number of blocks.  Each unit is still computed by exactly one workgroup.
#include <cmath>

#include "device_common.h"
#include "launch.h"

namespace pcache {
namespace {

constexpr int kBlockTokens = 16;
constexpr int kPartition = 512;
constexpr float kLazy = 8.f;         // log2-domain slack before the exponent reference moves
constexpr int kMaxRankedSeqs = 512;  // sequences ranked by length in-kernel (beyond: index order)

#ifndef PCACHE_ONEPASS_WAVES
#define PCACHE_ONEPASS_WAVES 8
#endif
#ifndef PCACHE_ONEPASS_STAGES
#define PCACHE_ONEPASS_STAGES 2
#endif
#ifndef PCACHE_SPLIT_WAVES
#define PCACHE_SPLIT_WAVES 4
#endif
#ifndef PCACHE_SPLIT_STAGES
#define PCACHE_SPLIT_STAGES 2
#endif

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <class ST>
__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c);
template <>
__device__ __forceinline__ f32x4_t mfma16<BF16>(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4_t mfma16<F16>(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int NW, int D, int G>
struct UnitLds {
  __align__(16) float p[NW][4][4 * G];  // probabilities of a row group (read as float4)
  __align__(16) float a[NW][4][G];      // rescale / fold factors of a row group
  __align__(16) float acc[NW][G][D];    // each wave's folded accumulator
  float mw[NW][G];
  float lw[NW][G];
  int bad[NW];
};

// One unit: kv head `kvh` of sequence `s`, tokens [t_begin, t_end).  All waves of
// the workgroup call it together (it ends with a barrier-separated merge).  Writes
// out (one pass) or the partition's partials (split).
template <class ST, int D, int G, int NW, int STAGES, bool SPLIT>
__device__ __forceinline__ void decode_unit(const DecodeArgs& a, UnitLds<NW, D, G>& sm, int s, int kvh, int part) {
  static_assert(ST::kBytes == 2, "16-bit storage only");
  static_assert(D == 64 || D == 128, "head size 64 or 128");
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group of 1, 2, 4 or 8 query heads");
  static_assert(STAGES >= 2 && STAGES <= 4, "prefetch ring of 2..4 register sets");
  constexpr int KS = D / 32;    // MFMA k-steps per block
  constexpr int RL = D / 8;     // lanes per V token row (16-byte slices)
  constexpr int RPG = 16 / RL;  // V rows per row group per load
  constexpr int NJ = 4 / RPG;   // V loads per block

  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int rg = lane >> 4;     // row group: tokens 4*rg .. 4*rg+3 of a block
  const int col = lane & 15;    // MFMA column (query head of the group) / V slice index
  const int vsub = col / RL;    // which of the row group's rows this lane loads per V load
  const int vchunk = col % RL;  // 16-byte slice of a V row

  const int L = a.seq_lens[s];
  bool bad = L < 0 || (int64_t)L > (int64_t)a.max_blocks_per_seq * kBlockTokens ||
             (SPLIT && (int64_t)L > (int64_t)a.max_partitions * kPartition);
  const int t_begin = SPLIT ? part * kPartition : 0;
  const int t_end = bad ? t_begin : (SPLIT ? min(L, t_begin + kPartition) : L);
  const int b_begin = t_begin / kBlockTokens;
  const int b_end = (t_end + kBlockTokens - 1) / kBlockTokens;
  const int h0 = kvh * G;
  const float cs = a.scale_log2;  // > 0 (validated on the host)

  // B operand: query head `col` (zero for col >= G), dims 32*k + 8*rg .. +8
  uint4 qb[KS];
  {
    const int qh = col < G ? col : G - 1;  // keep the address inside q for the zero columns
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((int64_t)s * a.num_q_heads + h0 + qh) * D + 8 * rg;
#pragma unroll
    for (int k = 0; k < KS; ++k)
      qb[k] = col < G ? *reinterpret_cast<const uint4*>(qrow + 32 * k) : make_uint4(0, 0, 0, 0);
  }

  // softmax state of stream (row group rg, head col) -- meaningful for col < G
  float m_ref = -INFINITY, m_true = -INFINITY, lsum = 0.f;
  float acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;

  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int64_t head_off = (int64_t)kvh * a.head_stride * 2;
  const char* kbase = static_cast<const char*>(a.k_pool) + head_off;
  const char* vbase = static_cast<const char*>(a.v_pool) + head_off;
  const int64_t tok_bytes = a.token_stride * 2;
  const int64_t k_lane = (int64_t)col * tok_bytes + 16 * rg;  // + 64*k per MFMA step
  const int64_t v_lane = (int64_t)(4 * rg + vsub) * tok_bytes + 16 * vchunk;
  const int64_t v_step = (int64_t)RPG * tok_bytes;
  const int64_t block_bytes = a.block_stride * 2;

  // This wave takes blocks first, first + NW, ...: nw of them.
  const int first = b_begin + w;
  const int nw = first < b_end ? (b_end - first + NW - 1) / NW : 0;
  int tv = 0;
  auto fetch_table = [&](int chunk) {
    const int idx = chunk * kWave + lane;
    int v = 0;
    if (idx < nw) v = table[first + idx * NW];
    if (__builtin_amdgcn_ballot_w64(idx < nw && (v < 0 || (int64_t)v >= a.num_blocks)) != 0) bad = true;
    tv = v;
  };
  int n_iter = nw;
  if (n_iter > 0) {
    fetch_table(0);
    if (bad) n_iter = 0;  // a block id outside the pool: nothing is read, the outputs become NaN
  }

  uint4 kb[STAGES][KS], vb[STAGES][NJ];

#define PC_LOAD(KD, VD, IT)                                                                          \
  do {                                                                                               \
    const int64_t boff = (int64_t)__builtin_amdgcn_readlane(tv, (IT) & (kWave - 1)) * block_bytes; \
    _Pragma("unroll") for (int k = 0; k < KS; ++k) KD[k] =                                          \
        *reinterpret_cast<const uint4*>(kbase + boff + k_lane + 64 * k);                             \
    _Pragma("unroll") for (int j = 0; j < NJ; ++j) VD[j] =                                          \
        *reinterpret_cast<const uint4*>(vbase + boff + v_lane + j * v_step);                         \
  } while (0)

  // consume block IT whose K/V sit in KC/VC
#define PC_BLOCK(KC, VC, IT)                                                                         \
  do {                                                                                               \
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};                                                                \
    _Pragma("unroll") for (int k = 0; k < KS; ++k) c = mfma16<ST>(KC[k], qb[k], c);                 \
    const int visible = t_end - (first + (IT) * NW) * kBlockTokens;                                  \
    if (visible < kBlockTokens) {                                                                    \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) c[i] = 4 * rg + i < visible ? c[i] : -INFINITY; \
      _Pragma("unroll") for (int j = 0; j < NJ; ++j) {                                              \
        const bool mk = 4 * rg + j * RPG + vsub >= visible;                                          \
        VC[j].x = mk ? 0u : VC[j].x;                                                                 \
        VC[j].y = mk ? 0u : VC[j].y;                                                                 \
        VC[j].z = mk ? 0u : VC[j].z;                                                                 \
        VC[j].w = mk ? 0u : VC[j].w;                                                                 \
      }                                                                                              \
    }                                                                                                \
    const float bm = fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3]));                                    \
    m_true = fmaxf(m_true, bm);                                                                      \
    const bool need = col < G && bm > m_ref + lazy_raw;                                              \
    const bool rescale = __builtin_amdgcn_ballot_w64(need) != 0;                                     \
    wave_lds_sync(); /* the previous block's loads of sm.p / sm.a come before these stores */        \
    if (rescale) {                                                                                   \
      const float alpha = need ? exp2_fast((m_ref - bm) * cs) : 1.f;                                 \
      m_ref = need ? bm : m_ref;                                                                     \
      lsum *= alpha;                                                                                 \
      if (col < G) sm.a[w][rg][col] = alpha;                                                         \
    }                                                                                                \
    const float ref = m_ref == -INFINITY ? 0.f : m_ref * cs;                                         \
    float pr[4];                                                                                     \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) pr[i] = exp2_fast(fmaf(c[i], cs, -ref));          \
    lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);                                                       \
    if (col < G)                                                                                     \
      *reinterpret_cast<float4*>(&sm.p[w][rg][4 * col]) = make_float4(pr[0], pr[1], pr[2], pr[3]);  \
    wave_lds_sync(); /* other lanes' stores above are visible to the loads below */                 \
    if (rescale) {                                                                                   \
      _Pragma("unroll") for (int g = 0; g < G; ++g) {                                               \
        const float al = sm.a[w][rg][g];                                                             \
        _Pragma("unroll") for (int e = 0; e < 8; ++e) acc[g][e] *= al;                              \
      }                                                                                              \
    }                                                                                                \
    float pv[G][4];                                                                                  \
    _Pragma("unroll") for (int g = 0; g < G; ++g) {                                                 \
      const float4 t4 = *reinterpret_cast<const float4*>(&sm.p[w][rg][4 * g]);                      \
      pv[g][0] = t4.x;                                                                               \
      pv[g][1] = t4.y;                                                                               \
      pv[g][2] = t4.z;                                                                               \
      pv[g][3] = t4.w;                                                                               \
    }                                                                                                \
    _Pragma("unroll") for (int j = 0; j < NJ; ++j) {                                                \
      const int tj = j * RPG + vsub;                                                                 \
      _Pragma("unroll") for (int e = 0; e < 8; ++e) {                                               \
        const float v = elem<ST>(VC[j], e);                                                          \
        _Pragma("unroll") for (int g = 0; g < G; ++g) acc[g][e] = fmaf(pv[g][tj], v, acc[g][e]);    \
      }                                                                                              \
    }                                                                                                \
  } while (0)

  const float lazy_raw = kLazy / cs;
  if (n_iter > 0) {
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
      if (st < n_iter) PC_LOAD(kb[st], vb[st], st);
  }
  for (int it0 = 0; it0 < n_iter; it0 += STAGES) {
#pragma unroll
    for (int st = 0; st < STAGES; ++st) {
      const int it = it0 + st;
      if (it >= n_iter) break;
      const int nx = it + STAGES - 1;  // the block this step starts fetching
      if (nx < n_iter) {
        if ((nx & (kWave - 1)) == 0) {
          fetch_table(nx / kWave);
          if (bad) n_iter = nx;  // stop before the first chunk holding a bad id
        }
        if (nx < n_iter) PC_LOAD(kb[(st + STAGES - 1) % STAGES], vb[(st + STAGES - 1) % STAGES], nx);
      }
      PC_BLOCK(kb[st], vb[st], it);
    }
  }
#undef PC_LOAD
#undef PC_BLOCK

  // ---- this wave: fold its 4 row groups into one state per head ---------------------
  // reference for head g: the wave's true max M_w[g]; stream (rg, g) carries
  // f = 2^((m_ref - M_w) * cs) <= 1
  float mw = m_true;
  mw = fmaxf(mw, __shfl_xor(mw, 16));
  mw = fmaxf(mw, __shfl_xor(mw, 32));
  const float f = m_ref == -INFINITY ? 0.f : exp2_fast((m_ref - mw) * cs);
  float lw = lsum * f;
  lw += __shfl_xor(lw, 16);
  lw += __shfl_xor(lw, 32);
  wave_lds_sync();
  if (col < G) sm.a[w][rg][col] = f;
  wave_lds_sync();
  float fr[G];
#pragma unroll
  for (int g = 0; g < G; ++g) fr[g] = sm.a[w][rg][g];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[g][e] * fr[g];
      if constexpr (RPG == 2) x += dpp<0x128>(x);  // row_ror:8 -- the row group's other V row
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[g][e] = x;
    }
  if (rg == 0 && vsub == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.acc[w][g][8 * vchunk + e] = acc[g][e];
  }
  if (rg == 0 && col < G) {
    sm.mw[w][col] = mw;
    sm.lw[w][col] = lw;
  }
  if (lane == 0) sm.bad[w] = bad ? 1 : 0;
  __syncthreads();

  // ---- merge the waves and write ------------------------------------------------------
  bool any_bad = false;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) any_bad |= sm.bad[ww] != 0;
  for (int o = threadIdx.x; o < G * D; o += NW * kWave) {
    const int g = o / D;
    const int d = o - g * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm.mw[ww][g]);
    float ls = 0.f, os = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float fw = sm.mw[ww][g] == -INFINITY ? 0.f : exp2_fast((sm.mw[ww][g] - M) * cs);
        ls = fmaf(sm.lw[ww][g], fw, ls);
        os = fmaf(sm.acc[ww][g][d], fw, os);
      }
    }
    float res = M == -INFINITY ? 0.f : os / ls;
    if (any_bad) res = NAN;
    const int64_t sh = (int64_t)s * a.num_q_heads + h0 + g;
    if constexpr (SPLIT) {
      const int64_t sp = sh * a.max_partitions + part;
      a.tmp_out[sp * D + d] = res;
      if (d == 0) {
        a.max_logits[sp] = any_bad ? NAN : M * (cs * kLn2);  // back to the natural-log domain
        a.exp_sums[sp] = any_bad ? NAN : ls;
      }
    } else {
      static_cast<uint16_t*>(a.out)[sh * D + d] = (uint16_t)to_storage<ST>(res);
    }
  }
}

// Split path: workgroup = (kv head, sequence, partition), fastest-varying first.
template <class ST, int D, int G>
__global__ __launch_bounds__(PCACHE_SPLIT_WAVES* kWave) void decode_split_kernel(DecodeArgs a) {
  constexpr int NW = PCACHE_SPLIT_WAVES;
  __shared__ UnitLds<NW, D, G> sm;
  int64_t id = blockIdx.x;
  const int kvh = (int)(id % a.num_kv_heads);
  id /= a.num_kv_heads;
  const int s = (int)(id % a.num_seqs);
  const int part = (int)(id / a.num_seqs);
  const int L = a.seq_lens[s];
  const bool bad = L < 0 || (int64_t)L > (int64_t)a.max_blocks_per_seq * kBlockTokens ||
                   (int64_t)L > (int64_t)a.max_partitions * kPartition;
  if (!bad && part * kPartition >= L) return;  // a partition past the sequence writes nothing
  decode_unit<ST, D, G, NW, PCACHE_SPLIT_STAGES, true>(a, sm, s, kvh, part);
}

// One-pass path: persistent workgroups, units longest first, dealt in snake order.
template <class ST, int D, int G>
__global__ __launch_bounds__(PCACHE_ONEPASS_WAVES* kWave) void decode_onepass_kernel(DecodeArgs a) {
  constexpr int NW = PCACHE_ONEPASS_WAVES;
  constexpr int kThreads = NW * kWave;
  __shared__ UnitLds<NW, D, G> sm;
  __shared__ int order_lds[kMaxRankedSeqs];  // order_lds[rank] = sequence of that length rank
  __shared__ int len_lds[kMaxRankedSeqs];

  const int S = a.num_seqs;
  const bool ranked = a.longest_first && S <= kMaxRankedSeqs;
  if (ranked) {
    for (int t = threadIdx.x; t < S; t += kThreads) len_lds[t] = a.seq_lens[t];
    __syncthreads();
    for (int t = threadIdx.x; t < S; t += kThreads) {
      const int lt = len_lds[t];
      int rank = 0;
      for (int u = 0; u < S; ++u) {
        const int lu = len_lds[u];
        rank += (lu > lt) || (lu == lt && u < t);
      }
      order_lds[rank] = t;
    }
    __syncthreads();
  }
  const int64_t units = (int64_t)S * a.num_kv_heads;
  const int64_t W = gridDim.x;
  const int64_t k = blockIdx.x;
  for (int64_t round = 0; round * W < units; ++round) {
    const int64_t pos = round * W + ((round & 1) ? W - 1 - k : k);
    if (pos >= units) continue;  // the last round is partial
    const int rank = (int)(pos / a.num_kv_heads);
    const int kvh = (int)(pos % a.num_kv_heads);
    const int s = ranked ? order_lds[rank] : rank;
    decode_unit<ST, D, G, NW, PCACHE_ONEPASS_STAGES, false>(a, sm, s, kvh, 0);
    __syncthreads();  // the next unit reuses the LDS merge buffers
  }
}

// Resident workgroups per CU for the one-pass kernel, queried once per instance.
template <class ST, int D, int G>
int onepass_blocks_per_cu() {
  static int cached = 0;
  if (!cached) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_onepass_kernel<ST, D, G>,
                                                     PCACHE_ONEPASS_WAVES * kWave, 0) != hipSuccess ||
        n <= 0) {
      (void)hipGetLastError();
      n = 1;
    }
    cached = n;
  }
  return cached;
}

template <class ST, int D, int G>
hipError_t launch_typed(const DecodeArgs& a, bool split, hipStream_t stream) {
  if (split) {
    const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * a.max_partitions;
    if (units == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_split_kernel<ST, D, G>), dim3((unsigned)units), dim3(PCACHE_SPLIT_WAVES * kWave), 0,
                       stream, a);
    return hipGetLastError();
  }
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads;
  if (units == 0) return hipSuccess;
  const int64_t slots = (int64_t)device_compute_units() * onepass_blocks_per_cu<ST, D, G>();
  const int64_t grid = units < slots ? units : slots;
  hipLaunchKernelGGL((decode_onepass_kernel<ST, D, G>), dim3((unsigned)grid), dim3(PCACHE_ONEPASS_WAVES * kWave), 0,
                     stream, a);
  return hipGetLastError();
}

template <class ST, int D>
hipError_t launch_group(const DecodeArgs& a, bool split, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_typed<ST, D, 1>(a, split, stream);
    case 2: return launch_typed<ST, D, 2>(a, split, stream);
    case 4: return launch_typed<ST, D, 4>(a, split, stream);
    case 8: return launch_typed<ST, D, 8>(a, split, stream);
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

hipError_t launch_decode_mfma(const DecodeArgs& a_in, int dtype, int head_size, bool split, hipStream_t stream) {
  DecodeArgs a = a_in;
#ifndef PCACHE_LONGEST_FIRST
#define PCACHE_LONGEST_FIRST 1
#endif
  a.longest_first = PCACHE_LONGEST_FIRST && !split && a.num_seqs > 1;
  switch (dtype) {
    case 1: return launch_dim<F16>(a, head_size, split, stream);
    case 2: return launch_dim<BF16>(a, head_size, split, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pcache
