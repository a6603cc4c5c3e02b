// varlen.hip -- attention of several query tokens per request over the paged K/V
// (chunked prefill, speculative decode), 16-bit storage, on the matrix cores.
//
// What is computed ("Inside vLLM CUDA Kernels", Part 3, "How Metadata Connects a Q
// Tile to Paged K/V" and "How Each K/V Tile Contributes to the Output"): request r
// owns rows [qs[r], qs[r+1]) of the packed query -- its newest n = qs[r+1] - qs[r]
// tokens, so query token i sits at position p = L_r - n + i.  Causally it attends
// positions t <= p, otherwise all of [0, L_r); scores scale * q.k (plus an optional
// ALiBi bias slope_h * (t - p)), softmax, times V.  With n = 1 this is the decode.
//
// gfx950 mapping.  A work unit is (request, kv head, chunk of QT query tokens).  The
// unit's QC = 16 * NQ (query token, head) pairs are the columns of NQ score tiles
// computed exactly as the decode's single tile: v_mfma_f32_16x16x32 with A = a
// 16-token K block and B = the query columns, then a lazy online softmax per column
// and out^T += V^T . P^T on v_mfma_f32_16x16x16, the V^T operand of each output tile
// shared by the NQ column tiles.  So each K/V block read from HBM or L2 serves QC
// query rows.  The unit's visible blocks are dealt to the workgroup's waves
// round-robin, each with its own softmax state per column; the states meet once, in
// LDS, at the end.  Causality is a per-column limit applied to the scores; rows past
// the unit's last visible position are zeroed in V (they may be stale).
#include <cmath>

#include "device_common.h"
#include "launch.h"
#include "mfma_common.h"

namespace pcache {
namespace {

constexpr int kTok = 16;          // tokens per score tile row block (the block size)
constexpr int kWaves = 4;         // waves per unit
constexpr int kTable = 512;       // block ids staged in LDS at once
constexpr float kLazyV = 8.f;     // log2-domain slack before a column's exponent reference moves

template <int QC, int D>
struct VarlenLds {
  __align__(16) float acc[kWaves][QC][D];
  float mw[kWaves][QC];
  float lw[kWaves][QC];
  int ids[kTable];
  int bad;
};

template <class ST, int D, int G, int NQ, bool ALIBI>
__global__ __launch_bounds__(kWaves* kWave) __attribute__((amdgpu_waves_per_eu(2))) void varlen_kernel(VarlenArgs a) {
  static_assert(ST::kBytes == 2, "16-bit storage only");
  constexpr int QC = 16 * NQ;  // (query token, head) columns per unit
  constexpr int QT = QC / G;   // query tokens per unit
  constexpr int KS = D / 32;   // q.k k-steps per block
  constexpr int DPL = D / 16;  // V dims a lane loads per row = output tiles
  constexpr int NT = DPL;
  constexpr int kThreads = kWaves * kWave;
  constexpr int kStage = (kTable + kThreads - 1) / kThreads;
  using VRow = typename VRowOf<DPL>::type;
  __shared__ VarlenLds<QC, D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int rg = lane >> 4;
  const int col = lane & 15;

  int64_t unit = blockIdx.x;
  const int kvh = (int)(unit % a.num_kv_heads);
  unit /= a.num_kv_heads;
  const int r = (int)(unit % a.num_reqs);
  const int chunk0 = (int)(unit / a.num_reqs);
  const int chunks = (int)(gridDim.x / ((int64_t)a.num_kv_heads * a.num_reqs));

  const int q0 = uniform_load(a.query_start_loc, r);
  const int q1 = uniform_load(a.query_start_loc, r + 1);
  if (q0 < 0 || q1 < q0 || (int64_t)q1 > a.total_q) return;  // no rows this request may write
  const int n = q1 - q0;
  const int L = uniform_load(a.seq_lens, r);
  const bool bad_len = L < n || (int64_t)L > (int64_t)a.max_blocks_per_seq * kTok;
  const int h0 = kvh * G;
  const float cs = a.scale_log2;
  const float lazy_raw = kLazyV / cs;
  constexpr bool alibi = ALIBI;
  const int32_t* table = a.block_tables + (int64_t)r * a.max_blocks_per_seq;
  const int64_t head_bytes = (int64_t)kvh * a.head_stride * 2;
  const char* kpool = static_cast<const char*>(a.k_pool) + head_bytes;
  const char* vpool = static_cast<const char*>(a.v_pool) + head_bytes;
  const int64_t block_bytes = a.block_stride * 2;
  const int tok_bytes = (int)(a.token_stride * 2);
  const uint32_t tile_bytes = (uint32_t)(kTok * tok_bytes);
  const int k_off = col * tok_bytes + 16 * rg;
  const int v_off = 4 * rg * tok_bytes + col * (2 * DPL);

  for (int c = chunk0; c * QT < n; c += chunks) {
    const int i0 = c * QT;                   // first query token of the unit
    const int i_end = min(n, i0 + QT);       // one past its last
    // positions this unit may see: up to its last token's (causal) or the whole history
    const int vis_end = bad_len ? 0 : (a.causal ? L - n + i_end : L);
    bool bad = bad_len;

    // column 16*q + col of this lane: query token i0 + (16q + col) / G, head (16q + col) % G
    uint4 qb[NQ][KS];
    int lim[NQ];    // last visible position of the column (-1: no such column)
    int pos[NQ];    // position of the column's query token
    float ab[NQ];   // ALiBi slope in raw q.k units
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int cc = 16 * q + col;
      const int ti = i0 + cc / G;
      const bool valid = ti < i_end;
      const int g = cc % G;
      pos[q] = L - n + ti;
      lim[q] = valid ? (a.causal ? pos[q] : L - 1) : -1;
      const int tq = valid ? ti : i_end - 1;  // keeps the address inside q
      const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((int64_t)(q0 + tq) * a.num_q_heads + h0 + g) * D +
                             8 * rg;
#pragma unroll
      for (int k = 0; k < KS; ++k)
        qb[q][k] = valid ? *reinterpret_cast<const uint4*>(qrow + 32 * k) : make_uint4(0, 0, 0, 0);
      ab[q] = 0.f;
      if (alibi) {
        float sl = 0.f;
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
          const float v = uniform_load(a.alibi_slopes, h0 + gg);
          sl = g == gg ? v : sl;
        }
        ab[q] = sl * kLog2e / cs;
      }
    }

    float m_ref[NQ], m_true[NQ], lsum[NQ];
    f32x4_t acc[NQ][NT];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      m_ref[q] = -INFINITY;
      m_true[q] = -INFINITY;
      lsum[q] = 0.f;
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[q][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    uint4 kb[2][KS];
    VRow vb[2][4];

#define VL_LOAD(SL, BID)                                                                              \
  do {                                                                                                \
    const int64_t boff_ = (int64_t)(BID) * block_bytes;                                               \
    const __amdgpu_buffer_rsrc_t kr_ = tile_rsrc(kpool + boff_, tile_bytes);                          \
    const __amdgpu_buffer_rsrc_t vr_ = tile_rsrc(vpool + boff_, tile_bytes);                          \
    _Pragma("unroll") for (int k = 0; k < KS; ++k) kb[SL][k] =                                       \
        __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr_, k_off + 64 * k, 0, 0));  \
    _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                                  \
      if constexpr (DPL == 8)                                                                         \
        vb[SL][e] = __builtin_bit_cast(VRow, __builtin_amdgcn_raw_buffer_load_b128(vr_, v_off, e * tok_bytes, 0)); \
      else                                                                                            \
        vb[SL][e] = __builtin_bit_cast(VRow, __builtin_amdgcn_raw_buffer_load_b64(vr_, v_off, e * tok_bytes, 0)); \
    }                                                                                                 \
  } while (0)

#define VL_BLOCK(SL, TOK0)                                                                            \
  do {                                                                                                \
    const int t0_ = (TOK0) + 4 * rg; /* this lane's first token row */                                \
    if (vis_end - (TOK0) < kTok) { /* rows past the unit's last visible position: stale V */          \
      _Pragma("unroll") for (int e = 0; e < 4; ++e) vb[SL][e] = t0_ + e < vis_end ? vb[SL][e] : VRow{}; \
    }                                                                                                 \
    uint2 pb[NQ], pl[NQ];                                                                             \
    _Pragma("unroll") for (int q = 0; q < NQ; ++q) {                                                  \
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};                                                               \
      _Pragma("unroll") for (int k = 0; k < KS; ++k) c = mfma16<ST>(kb[SL][k], qb[q][k], c);          \
      _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                                 \
        if (alibi) c[e] = fmaf(ab[q], (float)(t0_ + e - pos[q]), c[e]);                               \
        c[e] = t0_ + e <= lim[q] ? c[e] : -INFINITY;                                                  \
      }                                                                                               \
      const float lm = fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3]));                                   \
      m_true[q] = fmaxf(m_true[q], lm);                                                               \
      if (__builtin_amdgcn_ballot_w64(lm > m_ref[q] + lazy_raw) != 0) {                               \
        float hm = fmaxf(lm, __shfl_xor(lm, 16));                                                     \
        hm = fmaxf(hm, __shfl_xor(hm, 32));                                                           \
        const bool mv = hm > m_ref[q] + lazy_raw;                                                     \
        const float alpha = mv ? exp2_fast((m_ref[q] - hm) * cs) : 1.f;                               \
        m_ref[q] = mv ? hm : m_ref[q];                                                                \
        lsum[q] *= alpha;                                                                             \
        _Pragma("unroll") for (int j = 0; j < NT; ++j) acc[q][j] *= alpha;                           \
      }                                                                                               \
      const float ref = m_ref[q] == -INFINITY ? 0.f : m_ref[q] * cs;                                  \
      float pr[4];                                                                                    \
      _Pragma("unroll") for (int e = 0; e < 4; ++e) pr[e] = exp2_fast(fmaf(c[e], cs, -ref));         \
      lsum[q] += (pr[0] + pr[1]) + (pr[2] + pr[3]);                                                   \
      pb[q] = make_uint2(pack2<ST>(pr[0], pr[1]), pack2<ST>(pr[2], pr[3]));                           \
      if constexpr (kSplitP<ST>)                                                                      \
        pl[q] = make_uint2(residual2(pb[q].x, pr[0], pr[1]), residual2(pb[q].y, pr[2], pr[3]));       \
    }                                                                                                 \
    _Pragma("unroll") for (int j = 0; j < NT; ++j) {                                                  \
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;                                       \
      const uint2 va = make_uint2(__builtin_amdgcn_perm(vword(vb[SL][1], j >> 1), vword(vb[SL][0], j >> 1), sel), \
                                  __builtin_amdgcn_perm(vword(vb[SL][3], j >> 1), vword(vb[SL][2], j >> 1), sel)); \
      _Pragma("unroll") for (int q = 0; q < NQ; ++q) {                                                \
        acc[q][j] = mfma_pv<ST>(va, pb[q], acc[q][j]);                                                \
        if constexpr (kSplitP<ST>) acc[q][j] = mfma_pv<ST>(va, pl[q], acc[q][j]);                     \
      }                                                                                               \
    }                                                                                                 \
  } while (0)

    if (tid == 0) sm.bad = 0;
    lds_barrier();  // the previous unit's readers of sm are done
    const int b_end = (vis_end + kTok - 1) / kTok;
    for (int cb = 0; cb < b_end; cb += kTable) {
      const int cn = min(kTable, b_end - cb);
      if (cb != 0) lds_barrier();  // every wave has read the previous chunk's ids
      const int nwc = __builtin_amdgcn_readfirstlane(w < cn ? (cn - w + kWaves - 1) / kWaves : 0);
      int staged[kStage];
#pragma unroll
      for (int s = 0; s < kStage; ++s) {
        const int i = tid + s * kThreads;
        staged[s] = i < cn ? table[cb + i] : 0;
      }
      {  // the wave's first block, loaded before the staging completes (invalid ids: block 0)
        const int id0 = uniform_load(table, cb + min(w, cn - 1));
        VL_LOAD(0, (id0 >= 0 && (int64_t)id0 < a.num_blocks) ? id0 : 0);
      }
#pragma unroll
      for (int s = 0; s < kStage; ++s) {
        const int i = tid + s * kThreads;
        if (i < cn) {
          sm.ids[i] = staged[s];
          if (staged[s] < 0 || (int64_t)staged[s] >= a.num_blocks) sm.bad = 1;
        }
      }
      lds_barrier();
      if (__builtin_amdgcn_readfirstlane(sm.bad)) {
        bad = true;
        break;
      }
      if (nwc == 0) continue;
      auto id_of = [&](int j) -> int { return sm.ids[w + min(j, nwc - 1) * kWaves]; };
      int id_next = id_of(1);
      int it0 = 0;
      do {  // a whole number of two-step turns; a step past the last block is fully masked
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int it = it0 + st;
          VL_LOAD(st ^ 1, __builtin_amdgcn_readfirstlane(id_next));
          id_next = id_of(it + 2);
          __builtin_amdgcn_sched_barrier(0);
          VL_BLOCK(st, it < nwc ? (cb + w + it * kWaves) * kTok : vis_end);
        }
        it0 += 2;
      } while (it0 < nwc);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // retire the unconsumed prefetch
    }
#undef VL_LOAD
#undef VL_BLOCK

    // ---- this wave's state per column, relative to the column's true max -------------
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float mt = fmaxf(m_true[q], __shfl_xor(m_true[q], 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float f = m_ref[q] == -INFINITY ? 0.f : exp2_fast((m_ref[q] - mt) * cs);
      float lw = lsum[q];
      lw += __shfl_xor(lw, 16);
      lw += __shfl_xor(lw, 32);
      const int cc = 16 * q + col;
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.acc[w][cc][DPL * (4 * rg + i) + j] = acc[q][j][i] * f;
      if (rg == 0) {
        sm.mw[w][cc] = mt;
        sm.lw[w][cc] = lw * f;
      }
    }
    __syncthreads();

    // ---- merge the waves and write the unit's rows ------------------------------------
    for (int o = tid; o < QC * D; o += kThreads) {
      const int cc = o / D;
      const int d = o - cc * D;
      const int ti = i0 + cc / G;
      if (ti >= i_end) continue;
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.mw[ww][cc]);
      float ls = 0.f, os = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
          const float fw = sm.mw[ww][cc] == -INFINITY ? 0.f : exp2_fast((sm.mw[ww][cc] - M) * cs);
          ls = fmaf(sm.lw[ww][cc], fw, ls);
          os = fmaf(sm.acc[ww][cc][d], fw, os);
        }
      }
      float res = M == -INFINITY ? 0.f : os / ls;
      if (bad) res = NAN;
      const int64_t row = (int64_t)(q0 + ti) * a.num_q_heads + h0 + cc % G;
      static_cast<uint16_t*>(a.out)[row * D + d] = (uint16_t)to_storage<ST>(res);
    }
  }
}

// ---- many query columns per request: K/V tiles shared through LDS --------------------
//
// A unit of 4 waves owns 128 (query token, head) columns -- 32 per wave, two 16-column
// score tiles each, with the wave's own q, softmax state and accumulator -- and scans
// the request's visible K/V once.  Tiles go by pairs: the whole workgroup loads a pair
// of 16-token K/V tiles (each thread a fixed share of 16-byte chunks), writes it to one
// of two LDS stages and all four waves read it, after one LDS-only barrier per pair.
// Loads run kPipe - 1 = 2 pairs ahead in registers (so the compiler's waits on them stay
// exact); one pair ahead leaves the LDS writes waiting on the loads.  A pair gives each column 32 scores: one softmax update, and P.V as one
// v_mfma_f32_16x16x32 per output tile whose contraction index k = 8 rg + i stands for
// row 4 rg + i of the first tile (i < 4) or of the second (i >= 4) -- the same map for
// the V^T operand and for P^T.  Chunk c of token row r is stored at slot c ^ (r mod
// chunks-per-row), so the row-indexed 16-byte reads of K and V hit distinct banks.
// Rows past the unit's last visible position are written as zeros (the pool there may
// hold stale values).  A wave skips pairs that lie wholly past its columns' causal
// limits.
#ifndef PCACHE_VARLEN_PIPE
#define PCACHE_VARLEN_PIPE 3
#endif
constexpr int kPipe = PCACHE_VARLEN_PIPE;  // tile pairs in flight per workgroup, the one being used included

// The request of rank k when the batch's requests are ordered by history length,
// longest first (ties by index), for every thread of the workgroup.  lens is
// kRankMax + 1 ints of LDS; the batch has at most kRankMax requests.
constexpr int kRankMax = 128;
__device__ __forceinline__ int request_of_rank(const VarlenArgs& a, int k, int* lens) {
  const int tid = threadIdx.x;
  const int R = a.num_reqs;
  if (tid < R) lens[tid] = a.seq_lens[tid];
  __syncthreads();
  if (tid < R) {
    const int mine = lens[tid];
    int rk = 0;
    for (int j = 0; j < R; ++j) {
      const int o = lens[j];
      rk += (o > mine || (o == mine && j < tid)) ? 1 : 0;
    }
    if (rk == k) lens[kRankMax] = tid;  // ranks are a permutation: exactly one writer
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(lens[kRankMax]);
}

typedef short tr16x4_t __attribute__((ext_vector_type(4)));
using lds_bytes = __attribute__((address_space(3))) char*;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives 16-bit element i % 4 of
// the 8-byte reads of lanes i / 4 + 4 e, e = 0..3 (in that order)
__device__ __forceinline__ uint2 lds_read_tr16(lds_bytes p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tr16x4_t*)p));
}

// 16-byte chunk c of token row r sits at slot c ^ swizzle(r) of its LDS row.  K rows are
// read one row per lane (16 rows at once): r mod CPR spreads them over the banks.  V rows
// are read transposed, four lanes per row and four rows per 16 lanes; for 256-byte rows
// those rows need swizzles two slots apart (128-byte rows already fall on both halves of
// the banks).
template <int CPR>
__device__ __forceinline__ int k_swizzle(int r) { return r & (CPR - 1); }
template <int CPR>
__device__ __forceinline__ int v_swizzle(int r) {
  return CPR == 16 ? ((2 * r + (r >> 3)) & 15) : (r & (CPR - 1));
}

#ifndef PCACHE_VARLEN_WPE
#define PCACHE_VARLEN_WPE 2
#endif

template <class ST, int D, int G, bool ALIBI>
__global__ __launch_bounds__(kWaves* kWave) __attribute__((amdgpu_waves_per_eu(PCACHE_VARLEN_WPE)))
void varlen_lds_kernel(VarlenArgs a) {
  static_assert(ST::kBytes == 2, "16-bit storage only");
  constexpr int NQ = 2;                 // 16-column score tiles per wave
  constexpr int WC = 16 * NQ;           // columns per wave
  constexpr int QT = kWaves * WC / G;   // query tokens per unit
  constexpr int WT = WC / G;            // query tokens per wave
  constexpr int KS = D / 32;
  constexpr int NT = D / 16;            // output tiles of 16 dims
  constexpr int CPR = D / 8;            // 16-byte chunks per token row
  constexpr int TCH = kTok * CPR;       // chunks per K (or V) tile
  constexpr int kThreads = kWaves * kWave;
  constexpr int LPT = 2 * TCH / kThreads;  // chunks a thread moves per tile (K and V together)
  static_assert(LPT >= 1 && LPT * kThreads == 2 * TCH, "a tile splits evenly over the threads");
  __shared__ __align__(16) uint4 kvs[2][2][2 * TCH];  // [stage][tile of the pair][K chunks, then V chunks]
  __shared__ int rank_lens[kRankMax + 1];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int rg = lane >> 4;
  const int col = lane & 15;

  // units go request by request -- the longest history first when the batch is small
  // enough to rank here -- and within a request from its last chunk (the most visible
  // K/V) down: long units start first and short ones fill the tail.  The kv head is the
  // fastest index, so all chunks of one (request, kv head) land on the same XCD (and L2)
  // whenever the number of kv heads is a multiple of 8.
  int64_t unit = blockIdx.x;
  const int kvh = (int)(unit % a.num_kv_heads);
  unit /= a.num_kv_heads;
  const int chunks = (int)(gridDim.x / ((int64_t)a.num_kv_heads * a.num_reqs));
  const int c = chunks - 1 - (int)(unit % chunks);
  const int rank = (int)(unit / chunks);
  const int r = a.num_reqs <= kRankMax ? request_of_rank(a, rank, rank_lens) : rank;

  const int q0 = uniform_load(a.query_start_loc, r);
  const int q1 = uniform_load(a.query_start_loc, r + 1);
  if (q0 < 0 || q1 < q0 || (int64_t)q1 > a.total_q) return;  // no rows this request may write
  const int n = q1 - q0;
  const int L = uniform_load(a.seq_lens, r);
  const bool bad_len = L < n || (int64_t)L > (int64_t)a.max_blocks_per_seq * kTok;
  const int h0 = kvh * G;
  const float cs = a.scale_log2;
  const float lazy_raw = kLazyV / cs;
  constexpr bool alibi = ALIBI;
  const int32_t* table = a.block_tables + (int64_t)r * a.max_blocks_per_seq;
  const int64_t head_bytes = (int64_t)kvh * a.head_stride * 2;
  const char* kpool = static_cast<const char*>(a.k_pool) + head_bytes;
  const char* vpool = static_cast<const char*>(a.v_pool) + head_bytes;
  const int64_t block_bytes = a.block_stride * 2;
  const int tok_bytes = (int)(a.token_stride * 2);
  const uint32_t tile_bytes = (uint32_t)(kTok * tok_bytes);

  // this thread's chunks of a tile: linear index m = tid + j * kThreads over [K | V]
  int g_off[LPT];   // byte offset inside the tile of the chunk the thread loads
  int row_of[LPT];  // its token row
  const char* src[LPT];  // K or V pool (a wave's chunks are all K or all V)
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int m = tid + j * kThreads;
    const bool is_v = (w * kWave + j * kThreads) >= TCH;
    src[j] = is_v ? vpool : kpool;
    const int p = m % TCH;
    const int row = p / CPR;
    const int slot = p % CPR;
    row_of[j] = row;
    g_off[j] = row * tok_bytes + 16 * (slot ^ (is_v ? v_swizzle<CPR>(row) : k_swizzle<CPR>(row)));
  }
  // this lane's transposed V reads: row 4 rg + col / 4, dims 16 j + 4 (col % 4) .. + 3,
  // so that it receives dims 16 j + col of rows 4 rg .. 4 rg + 3 (the V^T operand)
  int v_rd[NT];
  {
    const int row = 4 * rg + (col >> 2);
    const int c4 = col & 3;
#pragma unroll
    for (int j = 0; j < NT; ++j) v_rd[j] = 16 * (TCH + row * CPR + ((2 * j + (c4 >> 1)) ^ v_swizzle<CPR>(row))) + 8 * (c4 & 1);
  }

  const uint32_t nb_lim = (uint32_t)min(a.num_blocks, (int64_t)0x7fffffff);
  // chunk c, then any chunks that a grid sized from an understated max_query_len left
  for (int cu = c; cu * QT < n; cu += chunks) {
    if (cu != c) lds_barrier();  // every wave is done with the previous chunk's tiles
    const int i0 = cu * QT;
    const int i_end = min(n, i0 + QT);
    const int vis_end = bad_len ? 0 : (a.causal ? L - n + i_end : L);
    const int ntile = (vis_end + kTok - 1) / kTok;
    bool bad = bad_len;

    // this wave's columns: w * WC + 16 q + col -> query token i0 + (w WC + 16 q + col) / G
    uint4 qb[NQ][KS];
    int lim[NQ], pos[NQ];
    float ab[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int cc = w * WC + 16 * q + col;
      const int ti = i0 + cc / G;
      const bool valid = ti < i_end;
      const int g = cc % G;
      pos[q] = L - n + ti;
      lim[q] = valid ? (a.causal ? pos[q] : L - 1) : -1;
      const int tq = valid ? ti : i_end - 1;
      const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((int64_t)(q0 + tq) * a.num_q_heads + h0 + g) * D +
                             8 * rg;
#pragma unroll
      for (int k = 0; k < KS; ++k)
        qb[q][k] = valid ? *reinterpret_cast<const uint4*>(qrow + 32 * k) : make_uint4(0, 0, 0, 0);
      ab[q] = 0.f;
      if (alibi) {
        float sl = 0.f;
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
          const float v = uniform_load(a.alibi_slopes, h0 + gg);
          sl = g == gg ? v : sl;
        }
        ab[q] = sl * kLog2e / cs;
      }
    }
    // tiles this wave needs scores for: up to its last column's limit
    const int w_first = i0 + w * WT;
    const int w_last_pos = w_first >= i_end ? -1 : (a.causal ? L - n + min(i_end, w_first + WT) - 1 : L - 1);
    const int w_tiles = bad_len || w_last_pos < 0 ? 0 : min(ntile, w_last_pos / kTok + 1);
    // the smallest limit over this wave's columns (-1 when some column is empty): a pair
    // wholly at or below it needs no mask
    const int w_min_lim = (w_first + WT - 1 < i_end) ? (a.causal ? L - n + w_first : L - 1) : -1;

    // per column: the exponent reference m_ref, the max that moves it (m_ref + slack) and
    // the offset -m_ref * cs (0 while nothing is visible), updated only when it moves
    float m_ref[NQ], thr[NQ], noff[NQ], lsum[NQ];
    f32x4_t acc[NQ][NT];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      m_ref[q] = -INFINITY;
      thr[q] = -INFINITY;
      noff[q] = 0.f;
      lsum[q] = 0.f;
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[q][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // block id of tile t (clamped into the unit's tiles); one outside the pool turns the
    // unit's rows to NaN and is replaced by block 0 (every thread sees the same ids)
    auto tile_id = [&](int t) -> int {
      const int id = uniform_load(table, min(t, ntile - 1));
      const bool out = (uint32_t)id >= nb_lim;  // negative ids too
      bad = bad || out;
      return out ? 0 : id;
    };
    // pairs of tiles: p covers tiles 2p (rows k = 8 rg + 0..3 of the P.V contraction) and
    // 2p + 1 (k = 8 rg + 4..7), so P.V runs on 16x16x32 matrix instructions
    const int npair = (ntile + 1) / 2;
    uint4 R[kPipe - 1][2][LPT];
#define VL_FETCH(DST, ID)                                                                             \
  do {                                                                                                \
    const int64_t boff_ = (int64_t)(ID) * block_bytes;                                                \
    _Pragma("unroll") for (int j = 0; j < LPT; ++j) {                                                 \
      const __amdgpu_buffer_rsrc_t r_ = tile_rsrc(src[j] + boff_, tile_bytes);                        \
      DST[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_, g_off[j], 0, 0));   \
    }                                                                                                 \
  } while (0)

    if (npair > 0) {
#pragma unroll
      for (int p = 0; p < kPipe - 1; ++p) {
        VL_FETCH(R[p][0], tile_id(2 * p));
        VL_FETCH(R[p][1], tile_id(2 * p + 1));
      }
      int ida_next = tile_id(2 * (kPipe - 1));
      int idb_next = tile_id(2 * (kPipe - 1) + 1);
      int p0 = 0;
      do {  // whole turns of kPipe - 1 pairs, the exit at the bottom (exact waits on R)
#pragma unroll
        for (int u = 0; u < kPipe - 1; ++u) {
          const int pr = p0 + u;  // may pass npair: then repeats of the last tile, never scored
          uint4(*st)[2 * TCH] = kvs[pr & 1];
          if ((2 * pr + 2) * kTok <= vis_end) {  // the whole pair is visible
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int j = 0; j < LPT; ++j) st[h][tid + j * kThreads] = R[u][h][j];
          } else {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int j = 0; j < LPT; ++j) {
                const uint32_t keep = (2 * pr + h) * kTok + row_of[j] < vis_end ? 0xffffffffu : 0u;
                const uint4 v = R[u][h][j];
                st[h][tid + j * kThreads] = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
              }
          }
          VL_FETCH(R[u][0], ida_next);
          VL_FETCH(R[u][1], idb_next);
          ida_next = tile_id(2 * (pr + kPipe));
          idb_next = tile_id(2 * (pr + kPipe) + 1);
          __builtin_amdgcn_sched_barrier(0);  // the prefetch stays ahead of this pair's work
          lds_barrier();
          if (2 * pr < w_tiles) {
            const int tA = 2 * pr * kTok + 4 * rg;  // token of this lane's row 0 in the first tile
            f32x4_t sc[2][NQ];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint4* Ks = st[h];
              uint4 kk[KS];
#pragma unroll
              for (int k = 0; k < KS; ++k) kk[k] = Ks[col * CPR + ((4 * k + rg) ^ (col & (CPR - 1)))];
#pragma unroll
              for (int q = 0; q < NQ; ++q) {
                f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < KS; ++k) c = mfma16<ST>(kk[k], qb[q][k], c);
                sc[h][q] = c;
              }
            }
            // score i of a lane: tile i / 4, row 4 rg + i % 4 -> token tA + (i < 4 ? i : 12 + i)
            float xs[NQ][8];
#pragma unroll
            for (int q = 0; q < NQ; ++q)
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                float v = sc[i >> 2][q][i & 3];
                if (alibi) v = fmaf(ab[q], (float)(tA + (i < 4 ? i : kTok + i - 4) - pos[q]), v);
                xs[q][i] = v;
              }
            if ((2 * pr + 2) * kTok - 1 > w_min_lim) {  // some score of the pair is masked (uniform)
#pragma unroll
              for (int q = 0; q < NQ; ++q)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                  xs[q][i] = tA + (i < 4 ? i : kTok + i - 4) <= lim[q] ? xs[q][i] : -INFINITY;
            }
            uint4 pb[NQ], pl[NQ];
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
              const float* x = xs[q];
              // NaN-propagating maximum (v_maximum3_f32): no quieting of each input, and a
              // NaN score ends in the output through its own exponential either way
              const float lm = __builtin_elementwise_maximum(
                  __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[0], x[1]), __builtin_elementwise_maximum(x[2], x[3])),
                  __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[4], x[5]), __builtin_elementwise_maximum(x[6], x[7])));
              if (__builtin_amdgcn_ballot_w64(lm > thr[q]) != 0) {
                float hm = fmaxf(lm, __shfl_xor(lm, 16));
                hm = fmaxf(hm, __shfl_xor(hm, 32));
                const bool mv = hm > thr[q];
                const float alpha = mv ? exp2_fast((m_ref[q] - hm) * cs) : 1.f;
                m_ref[q] = mv ? hm : m_ref[q];
                thr[q] = m_ref[q] + lazy_raw;
                noff[q] = m_ref[q] == -INFINITY ? 0.f : -m_ref[q] * cs;
                lsum[q] *= alpha;
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[q][j] *= alpha;
              }
              float pr8[8];
#pragma unroll
              for (int i = 0; i < 8; ++i) pr8[i] = exp2_fast(fmaf(x[i], cs, noff[q]));
              lsum[q] += ((pr8[0] + pr8[1]) + (pr8[2] + pr8[3])) + ((pr8[4] + pr8[5]) + (pr8[6] + pr8[7]));
              pb[q] = make_uint4(pack2<ST>(pr8[0], pr8[1]), pack2<ST>(pr8[2], pr8[3]), pack2<ST>(pr8[4], pr8[5]),
                                 pack2<ST>(pr8[6], pr8[7]));
              if constexpr (kSplitP<ST>)
                pl[q] = make_uint4(residual2(pb[q].x, pr8[0], pr8[1]), residual2(pb[q].y, pr8[2], pr8[3]),
                                   residual2(pb[q].z, pr8[4], pr8[5]), residual2(pb[q].w, pr8[6], pr8[7]));
            }
            // output tile j = dims 16 j .. 16 j + 15; its V^T operand (k = 8 rg + 0..3 from
            // the first tile, + 4..7 from the second) comes straight from LDS, transposed
            const lds_bytes sb = (lds_bytes)st[0];
#pragma unroll
            for (int j = 0; j < NT; ++j) {
              const uint2 lo = lds_read_tr16(sb + v_rd[j]);
              const uint2 hi = lds_read_tr16(sb + 2 * TCH * 16 + v_rd[j]);
              const uint4 va = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
              for (int q = 0; q < NQ; ++q) {
                acc[q][j] = mfma16<ST>(va, pb[q], acc[q][j]);
                if constexpr (kSplitP<ST>) acc[q][j] = mfma16<ST>(va, pl[q], acc[q][j]);
              }
            }
          }
        }
        p0 += kPipe - 1;
      } while (p0 < npair);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // retire the unconsumed prefetch
    }
#undef VL_FETCH

    // ---- this wave's columns: out = acc / sum (both relative to the same reference) -----
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float lw = lsum[q];
      lw += __shfl_xor(lw, 16);
      lw += __shfl_xor(lw, 32);
      const int cc = w * WC + 16 * q + col;
      const int ti = i0 + cc / G;
      if (ti < i_end) {
        const float inv = lw > 0.f ? 1.f / lw : 0.f;
        const int64_t row = (int64_t)(q0 + ti) * a.num_q_heads + h0 + cc % G;
        uint16_t* orow = static_cast<uint16_t*>(a.out) + row * D;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          // dims 16 j + 4 rg + i, i < 4: contiguous
          float x[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = bad ? NAN : acc[q][j][i] * inv;
          *reinterpret_cast<uint2*>(orow + 16 * j + 4 * rg) =
              make_uint2(to_storage<ST>(x[0]) | (to_storage<ST>(x[1]) << 16), to_storage<ST>(x[2]) | (to_storage<ST>(x[3]) << 16));
        }
      }
    }
  }
}

template <class ST, int D, int G>
hipError_t launch_lds_g(const VarlenArgs& a, hipStream_t stream) {
  constexpr int QT = kWaves * 32 / G;
  const int64_t chunks = a.max_query_len <= 0 ? 1 : (a.max_query_len + QT - 1) / QT;
  const int64_t grid = (int64_t)a.num_kv_heads * a.num_reqs * chunks;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (a.alibi_slopes)
    hipLaunchKernelGGL((varlen_lds_kernel<ST, D, G, true>), dim3((unsigned)grid), dim3(kWaves * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((varlen_lds_kernel<ST, D, G, false>), dim3((unsigned)grid), dim3(kWaves * kWave), 0, stream, a);
  return hipGetLastError();
}

template <class ST, int D, int G>
hipError_t launch_g(const VarlenArgs& a, hipStream_t stream) {
  // many columns per request: the LDS-sharing kernel; a few (speculative decode): the
  // kernel that splits each request's K/V over the waves
  if ((int64_t)a.max_query_len * G > 32) return launch_lds_g<ST, D, G>(a, stream);
  constexpr int NQ = 2;
  constexpr int QT = 16 * NQ / G;
  const int64_t chunks = a.max_query_len <= 0 ? 1 : (a.max_query_len + QT - 1) / QT;
  const int64_t grid = (int64_t)a.num_kv_heads * a.num_reqs * chunks;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (a.alibi_slopes)
    hipLaunchKernelGGL((varlen_kernel<ST, D, G, NQ, true>), dim3((unsigned)grid), dim3(kWaves * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((varlen_kernel<ST, D, G, NQ, false>), dim3((unsigned)grid), dim3(kWaves * kWave), 0, stream, a);
  return hipGetLastError();
}

template <class ST, int D>
hipError_t launch_d(const VarlenArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<ST, D, 1>(a, stream);
    case 2: return launch_g<ST, D, 2>(a, stream);
    case 4: return launch_g<ST, D, 4>(a, stream);
    case 8: return launch_g<ST, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class ST>
hipError_t launch_st(const VarlenArgs& a, int head_size, hipStream_t stream) {
  switch (head_size) {
    case 64: return launch_d<ST, 64>(a, stream);
    case 128: return launch_d<ST, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

#ifndef PCACHE_VARLEN_DECODE_MT
#define PCACHE_VARLEN_DECODE_MT 1
#endif

hipError_t launch_varlen(const VarlenArgs& a, int dtype, int head_size, hipStream_t stream) {
  // up to 16 (query token, head) columns per request and kv head (speculative decode):
  // the one-pass decode's persistent, longest-first unit scheme with one 16-column tile
  if (PCACHE_VARLEN_DECODE_MT && a.num_kv_heads > 0 && a.max_query_len > 0 &&
      (int64_t)a.max_query_len * (a.num_q_heads / a.num_kv_heads) <= 16)
    return launch_decode_multitoken(a, dtype, head_size, stream);
  switch (dtype) {
    case 1: return launch_st<F16>(a, head_size, stream);
    case 2: return launch_st<BF16>(a, head_size, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pcache
