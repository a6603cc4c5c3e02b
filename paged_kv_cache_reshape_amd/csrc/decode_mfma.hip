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
//   Lane l receives the scores of tokens 4*(l/16) + i (i < 4) for head l % 16.
// * Online softmax per query head with a lazy reference: the exponent reference
//   m_ref of a head moves only when a block's max exceeds it by more than 2^8
//   (log2 domain), so most blocks skip the accumulator rescale entirely (a
//   wave-uniform branch); the true running max is tracked alongside and the final
//   state is expressed relative to it.
// * P.V on the matrix cores too, as out^T = V^T . P^T in 16x16 tiles with
//   v_mfma_f32_16x16x16_{bf16,f16}: the B operand P^T (16 tokens x 16 heads) is the
//   score tile's own register layout after the exponential (lane l holds tokens
//   4*(l/16) .. +3 of head l % 16), rounded to the storage type, so probabilities
//   never move between lanes.  For bf16 a second product adds the part of each
//   probability that rounding drops (kSplitP).  The A operand of tile j holds dims
//   (D/16)*m + j (m < 16) of the same four tokens: lane (r, c) loads 16 (head_size
//   128) or 8 (64) contiguous bytes of each of its four V rows (dims (D/16)*c ..)
//   and picks element j of each with v_perm_b32.  Lane (r, c) accumulates, for
//   head c, dims (D/16)*(4r + i) + j (i < 4, j < D/16): D/4 fp32 registers, no
//   cross-lane reduction.
// * Loads are buffer loads whose base is the block's tile, formed in scalar
//   registers from the block id; the per-lane offsets are loop constants.  A ring
//   of STAGES register sets keeps the next STAGES-1 blocks in flight while one is
//   consumed.  The ring loop has wave-uniform control flow, issues every load
//   unconditionally and exits only at its bottom, so the compiler waits for exactly
//   the ring stage being consumed; the steps past the wave's last block load through
//   a buffer resource of extent 0, which returns zeros without touching memory.
// * A unit's block ids are staged in LDS by the whole workgroup, which checks them
//   against the pool once; each wave reads its ids from there one block ahead.
//
// 8-bit (OCP E4M3) pools ("Inside vLLM CUDA Kernels", Part 2, "Why Layout and
// Quantization Scale Produce Two Copy Paths": the stored code times the kv head's
// scale stands for the value): the ring holds the raw codes -- half the bytes in
// flight per block -- and each block is widened to the query's 16-bit type just
// before the same two MFMA stages.  Every E4M3 value is exact in bf16 and fp16, so
// the widening (v_cvt_scalef32_pk_{bf16,f16}_fp8 with scale 1) loses nothing; the
// head's k_scale is folded into the score scale and v_scale multiplies the final
// output.  The q.k contraction runs over the dims in a permuted order (the same for
// K and q, so the dot product is unchanged): k-step k of lane row group rg covers
// dims rg*(D/4) + 8k .. +8, which makes each lane's K bytes one contiguous run.
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
#include "mfma_common.h"

namespace pcache {
namespace {

constexpr int kBlockTokens = 16;  // tokens per score tile (the MFMA's 16 rows); pool blocks hold BS
constexpr int kPartition = 512;
constexpr float kLazy = 8.f;            // log2-domain slack before the exponent reference moves
constexpr int kMaxRankedSeqs = 512;     // sequences ranked by length in-kernel (beyond: index order)

// One-pass workgroup at head size 128: one per CU, as many waves as the register
// allocation lets a CU hold (3 per SIMD), so the persistent grid fills the chip with one
// workgroup per CU and the units dealt to it share its waves.  At head size 64 a unit
// carries half the bytes per token, and a 16-wave workgroup spent a large share of each
// unit in its fixed costs (id staging, first loads, merge) with every wave of the CU
// waiting at them together; two 8-wave workgroups per CU (4 waves per SIMD) overlap one
// unit's fixed costs with the other's stream: the combined-block workload (128
// sequences of 1..2048 tokens) ran 12% faster than with 16 waves (4 waves, four
// workgroups per CU: 8% slower than 16).
#ifndef PCACHE_ONEPASS_WAVES_D128
#define PCACHE_ONEPASS_WAVES_D128 12
#endif
#ifndef PCACHE_ONEPASS_WAVES_D64
#define PCACHE_ONEPASS_WAVES_D64 8
#endif
#ifndef PCACHE_ONEPASS_OCC_D64
#define PCACHE_ONEPASS_OCC_D64 4
#endif
// The 8-bit pool at head size 128 has its own wave count: 8 waves (2 per SIMD) ran the
// one-pass decode 3% faster than 12 (measured with the non-temporal V loads below);
// deeper rings on the 8 waves (3 or 4 stages) lost that gain again.
#ifndef PCACHE_ONEPASS_WAVES_D128_KV8
#define PCACHE_ONEPASS_WAVES_D128_KV8 8
#endif
#ifndef PCACHE_ONEPASS_OCC_KV8
#define PCACHE_ONEPASS_OCC_KV8 2
#endif
// several query tokens per sequence (16 score columns) at head size 128: 8 waves ran
// the speculative-decode workload 5% faster than 12 (the merge of 16 columns per wave
// through LDS shrinks with the wave count; 4 waves: no gain)
#ifndef PCACHE_ONEPASS_WAVES_D128_MT
#define PCACHE_ONEPASS_WAVES_D128_MT 8
#endif
#ifndef PCACHE_ONEPASS_OCC_MT
#define PCACHE_ONEPASS_OCC_MT PCACHE_ONEPASS_OCC
#endif
template <int D, bool KV8 = false, bool MT = false>
constexpr int onepass_waves() {
  return D == 64 ? PCACHE_ONEPASS_WAVES_D64
                 : KV8 ? PCACHE_ONEPASS_WAVES_D128_KV8 : MT ? PCACHE_ONEPASS_WAVES_D128_MT : PCACHE_ONEPASS_WAVES_D128;
}
#ifndef PCACHE_ONEPASS_STAGES
#define PCACHE_ONEPASS_STAGES 2
#endif
#ifndef PCACHE_ONEPASS_TABLE
#define PCACHE_ONEPASS_TABLE 1024  // block ids staged in LDS at once (16384 tokens)
#endif
#ifndef PCACHE_SPLIT_WAVES
#define PCACHE_SPLIT_WAVES 4
#endif
// the 8-bit pool's split workgroups: 2 waves ran workload 3 2% faster than 4 (3 and 8
// waves: 8-11% slower), measured with the non-temporal V loads
#ifndef PCACHE_SPLIT_WAVES_KV8
#define PCACHE_SPLIT_WAVES_KV8 2
#endif
// one query head per kv head (MHA), 16-bit pools: 2 waves ran the mixed-serving workload
// (256 sequences of 16-8192 tokens, most partitions short) 2-3% faster than 4
#ifndef PCACHE_SPLIT_WAVES_MHA
#define PCACHE_SPLIT_WAVES_MHA 2
#endif
template <bool KV8, int G>
constexpr int split_waves() {
  return KV8 ? PCACHE_SPLIT_WAVES_KV8 : (G == 1 ? PCACHE_SPLIT_WAVES_MHA : PCACHE_SPLIT_WAVES);
}
// waves per SIMD the register allocation must allow (the kernels fit 3 without spills)
#ifndef PCACHE_SPLIT_OCC
#define PCACHE_SPLIT_OCC 3
#endif
#ifndef PCACHE_ONEPASS_OCC
#define PCACHE_ONEPASS_OCC 3
#endif
#ifndef PCACHE_SPLIT_STAGES
#define PCACHE_SPLIT_STAGES 2
#endif
// 8-bit pools: a block is half the bytes, so more blocks go in flight per wave
#ifndef PCACHE_ONEPASS_STAGES_KV8
#define PCACHE_ONEPASS_STAGES_KV8 2
#endif
#ifndef PCACHE_SPLIT_STAGES_KV8
#define PCACHE_SPLIT_STAGES_KV8 2
#endif
// Cache-policy operand of the K and V tile loads (each tile is read once per step).  The
// V loads carry the non-temporal hint (nt, 2): measured 2% faster one-pass and 6% faster
// split decode on the 16-bit cache, 2-4% on the 8-bit one; the same hint on the K loads
// made both paths slower (3-7%), alone or together with V.
#ifndef PCACHE_K_CPOL
#define PCACHE_K_CPOL 0
#endif
#ifndef PCACHE_V_CPOL
#define PCACHE_V_CPOL 2
#endif

template <int NW, int D, int NC, int TABLE>
struct UnitLds {
  __align__(16) float acc[NW][NC][D];  // each wave's scaled accumulator, per score column
  float mw[NW][NC];
  float lw[NW][NC];
  int ids[TABLE];  // block ids of the unit's current chunk
  int bad;         // some id of the unit lies outside the pool
};


// One unit: kv head `kvh` of sequence `s`, tokens [t_begin, t_end).  All waves of
// the workgroup call it together (it uses block-wide barriers).  Writes out (one
// pass) or the partition's partials (split).  KV8: the pool holds E4M3 codes.
// Score columns: NC = G is the decode (column c = query head h0 + c of the sequence's
// one token).  NC = 16 > G takes several query tokens per sequence (query_start_loc):
// column c = token tok0 + c / G, head h0 + c % G, each with its own causal limit; the
// call covers tokens tok0 .. tok0 + 16/G - 1 and returns whether more remain.
// PFX: a common-prefix unit (split path, NC = 16): column c is query head h0 + c % G of
// sequence s * (16 / G) + c / G (`s` numbers the unit's group of sequences), and the
// unit reads partition `part` of the prefix blocks a.prefix_table once for all of them.
// A column is written when its sequence's shared tokens cover the partition completely;
// NaN when its table does not hold the prefix blocks there (or its length is invalid).
template <class ST, int D, int G, int NW, int STAGES, int TABLE, bool SPLIT, bool KV8, int BS, int NC = G,
          bool FUSED = false, bool PFX = false>
__device__ __forceinline__ bool decode_unit(const DecodeArgs& a, UnitLds<NW, D, NC, TABLE>& sm, int s, int kvh,
                                            int part, int tok0 = 0) {
  static_assert(ST::kBytes == 2, "16-bit storage only");
  static_assert(D == 64 || D == 128, "head size 64 or 128");
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group of 1, 2, 4 or 8 query heads");
  static_assert(STAGES >= 2 && STAGES <= 4, "prefetch ring of 2..4 register sets");
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size 8, 16 or 32");
  constexpr bool MC = NC != G;       // several score columns per unit
  constexpr bool MT = MC && !PFX;    // several query tokens per sequence
  static_assert(NC == G || (NC == 16 && !KV8 && (PFX ? SPLIT && !FUSED && BS == 16 : !SPLIT)),
                "multi-token units: one pass, 16-bit pools; common-prefix units: split, 16-token blocks");
  // tiles per staged chunk: the chunk's block ids must fit the TABLE entries
  constexpr int CT = BS >= 16 ? TABLE * (BS / 16) : TABLE / (16 / BS);
  static_assert(!SPLIT || CT >= kPartition / kBlockTokens, "a partition's ids fit the table");
  constexpr int KS = D / 32;   // q.k MFMA k-steps per block
  constexpr int DPL = D / 16;  // V dims a lane loads per row = out^T tiles per block
  constexpr int NT = DPL;
  constexpr int kThreads = NW * kWave;
  using VRow = typename VRowOf<DPL>::type;
  using VRow8 = typename VRow8Of<DPL>::type;
  constexpr int EB = KV8 ? 1 : 2;  // pool bytes per element
  constexpr int K8 = KS / 2;        // 16-byte K loads per block and lane (8-bit pool)
  constexpr int kKCpol = PCACHE_K_CPOL;
  constexpr int kVCpol = PCACHE_V_CPOL;
  // kv head pairs (a.pair): 16-bit pools, one query token, head size 128 = two heads of 64
  constexpr bool PAIRABLE = !KV8 && !MC && !FUSED && D == 128 && G >= 2;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int rg = lane >> 4;   // row group of the score tile: tokens 4*rg .. 4*rg+3
  const int col = lane & 15;  // score column: query head of the group

  // a common-prefix unit covers its whole partition
  const int L = PFX ? (part + 1) * kPartition : uniform_load(a.seq_lens, s);
  // PFX: this lane's column: sequence pcs of length pcL; pc_out = the column's
  // (sequence, head, partition) partial is written here, pc_on = it is computed (else NaN)
  int pcs = 0, pcL = 0;
  bool pc_out = false, pc_on = false;
  if constexpr (PFX) {
    pcs = s * (NC / G) + col / G;
    const bool in = pcs < a.num_seqs;
    const int sl = in ? a.shared_lens[pcs] : 0;
    pcL = in ? a.seq_lens[pcs] : 0;
    pc_out = in && sl >= (part + 1) * kPartition;
    bool ok = pc_out && sl <= pcL && sl <= a.prefix_blocks * BS &&
              (int64_t)pcL <= (int64_t)a.max_partitions * kPartition && (int64_t)pcL <= (int64_t)a.max_blocks_per_seq * BS;
    // the column's table holds the prefix blocks over this partition: the four lanes of
    // a column check 8 of its 32 entries each
    const int e0 = part * (kPartition / BS) + 8 * rg;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      ok = ok && a.block_tables[(int64_t)pcs * a.max_blocks_per_seq + e0 + i] == a.prefix_table[e0 + i];
    int okv = ok ? 1 : 0;
    okv &= __shfl_xor(okv, 16);
    okv &= __shfl_xor(okv, 32);
    pc_on = okv != 0;
  }
  // the sequence's query rows: q0 .. q0 + n - 1 (the decode: row s alone)
  int q0 = s, n = 1;
  if constexpr (MT) {
    q0 = uniform_load(a.query_start_loc, s);
    const int q1 = uniform_load(a.query_start_loc, s + 1);
    if (q0 < 0 || q1 < q0 || (int64_t)q1 > a.total_q) return false;  // no rows this sequence may write
    n = q1 - q0;
    if (tok0 >= n) return false;
  }
  constexpr int TPC = NC / G;                      // query tokens per call
  const int C = MT ? min(n - tok0, TPC) * G : NC;  // score columns in use
  const int ci = MT ? tok0 + col / G : 0;          // this lane's query token
  // the column's own position (the ALiBi origin) and last visible position
  const int qpos = MT ? L - n + ci : (PFX ? pcL - 1 : L - 1);
  const int lim = (MT && !a.causal) ? L - 1 : qpos;
  const int min_lim = (MT && a.causal) ? L - n + tok0 : L - 1;  // smallest over the call's columns
  // 8-bit pool: the kv head's dequantisation scales (k_scale folded into the score scale)
  const float ksc = KV8 ? uniform_load(a.k_scale, (int64_t)kvh * a.scale_stride) : 1.f;
  const float vsc = KV8 ? uniform_load(a.v_scale, (int64_t)kvh * a.scale_stride) : 1.f;
  const float cs_raw = a.scale_log2 * ksc;
  const bool bad_scale = KV8 && !(cs_raw >= 0x1p-120f && cs_raw <= 0x1p120f && vsc > 0.f && vsc <= 3.4e38f);
  bool bad = !PFX && (L < 0 || (int64_t)L > (int64_t)a.max_blocks_per_seq * BS ||
                      (SPLIT && (int64_t)L > (int64_t)a.max_partitions * kPartition) || bad_scale || (MT && L < n));
  const int t_begin = SPLIT ? part * kPartition : 0;
  const int t_end = bad ? t_begin : (SPLIT ? min(L, t_begin + kPartition) : L);
  const int b_begin = t_begin / kBlockTokens;
  const int b_end = (t_end + kBlockTokens - 1) / kBlockTokens;
  const int h0 = kvh * G;
  const float cs = bad_scale ? 1.f : cs_raw;  // > 0 (scale validated on the host, k_scale here)
  const int32_t* table = PFX ? a.prefix_table : a.block_tables + (int64_t)s * a.max_blocks_per_seq;

  // B operand: column `col` (zero for col >= C), dims 32*k + 8*rg .. +8 (16-bit
  // pool) or rg*(D/4) + 8*k .. +8 (8-bit pool, the order its K rows are read in)
  uint4 qb[KS];
  if (PAIRABLE && a.pair) {
    // kv head pair: column c belongs to kv head 2p + (c >= G/2), whose 64 dims are dims
    // 64*(c >= G/2) .. +64 of the pair's 128-element row; its q fills its own half of the
    // contraction and zeros the other, so one tile scores both heads
    const int qc = col < C ? col : C - 1;
    const int hi = qc >= G / 2;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((int64_t)s * a.num_q_heads + h0 + qc) * (D / 2) + 8 * rg;
#pragma unroll
    for (int k = 0; k < KS; ++k)
      qb[k] = (col < C && (k >= KS / 2) == (bool)hi) ? *reinterpret_cast<const uint4*>(qrow + 32 * (k % (KS / 2)))
                                                      : make_uint4(0, 0, 0, 0);
  } else {
    // keep the address inside q for the zero columns
    const int qc = col < C ? col : C - 1;
    const int64_t qr = MT ? (int64_t)(q0 + tok0 + qc / G) : (PFX ? (int64_t)pcs : (int64_t)s);
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (qr * a.num_q_heads + h0 + (qc & (G - 1))) * D +
                           (KV8 ? rg * (D / 4) : 8 * rg);
#pragma unroll
    for (int k = 0; k < KS; ++k)
      qb[k] = (PFX ? pc_on : col < C) ? *reinterpret_cast<const uint4*>(qrow + (KV8 ? 8 : 32) * k)
                                       : make_uint4(0, 0, 0, 0);
  }

  // softmax state of head `col` (meaningful for col < G): the four row-group lanes
  // of a head share m_ref; m_true and the sum cover the lane's own tokens
  float m_ref = -INFINITY, m_true = -INFINITY, lsum = 0.f;
  f32x4_t acc[NT];  // out^T tiles: acc[j][i] = head col, dim DPL*(4*rg + i) + j
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t head_bytes = (int64_t)kvh * a.head_stride * EB;
  const char* kpool = static_cast<const char*>(a.k_pool) + head_bytes;
  const char* vpool = static_cast<const char*>(a.v_pool) + head_bytes;
  const int64_t block_bytes = a.block_stride * EB;
  const int tok_bytes = (int)(a.token_stride * EB);                  // 16 * tok_bytes < 2^31 (validated on the host)
  const uint32_t tile_bytes = (uint32_t)(kBlockTokens * tok_bytes);  // extent of one tile's rows
  // 16-bit: + 64*k per MFMA step; 8-bit: the lane's D/4 contiguous codes, 16 bytes per load
  const int k_off = col * tok_bytes + (KV8 ? rg * (D / 4) : 16 * rg);
  const int v_off = 4 * rg * tok_bytes + col * (EB * DPL);  // + e*tok_bytes for row 4*rg + e
  // 8-token blocks: a tile's rows 0-7 lie in one block, 8-15 in the next; a lane's K row
  // (token col) and V rows (4*rg .. +3) sit at these offsets inside their block
  const int k_off8 = (col & 7) * tok_bytes + (KV8 ? rg * (D / 4) : 16 * rg);
  const int v_off8 = 4 * (rg & 1) * tok_bytes + col * (EB * DPL);
  const int nblk = (t_end + BS - 1) / BS;  // blocks holding the unit's tokens (from block 0)
  const float lazy_raw = kLazy / cs;
  // ALiBi: the bias of head `col` in raw q.k units (times cs it is slope * log2 e per
  // token).  The slope is loaded here and converted after the first K/V loads are out.
  const bool alibi = a.alibi_slopes != nullptr;
  float slope = 0.f;
  if (alibi) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sg = uniform_load(a.alibi_slopes, h0 + g);
      slope = (col & (G - 1)) == g ? sg : slope;
    }
  }
  float ab = 0.f;
  const int last_pos = qpos;  // the bias is zero at the column's own position

  uint4 kb[STAGES][KS];  // 16-bit pool ring
  VRow vb[STAGES][4];
  uint4 kq[STAGES][K8];  // 8-bit pool ring (raw codes)
  VRow8 vq[STAGES][4];

  // K/V of tile (A, B) into ring slot ST.  16-token blocks: block A.  32: rows 16*B ..
  // of block A.  8: rows 0-7 from block A, 8-15 from block B (each lane addresses its own
  // block, so these are global loads with 64-bit lane addresses).  EXT is the extent of the
  // tile's buffer resources: tile_bytes, or 0 for a ring step that only keeps the load
  // count static (past the wave's last tile): a buffer load past its extent returns zeros
  // without a memory access, so such a step costs no HBM traffic (16- and 32-token blocks).
#define PC_LOAD(ST, A, B, EXT)                                                                       \
  do {                                                                                               \
    if constexpr (BS == 8) {                                                                         \
      const int64_t ka_ = (int64_t)((col < 8) ? (A) : (B)) * block_bytes + k_off8;                   \
      const int64_t va_ = (int64_t)((rg < 2) ? (A) : (B)) * block_bytes + v_off8;                   \
      if constexpr (KV8) {                                                                           \
        _Pragma("unroll") for (int k = 0; k < K8; ++k) kq[ST][k] =                                  \
            *reinterpret_cast<const uint4*>(kpool + ka_ + 16 * k);                                   \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) vq[ST][e] =                                   \
            *reinterpret_cast<const VRow8*>(vpool + va_ + (int64_t)e * tok_bytes);                   \
      } else {                                                                                       \
        _Pragma("unroll") for (int k = 0; k < KS; ++k) kb[ST][k] =                                  \
            *reinterpret_cast<const uint4*>(kpool + ka_ + 64 * k);                                   \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) vb[ST][e] =                                   \
            *reinterpret_cast<const VRow*>(vpool + va_ + (int64_t)e * tok_bytes);                    \
      }                                                                                              \
    } else {                                                                                         \
      const int64_t boff_ = (int64_t)(A) * block_bytes + (BS == 32 ? (int64_t)(B) * tile_bytes : 0); \
      const __amdgpu_buffer_rsrc_t kr_ = tile_rsrc(kpool + boff_, (EXT));                            \
      const __amdgpu_buffer_rsrc_t vr_ = tile_rsrc(vpool + boff_, (EXT));                            \
      if constexpr (KV8) {                                                                           \
        _Pragma("unroll") for (int k = 0; k < K8; ++k) kq[ST][k] =                                  \
            __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr_, k_off + 16 * k, 0, kKCpol)); \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                             \
          if constexpr (DPL == 8)                                                                    \
            vq[ST][e] = __builtin_bit_cast(VRow8, __builtin_amdgcn_raw_buffer_load_b64(vr_, v_off, e * tok_bytes, kVCpol)); \
          else                                                                                       \
            vq[ST][e] = __builtin_bit_cast(VRow8, __builtin_amdgcn_raw_buffer_load_b32(vr_, v_off, e * tok_bytes, kVCpol)); \
        }                                                                                            \
      } else {                                                                                       \
        _Pragma("unroll") for (int k = 0; k < KS; ++k) kb[ST][k] =                                  \
            __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr_, k_off + 64 * k, 0, kKCpol)); \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                             \
          if constexpr (DPL == 8)                                                                    \
            vb[ST][e] = __builtin_bit_cast(VRow, __builtin_amdgcn_raw_buffer_load_b128(vr_, v_off, e * tok_bytes, kVCpol)); \
          else                                                                                       \
            vb[ST][e] = __builtin_bit_cast(VRow, __builtin_amdgcn_raw_buffer_load_b64(vr_, v_off, e * tok_bytes, kVCpol)); \
        }                                                                                            \
      }                                                                                              \
    }                                                                                                \
  } while (0)

  // consume the block in ring slot SL whose first token is TOK0
#define PC_BLOCK(SL, TOK0)                                                                           \
  do {                                                                                               \
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};                                                                \
    if constexpr (KV8) {                                                                             \
      /* each k-step's 8 codes widened to the query's type just before its MFMA */                   \
      _Pragma("unroll") for (int k = 0; k < KS; ++k) {                                              \
        const uint4 r_ = kq[SL][k >> 1];                                                             \
        const uint2 lo_ = widen4<ST>((k & 1) ? r_.z : r_.x), hi_ = widen4<ST>((k & 1) ? r_.w : r_.y); \
        c = mfma16<ST>(make_uint4(lo_.x, lo_.y, hi_.x, hi_.y), qb[k], c);                           \
      }                                                                                              \
    } else {                                                                                         \
      _Pragma("unroll") for (int k = 0; k < KS; ++k) c = mfma16<ST>(kb[SL][k], qb[k], c);           \
    }                                                                                                \
    if (alibi) {                                                                                     \
      /* signed distance of token 4*rg + e to the newest position, times the slope */                \
      const int d0_ = (TOK0) + 4 * rg - last_pos;                                                    \
      _Pragma("unroll") for (int e = 0; e < 4; ++e) c[e] = fmaf(ab, (float)(d0_ + e), c[e]);        \
    }                                                                                                \
    const int visible = t_end - (TOK0);                                                              \
    if (visible < kBlockTokens || (MT && (TOK0) + kBlockTokens - 1 > min_lim)) {                     \
      _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                               \
        const bool keep = 4 * rg + e < visible;                                                      \
        const bool seen = !MT || (TOK0) + 4 * rg + e <= lim; /* the column's causal limit */         \
        c[e] = keep && seen ? c[e] : -INFINITY;                                                      \
        if constexpr (KV8)                                                                           \
          vq[SL][e] = keep ? vq[SL][e] : VRow8{};                                                    \
        else                                                                                         \
          vb[SL][e] = keep ? vb[SL][e] : VRow{};                                                     \
      }                                                                                              \
    }                                                                                                \
    const float lm = fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3]));                                    \
    m_true = fmaxf(m_true, lm);                                                                      \
    if (__builtin_amdgcn_ballot_w64(col < C && lm > m_ref + lazy_raw) != 0) {                        \
      float hm = fmaxf(lm, __shfl_xor(lm, 16));                                                      \
      hm = fmaxf(hm, __shfl_xor(hm, 32));                                                            \
      const bool mv = hm > m_ref + lazy_raw;                                                         \
      const float alpha = mv ? exp2_fast((m_ref - hm) * cs) : 1.f;                                   \
      m_ref = mv ? hm : m_ref;                                                                       \
      lsum *= alpha;                                                                                 \
      _Pragma("unroll") for (int j = 0; j < NT; ++j) acc[j] *= alpha;                               \
    }                                                                                                \
    const float ref = m_ref == -INFINITY ? 0.f : m_ref * cs;                                         \
    float pr[4];                                                                                     \
    _Pragma("unroll") for (int e = 0; e < 4; ++e) pr[e] = exp2_fast(fmaf(c[e], cs, -ref));          \
    lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);                                                       \
    const uint2 pb = make_uint2(pack2<ST>(pr[0], pr[1]), pack2<ST>(pr[2], pr[3]));                   \
    /* bf16: the probabilities' rounding residuals, a second P^T operand */                          \
    const uint2 pl = kSplitP<ST> ? make_uint2(residual2(pb.x, pr[0], pr[1]), residual2(pb.y, pr[2], pr[3])) \
                                 : make_uint2(0u, 0u);                                               \
    if constexpr (KV8) {                                                                             \
      /* tiles j, j+1 (j even): bytes j, j+1 of the four rows gathered pairwise into two */         \
      /* dwords of codes, each widened into one operand dword of either tile */                      \
      _Pragma("unroll") for (int j = 0; j < NT; j += 2) {                                           \
        const uint32_t sel = (j & 2) ? 0x07030602u : 0x05010400u;                                    \
        const uint32_t x_ = __builtin_amdgcn_perm(vword(vq[SL][1], j >> 2), vword(vq[SL][0], j >> 2), sel); \
        const uint32_t y_ = __builtin_amdgcn_perm(vword(vq[SL][3], j >> 2), vword(vq[SL][2], j >> 2), sel); \
        const uint2 xw_ = widen4<ST>(x_), yw_ = widen4<ST>(y_);                                      \
        acc[j] = mfma_pv<ST>(make_uint2(xw_.x, yw_.x), pb, acc[j]);                                  \
        acc[j + 1] = mfma_pv<ST>(make_uint2(xw_.y, yw_.y), pb, acc[j + 1]);                          \
        if constexpr (kSplitP<ST>) {                                                                 \
          acc[j] = mfma_pv<ST>(make_uint2(xw_.x, yw_.x), pl, acc[j]);                                \
          acc[j + 1] = mfma_pv<ST>(make_uint2(xw_.y, yw_.y), pl, acc[j + 1]);                        \
        }                                                                                            \
      }                                                                                              \
    } else {                                                                                         \
      _Pragma("unroll") for (int j = 0; j < NT; ++j) {                                              \
        /* element j of each of the four rows: tokens 4*rg .. 4*rg+3 at dim DPL*col + j */           \
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;                                    \
        const uint2 va = make_uint2(__builtin_amdgcn_perm(vword(vb[SL][1], j >> 1), vword(vb[SL][0], j >> 1), sel), \
                                    __builtin_amdgcn_perm(vword(vb[SL][3], j >> 1), vword(vb[SL][2], j >> 1), sel)); \
        acc[j] = mfma_pv<ST>(va, pb, acc[j]);                                                        \
        if constexpr (kSplitP<ST>) acc[j] = mfma_pv<ST>(va, pl, acc[j]);                             \
      }                                                                                              \
    }                                                                                                \
  } while (0)

  // ---- the unit's blocks, TABLE ids at a time -----------------------------------------
  // the previous unit read sm.bad before its merge barrier, so it can be cleared here
  // The step's own K/V write, fused (16-bit pools, one token per sequence): token s is
  // sequence s's newest token, and the unit whose tokens include position L - 1 stores
  // its row for this kv head.  Wave 0 does it: the row (16 bytes per lane, lanes
  // < 2*D/8) is read, the slot checked against the table, the row stored and the stores
  // waited for, before a workgroup barrier that precedes every read of the tile holding
  // L - 1.  That is the chunk's staging barrier below (wave 0 writes while the other
  // waves issue their early first-tile loads), or, when that tile is itself one of the
  // early first tiles (a unit of fewer than NW tiles), the barrier just below.  A slot
  // inside the pool that is not position L - 1 of sequence s makes the step invalid for
  // s: nothing is written and sm.bad turns its outputs to NaN; a slot outside the pool
  // (padding) writes nothing, as in the plain write.
  static_assert(!FUSED || (!MT && !KV8), "the fused write: one token per sequence, 16-bit pools");
  const bool fused = FUSED && !bad && L >= 1;
  const bool fused_early = fused && (L - 1) / kBlockTokens - b_begin < NW;
  auto fused_write = [&]() __attribute__((always_inline)) {
    const bool owner = !SPLIT || part == (L - 1) / kPartition;
    const bool isv = lane >= D / 8;
    const int piece = isv ? lane - D / 8 : lane;
    uint4 row = make_uint4(0, 0, 0, 0);
    if (owner && lane < 2 * (D / 8))
      row = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(isv ? a.step_value : a.step_key) +
                                            (int64_t)s * (isv ? a.step_value_stride : a.step_key_stride) +
                                            (int64_t)kvh * D + 8 * piece);
    const int64_t slot = uniform_load(a.step_slots, s);
    if (slot >= 0 && slot < a.num_blocks * BS) {
      const int id = uniform_load(table, (L - 1) / BS);
      if ((int64_t)id * BS + (L - 1) % BS != slot) {
        if (lane == 0) sm.bad = 1;
      } else if (owner) {
        if (lane < 2 * (D / 8)) {
          const int64_t blk = slot / BS;
          const int64_t dst = blk * a.block_stride + (slot - blk * BS) * a.token_stride +
                              (int64_t)kvh * a.head_stride + 8 * piece;
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(const_cast<void*>(isv ? a.v_pool : a.k_pool)) + dst) = row;
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the stores are complete
      }
    }
  };

  // the previous unit read sm.bad before its merge barrier, so it can be cleared here
  if (tid == 0) sm.bad = 0;
  if constexpr (FUSED) {
    if (fused_early && w == 0) fused_write();
    global_barrier();  // the previous unit's readers of sm are done; the row store is visible
  } else {
    lds_barrier();  // the previous unit's readers of sm are done
  }
  if constexpr (FUSED) {
    if (fused && !fused_early && w == 0) fused_write();
  }
  for (int cb = b_begin; cb < b_end; cb += CT) {
    const int cn = min(CT, b_end - cb);  // tiles in this chunk
    if (cb != b_begin) __syncthreads();  // every wave has read the previous chunk's ids
    // the chunk's block ids: blocks [blk0, blk0 + nb) (chunk starts are even tiles)
    const int blk0 = BS >= 16 ? cb / (BS / 16) : cb * (16 / BS);
    const int nb = BS >= 16 ? (cb + cn - 1) / (BS / 16) - blk0 + 1 : min((cb + cn) * (16 / BS), nblk) - blk0;
    // tile jl of the chunk as (A, B): (block, 0), (block, 16-row half) or (block, next block)
    auto tile_of = [&](int jl) -> int2 {
      if constexpr (BS == 16) return make_int2(sm.ids[jl], 0);
      else if constexpr (BS == 32) return make_int2(sm.ids[jl >> 1], jl & 1);
      else return make_int2(sm.ids[2 * jl], sm.ids[min(2 * jl + 1, nb - 1)]);
    };
    // this wave: chunk tiles w, w + NW, ...
    const int nwc = __builtin_amdgcn_readfirstlane(w < cn ? (cn - w + NW - 1) / NW : 0);
    // the chunk's ids, kStage per thread, requested before anything else of the chunk
    constexpr int kStage = (TABLE + kThreads - 1) / kThreads;
    int staged[kStage];
#pragma unroll
    for (int r = 0; r < kStage; ++r) {
      const int i = tid + r * kThreads;
      staged[r] = i < nb ? table[blk0 + i] : 0;
    }
    // The wave's first tile is read from the table directly (scalar cache) and its
    // loads issued before the workgroup's staging of the chunk's ids completes, so the
    // first K/V bytes are on their way one table round trip earlier.  An id outside the
    // pool is replaced by block 0 here; the staged check below then discards the unit.
    // (issued by every wave, so that the wait for the staged ids below is exact; a wave
    // with no tile in the chunk fetches the chunk's last one and never reads it)
    const int jt0 = cb + min(w, cn - 1);
    const uint32_t ext0 = w < cn ? tile_bytes : 0u;  // a wave with no tile in the chunk reads nothing
    auto valid = [&](int id) { return (id >= 0 && (int64_t)id < a.num_blocks) ? id : 0; };
#define PC_FIRST_LOAD()                                                                              \
  do {                                                                                               \
    if constexpr (BS == 16) {                                                                        \
      PC_LOAD(0, valid(uniform_load(table, jt0)), 0, ext0);                                          \
    } else if constexpr (BS == 32) {                                                                 \
      PC_LOAD(0, valid(uniform_load(table, jt0 >> 1)), jt0 & 1, ext0);                               \
    } else {                                                                                         \
      PC_LOAD(0, valid(uniform_load(table, 2 * jt0)), valid(uniform_load(table, min(2 * jt0 + 1, nblk - 1))), ext0); \
    }                                                                                                \
  } while (0)
    PC_FIRST_LOAD();
#pragma unroll
    for (int r = 0; r < kStage; ++r) {
      const int i = tid + r * kThreads;
      if (i < nb) {
        sm.ids[i] = staged[r];
        if (staged[r] < 0 || (int64_t)staged[r] >= a.num_blocks) sm.bad = 1;
      }
    }
    // fused step: this barrier follows the row store of a unit whose tile holding L - 1 is
    // read only after it, so it orders global memory too
    if constexpr (FUSED)
      global_barrier();
    else
      lds_barrier();
#undef PC_FIRST_LOAD
    if (__builtin_amdgcn_readfirstlane(sm.bad)) {
      bad = true;  // a block id outside the pool: nothing more is read, the outputs become NaN
      break;
    }
    if (nwc == 0) continue;
    if (alibi) ab = slope * kLog2e / cs;
    auto ref_of = [&](int j) -> int2 { return tile_of(w + min(j, nwc - 1) * NW); };
    auto ext_of = [&](int j) -> uint32_t { return j < nwc ? tile_bytes : 0u; };
#pragma unroll
    for (int st = 1; st < STAGES - 1; ++st) {
      const int2 t = ref_of(st);
      PC_LOAD(st, __builtin_amdgcn_readfirstlane(t.x), __builtin_amdgcn_readfirstlane(t.y), ext_of(st));
    }
    int2 ref_next = ref_of(STAGES - 1);
    // The ring turns a whole number of times: a step past the wave's last tile in the
    // chunk consumes the zeros of its empty-extent loads with every token masked, which
    // changes no state.
    int it0 = 0;
    do {
#pragma unroll
      for (int st = 0; st < STAGES; ++st) {
        const int it = it0 + st;
        PC_LOAD((st + STAGES - 1) % STAGES, __builtin_amdgcn_readfirstlane(ref_next.x),
                __builtin_amdgcn_readfirstlane(ref_next.y), ext_of(it + STAGES - 1));
        ref_next = ref_of(it + STAGES);
        // keep the scheduler from sinking the prefetch below the wait for this tile
        __builtin_amdgcn_sched_barrier(0);
        // a step past the wave's last tile of this chunk sees no token
        PC_BLOCK(st, it < nwc ? (cb + w + it * NW) * kBlockTokens : t_end);
      }
      it0 += STAGES;
    } while (it0 < nwc);
    // retire the unconsumed tail loads (s_waitcnt vmcnt(0)) before the ring is reused
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
#undef PC_LOAD
#undef PC_BLOCK

  // ---- this wave: one state per head, relative to the head's true max ----------------
  float mt = fmaxf(m_true, __shfl_xor(m_true, 16));
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  const float f = m_ref == -INFINITY ? 0.f : exp2_fast((m_ref - mt) * cs);
  float lw = lsum;
  lw += __shfl_xor(lw, 16);
  lw += __shfl_xor(lw, 32);
  if (col < C) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.acc[w][col][DPL * (4 * rg + i) + j] = acc[j][i] * f;
    if (rg == 0) {
      sm.mw[w][col] = mt;
      sm.lw[w][col] = lw * f;
    }
  }
  __syncthreads();

  // ---- merge the waves and write ------------------------------------------------------
  const bool any_bad = bad;  // block-uniform (the table check is a block-wide vote)
  // PFX: columns written and columns computed, bit c (lanes 0..15 hold columns 0..15)
  uint32_t pfx_out = 0, pfx_on = 0;
  if constexpr (PFX) {
    pfx_out = (uint32_t)__builtin_amdgcn_ballot_w64(pc_out) & 0xFFFFu;
    pfx_on = (uint32_t)__builtin_amdgcn_ballot_w64(pc_on) & 0xFFFFu;
  }
  if constexpr (MC) {
    // 16 columns: per column, once (one thread each), the max M over the waves, each
    // wave's weight exp2((m_w - M) cs) in place of m_w, the merged sum in place of
    // wave 0's and M in place of wave 1's (both read just before)
    static_assert(NW > 1, "the merge keeps M in lw[1]");
    for (int g = tid; g < C; g += kThreads) {
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm.mw[ww][g]);
      float ls = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float fw = (M == -INFINITY || sm.mw[ww][g] == -INFINITY) ? 0.f : exp2_fast((sm.mw[ww][g] - M) * cs);
        ls = fmaf(sm.lw[ww][g], fw, ls);
        sm.mw[ww][g] = fw;
      }
      sm.lw[0][g] = ls;
      sm.lw[1][g] = M;
    }
    __syncthreads();
  }
  // pairs: column g writes the 64 dims of its own head, dims 64*(g >= G/2) .. of the row
  const bool pr = PAIRABLE && a.pair;
  const int Dout = pr ? D / 2 : D;
  for (int o = tid; o < C * Dout; o += kThreads) {
    const int g = pr ? o / (D / 2) : o / D;  // score column
    const int dd = pr ? o - g * (D / 2) : o - g * D;
    const int d = pr ? dd + (g >= G / 2 ? D / 2 : 0) : dd;
    if (PFX && !((pfx_out >> g) & 1u)) continue;  // not this unit's partial
    const bool colbad = PFX && !((pfx_on >> g) & 1u);
    float M = -INFINITY, ls = 0.f, os = 0.f;
    if constexpr (MC) {
      M = sm.lw[1][g];
      ls = sm.lw[0][g];
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) os = fmaf(sm.acc[ww][g][d], sm.mw[ww][g], os);
    } else {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm.mw[ww][g]);
      if (M != -INFINITY) {
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
          const float fw = sm.mw[ww][g] == -INFINITY ? 0.f : exp2_fast((sm.mw[ww][g] - M) * cs);
          ls = fmaf(sm.lw[ww][g], fw, ls);
          os = fmaf(sm.acc[ww][g][d], fw, os);
        }
      }
    }
    float res = M == -INFINITY ? 0.f : os / ls * vsc;
    if (any_bad || colbad) res = NAN;
    const int64_t sh = MT    ? (int64_t)(q0 + tok0 + g / G) * a.num_q_heads + h0 + (g & (G - 1))
                       : PFX ? (int64_t)(s * (NC / G) + g / G) * a.num_q_heads + h0 + (g & (G - 1))
                             : (int64_t)s * a.num_q_heads + h0 + g;
    if constexpr (SPLIT) {
      const int64_t sp = sh * a.max_partitions + part;
      a.tmp_out[sp * Dout + dd] = res;
      if (dd == 0) {
        a.max_logits[sp] = (any_bad || colbad) ? NAN : M * (cs * kLn2);  // back to the natural-log domain
        a.exp_sums[sp] = (any_bad || colbad) ? NAN : ls;
      }
    } else {
      static_cast<uint16_t*>(a.out)[sh * Dout + dd] = (uint16_t)to_storage<ST>(res);
    }
  }
  return MT && tok0 + TPC < n;
}

// Split path: workgroup = (kv head, sequence, partition), fastest-varying first, the
// partitions in descending order.  Every sequence's partition p runs beside the others'
// partition p (a shared prefix's blocks are then read from L2 by all of them at once;
// partition fastest ran the mixed-serving workload at half speed), and the last
// partitions, which only the long sequences have, start first: the grid ends on the
// dense low partitions instead of a sparse tail of long sequences' last partitions.
// FUSED: the decode step's own K/V write in the same launch (a.step_slots).
template <class ST, int D, int G, bool KV8, int BS, bool FUSED = false>
__global__ __launch_bounds__((split_waves<KV8, G>() * kWave)) __attribute__((amdgpu_waves_per_eu(PCACHE_SPLIT_OCC)))
void decode_split_kernel(DecodeArgs a) {
  constexpr int NW = split_waves<KV8, G>();
  constexpr int TABLE = BS >= 16 ? kPartition / kBlockTokens : kPartition / BS;  // a partition's block ids
  __shared__ UnitLds<NW, D, G, TABLE> sm;
  int64_t id = blockIdx.x;
  const int kvh = (int)(id % a.num_kv_heads);
  id /= a.num_kv_heads;
  const int s = (int)(id % a.num_seqs);
  const int part = a.max_partitions - 1 - (int)(id / a.num_seqs);
  const int L = uniform_load(a.seq_lens, s);
  const bool bad = L < 0 || (int64_t)L > (int64_t)a.max_blocks_per_seq * BS ||
                   (int64_t)L > (int64_t)a.max_partitions * kPartition;
  if (!bad && part * kPartition >= L) return;  // a partition past the sequence writes nothing
  // a partition the sequence's shared prefix tokens cover completely: the prefix kernel's
  if (a.shared_lens != nullptr && (part + 1) * kPartition <= a.prefix_blocks * BS &&
      uniform_load(a.shared_lens, s) >= (part + 1) * kPartition)
    return;
  constexpr int STAGES = KV8 ? PCACHE_SPLIT_STAGES_KV8 : PCACHE_SPLIT_STAGES;
  decode_unit<ST, D, G, NW, STAGES, TABLE, true, KV8, BS, G, FUSED>(a, sm, s, kvh, part);
}

// Common-prefix units of the split path: workgroup = (kv head, group of 16 / G sequences,
// partition of the prefix), kv head fastest.  Each tile of the partition is read once for
// the group's 16 score columns (16 / G sequences x G query heads).
template <class ST, int D, int G>
__global__ __launch_bounds__(4 * kWave) __attribute__((amdgpu_waves_per_eu(PCACHE_SPLIT_OCC)))
void decode_prefix_kernel(DecodeArgs a) {
  constexpr int NW = 4;
  constexpr int TABLE = kPartition / kBlockTokens;
  __shared__ UnitLds<NW, D, 16, TABLE> sm;
  int64_t id = blockIdx.x;
  const int kvh = (int)(id % a.num_kv_heads);
  id /= a.num_kv_heads;
  const int groups = (a.num_seqs + 16 / G - 1) / (16 / G);
  const int grp = (int)(id % groups);
  const int part = (int)(id / groups);
  decode_unit<ST, D, G, NW, PCACHE_SPLIT_STAGES, TABLE, true, false, kBlockTokens, 16, false, true>(a, sm, grp, kvh,
                                                                                                    part);
}

// One-pass path for many short units: one workgroup of PCACHE_GRID_WAVES waves per
// (sequence, kv head), dealt by the hardware as earlier workgroups finish (several per
// CU, so one unit's start and merge overlap another's stream).
#ifndef PCACHE_GRID_WAVES
#define PCACHE_GRID_WAVES 4
#endif
#ifndef PCACHE_GRID_TABLE
#define PCACHE_GRID_TABLE 128  // block ids staged at once (2048 tokens of 16-token blocks)
#endif
template <class ST, int D, int G, bool KV8, int BS>
__global__ __launch_bounds__(PCACHE_GRID_WAVES * kWave) __attribute__((amdgpu_waves_per_eu(PCACHE_SPLIT_OCC)))
void decode_grid_kernel(DecodeArgs a) {
  constexpr int NW = PCACHE_GRID_WAVES;
  __shared__ UnitLds<NW, D, G, PCACHE_GRID_TABLE> sm;
  const int kvh = (int)(blockIdx.x % a.num_kv_heads);
  const int s = (int)(blockIdx.x / a.num_kv_heads);
  constexpr int STAGES = KV8 ? PCACHE_SPLIT_STAGES_KV8 : PCACHE_SPLIT_STAGES;
  decode_unit<ST, D, G, NW, STAGES, PCACHE_GRID_TABLE, false, KV8, BS>(a, sm, s, kvh, 0);
}

// One-pass path: persistent workgroups.  Turn 0 takes units in index order (unit u =
// kv head u % Hkv of sequence u / Hkv), so no ranking stands between the launch and the
// first loads.  While turn 0 runs, the sequence lengths are fetched; after it, the
// remaining units are ranked longest first and dealt in snake order, and the workgroup
// whose turn-0 unit was the r-th longest receives the r-th shortest unit of turn 1,
// which evens out the sums across workgroups.  NC > G: several query tokens per
// sequence, in passes of NC / G tokens (one pass unless max_query_len was understated).
// FUSED: the decode step's own K/V write in the same launch (a.step_slots).
template <class ST, int D, int G, bool KV8, int BS, int NC = G, bool FUSED = false>
__global__ __launch_bounds__((onepass_waves<D, KV8, (NC != G)>() * kWave))
__attribute__((amdgpu_waves_per_eu(D == 64 ? PCACHE_ONEPASS_OCC_D64
                                   : KV8 ? PCACHE_ONEPASS_OCC_KV8
                                   : (NC != G) ? PCACHE_ONEPASS_OCC_MT : PCACHE_ONEPASS_OCC)))
void decode_onepass_kernel(DecodeArgs a) {
  constexpr int NW = onepass_waves<D, KV8, (NC != G)>();
  constexpr int kThreads = NW * kWave;
  constexpr int STAGES = KV8 ? PCACHE_ONEPASS_STAGES_KV8 : PCACHE_ONEPASS_STAGES;
  __shared__ UnitLds<NW, D, NC, PCACHE_ONEPASS_TABLE> sm;
  __shared__ int order_lds[kMaxRankedSeqs];  // order_lds[rank] = later-turn sequence of that length rank
  __shared__ __align__(16) int len_lds[kMaxRankedSeqs];
  __shared__ int rank0_lds;                  // length rank of this workgroup's turn-0 sequence

  const int S = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int64_t units = (int64_t)S * Hkv;
  const int64_t W = gridDim.x;
  const int64_t k = blockIdx.x;
  // ranking needs whole sequences in turn 0 (W a multiple of Hkv) and a later turn
  const bool ranked = a.longest_first && S <= kMaxRankedSeqs && units > W && W % Hkv == 0;
  const int S0 = (int)(W / Hkv);  // sequences of turn 0 when ranked
  if (ranked)  // read here, used after turn 0 (its barriers publish the stores)
    for (int t = threadIdx.x; t < S; t += kThreads) len_lds[t] = a.seq_lens[t];

  auto unit = [&](int s, int kvh) __attribute__((always_inline)) {
    int tok0 = 0;
    while (decode_unit<ST, D, G, NW, STAGES, PCACHE_ONEPASS_TABLE, false, KV8, BS, NC, FUSED>(a, sm, s, kvh, 0, tok0))
      tok0 += NC / G;
  };
  if (k < units) unit((int)(k / Hkv), (int)(k % Hkv));
  if (units <= W) return;
  if (ranked) {
    // sequences S0 .. S-1 by length, longest first (ties by index)
    const int4* l4 = reinterpret_cast<const int4*>(len_lds);
    for (int t = S0 + (int)threadIdx.x; t < S; t += kThreads) {
      const int lt = len_lds[t];
      auto before = [&](int lu, int u) { return (int)((lu > lt) || (lu == lt && u < t)); };
      int rank = 0;
      int u = S0;
      for (; u < S && (u & 3) != 0; ++u) rank += before(len_lds[u], u);
      for (; u + 4 <= S; u += 4) {
        const int4 v = l4[u >> 2];
        rank += before(v.x, u) + before(v.y, u + 1) + before(v.z, u + 2) + before(v.w, u + 3);
      }
      for (; u < S; ++u) rank += before(len_lds[u], u);
      order_lds[rank] = t;
    }
    // rank of this workgroup's turn-0 sequence among sequences 0 .. S0-1
    if (threadIdx.x < kWave) {
      const int s0 = (int)(k / Hkv);
      const int l0 = len_lds[s0];
      int c = 0;
      for (int u = threadIdx.x; u < S0; u += kWave) {
        const int lu = len_lds[u];
        c += (lu > l0) || (lu == l0 && u < s0);
      }
      for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
      if (threadIdx.x == 0) rank0_lds = c;
    }
    __syncthreads();
  }
  // unit rank of the turn-0 unit: the Hkv units of one sequence are consecutive
  const int64_t r0 = ranked ? (int64_t)rank0_lds * Hkv + k % Hkv : k;
  const int64_t rest = units - W;
  for (int64_t turn = 1; (turn - 1) * W < rest; ++turn) {
    const int64_t f = (turn & 1) ? W - 1 - r0 : r0;  // snake, shortest first for the longest turn-0 unit
    const int64_t q = (turn - 1) * W + f;            // position among the later units
    if (q >= rest) continue;                          // the last turn is partial
    int s, kvh;
    if (ranked) {
      s = order_lds[(int)(q / Hkv)];
      kvh = (int)(q % Hkv);
    } else {
      s = (int)((W + q) / Hkv);
      kvh = (int)((W + q) % Hkv);
    }
    unit(s, kvh);
  }
}

// Resident workgroups per CU for the one-pass kernel, queried once per instance.
template <class ST, int D, int G, bool KV8, int BS, int NC = G, bool FUSED = false>
int onepass_blocks_per_cu() {
  static int cached = 0;
  if (!cached) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_onepass_kernel<ST, D, G, KV8, BS, NC, FUSED>,
                                                     onepass_waves<D, KV8, (NC != G)>() * kWave, 0) != hipSuccess ||
        n <= 0) {
      (void)hipGetLastError();
      n = 1;
    }
    cached = n;
  }
  return cached;
}

template <class ST, int D, int G, bool KV8, int BS, bool FUSED>
hipError_t launch_typed_as(const DecodeArgs& a, bool split, hipStream_t stream) {
  if (split) {
    const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * a.max_partitions;
    if (units == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_split_kernel<ST, D, G, KV8, BS, FUSED>), dim3((unsigned)units),
                       dim3(split_waves<KV8, G>() * kWave), 0, stream, a);
    return hipGetLastError();
  }
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads;
  if (units == 0) return hipSuccess;
  // PCACHE_ONEPASS_KERNEL (tuning builds): 1 always persistent, 2 always one workgroup
  // per unit; 0 (the library) the rule of onepass_grid
#ifndef PCACHE_ONEPASS_KERNEL
#define PCACHE_ONEPASS_KERNEL 0
#endif
  if constexpr (!FUSED && !KV8 && PCACHE_ONEPASS_KERNEL != 1) {
    if (PCACHE_ONEPASS_KERNEL == 2 || onepass_grid(units, a.max_seq_len, device_compute_units())) {
      hipLaunchKernelGGL((decode_grid_kernel<ST, D, G, KV8, BS>), dim3((unsigned)units),
                         dim3(PCACHE_GRID_WAVES * kWave), 0, stream, a);
      return hipGetLastError();
    }
  }
#ifdef PCACHE_ONEPASS_BLOCKS_PER_CU
  const int64_t slots = (int64_t)device_compute_units() * PCACHE_ONEPASS_BLOCKS_PER_CU;
#else
  const int64_t slots = (int64_t)device_compute_units() * onepass_blocks_per_cu<ST, D, G, KV8, BS, G, FUSED>();
#endif
  const int64_t grid = units < slots ? units : slots;
  hipLaunchKernelGGL((decode_onepass_kernel<ST, D, G, KV8, BS, G, FUSED>), dim3((unsigned)grid),
                     dim3(onepass_waves<D, KV8>() * kWave), 0, stream, a);
  return hipGetLastError();
}

template <class ST, int D, int G, bool KV8, int BS>
hipError_t launch_typed(const DecodeArgs& a, bool split, hipStream_t stream) {
  if (a.step_slots == nullptr) return launch_typed_as<ST, D, G, KV8, BS, false>(a, split, stream);
  // the fused write moves 16-bit rows; with 8-token blocks and 8 heads per kv head at
  // head size 128 the fused one-pass kernel would spill registers (not built)
  if constexpr (KV8 || (BS == 8 && G == 8 && D == 128)) return hipErrorInvalidValue;
  else return launch_typed_as<ST, D, G, KV8, BS, true>(a, split, stream);
}

template <class ST, int D, bool KV8, int BS>
hipError_t launch_group(const DecodeArgs& a, bool split, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_typed<ST, D, 1, KV8, BS>(a, split, stream);
    case 2: return launch_typed<ST, D, 2, KV8, BS>(a, split, stream);
    case 4: return launch_typed<ST, D, 4, KV8, BS>(a, split, stream);
    case 8: return launch_typed<ST, D, 8, KV8, BS>(a, split, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class ST, int D, bool KV8>
hipError_t launch_bs(const DecodeArgs& a, bool split, hipStream_t stream) {
  switch (a.block_size) {
    case 8: return launch_group<ST, D, KV8, 8>(a, split, stream);
    case 16: return launch_group<ST, D, KV8, 16>(a, split, stream);
    case 32: return launch_group<ST, D, KV8, 32>(a, split, stream);
    default: return hipErrorInvalidValue;
  }
}

// several query tokens per sequence: the one-pass kernel with 16 score columns
template <class ST, int D, int G>
hipError_t launch_multitoken_typed(const DecodeArgs& a, hipStream_t stream) {
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads;
  if (units == 0) return hipSuccess;
  const int64_t slots = (int64_t)device_compute_units() * onepass_blocks_per_cu<ST, D, G, false, 16, 16>();
  const int64_t grid = units < slots ? units : slots;
  hipLaunchKernelGGL((decode_onepass_kernel<ST, D, G, false, 16, 16>), dim3((unsigned)grid),
                     dim3(onepass_waves<D, false, true>() * kWave), 0, stream, a);
  return hipGetLastError();
}

template <class ST, int D>
hipError_t launch_multitoken_group(const DecodeArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_multitoken_typed<ST, D, 1>(a, stream);
    case 2: return launch_multitoken_typed<ST, D, 2>(a, stream);
    case 4: return launch_multitoken_typed<ST, D, 4>(a, stream);
    case 8: return launch_multitoken_typed<ST, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class ST>
hipError_t launch_dim(const DecodeArgs& a, int head_size, bool split, hipStream_t stream) {
  switch (head_size) {
    case 64: return a.kv8 ? launch_bs<ST, 64, true>(a, split, stream) : launch_bs<ST, 64, false>(a, split, stream);
    case 128: return a.kv8 ? launch_bs<ST, 128, true>(a, split, stream) : launch_bs<ST, 128, false>(a, split, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

#ifndef PCACHE_LONGEST_FIRST
#define PCACHE_LONGEST_FIRST 1
#endif

hipError_t launch_decode_multitoken(const VarlenArgs& v, int dtype, int head_size, hipStream_t stream) {
  DecodeArgs a{};
  a.out = v.out;
  a.q = v.q;
  a.k_pool = v.k_pool;
  a.v_pool = v.v_pool;
  a.num_blocks = v.num_blocks;
  a.block_stride = v.block_stride;
  a.token_stride = v.token_stride;
  a.head_stride = v.head_stride;
  a.block_tables = v.block_tables;
  a.max_blocks_per_seq = v.max_blocks_per_seq;
  a.seq_lens = v.seq_lens;
  a.num_seqs = v.num_reqs;
  a.num_q_heads = v.num_q_heads;
  a.num_kv_heads = v.num_kv_heads;
  a.block_size = 16;
  a.scale_log2 = v.scale_log2;
  a.longest_first = PCACHE_LONGEST_FIRST && v.num_reqs > 1;
  a.alibi_slopes = v.alibi_slopes;
  a.query_start_loc = v.query_start_loc;
  a.total_q = v.total_q;
  a.causal = v.causal;
  switch (dtype * 1000 + head_size) {
    case 1064: return launch_multitoken_group<F16, 64>(a, stream);
    case 1128: return launch_multitoken_group<F16, 128>(a, stream);
    case 2064: return launch_multitoken_group<BF16, 64>(a, stream);
    case 2128: return launch_multitoken_group<BF16, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class ST, int D, int G>
hipError_t launch_prefix_typed(const DecodeArgs& a, hipStream_t stream) {
  const int64_t pp = (int64_t)a.prefix_blocks * kBlockTokens / kPartition;  // partitions the prefix fills
  const int64_t parts = pp < a.max_partitions ? pp : a.max_partitions;
  const int64_t groups = (a.num_seqs + 16 / G - 1) / (16 / G);
  const int64_t wgs = (int64_t)a.num_kv_heads * groups * parts;
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_prefix_kernel<ST, D, G>), dim3((unsigned)wgs), dim3(4 * kWave), 0, stream, a);
  return hipGetLastError();
}

template <class ST, int D>
hipError_t launch_prefix_group(const DecodeArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_prefix_typed<ST, D, 1>(a, stream);
    case 2: return launch_prefix_typed<ST, D, 2>(a, stream);
    case 4: return launch_prefix_typed<ST, D, 4>(a, stream);
    case 8: return launch_prefix_typed<ST, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_prefix(const DecodeArgs& a, int dtype, int head_size, hipStream_t stream) {
  if (a.block_size != kBlockTokens || a.kv8 || a.pair) return hipErrorInvalidValue;
  switch (dtype * 1000 + head_size) {
    case 1064: return launch_prefix_group<F16, 64>(a, stream);
    case 1128: return launch_prefix_group<F16, 128>(a, stream);
    case 2064: return launch_prefix_group<BF16, 64>(a, stream);
    case 2128: return launch_prefix_group<BF16, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a_in, int dtype, int head_size, bool split, hipStream_t stream) {
  DecodeArgs a = a_in;
  a.longest_first = PCACHE_LONGEST_FIRST && !split && a.num_seqs > 1;
  switch (dtype) {
    case 1: return launch_dim<F16>(a, head_size, split, stream);
    case 2: return launch_dim<BF16>(a, head_size, split, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pcache
