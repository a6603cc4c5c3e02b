// device_common.h -- storage-type traits and wavefront helpers for gfx950 kernels.
//
// Storage types are carried as raw bits: a 16-byte vector (uint4) holds 8 fp16 /
// bf16 or 4 fp32 elements.  Arithmetic is fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pcache {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

struct F32 {
  static constexpr int kBytes = 4;
  static constexpr int kCode = 0;
};
struct F16 {
  static constexpr int kBytes = 2;
  static constexpr int kCode = 1;
};
struct BF16 {
  static constexpr int kBytes = 2;
  static constexpr int kCode = 2;
};

// ---- element decode -------------------------------------------------------------
// Element e (0..3 for fp32, 0..7 for 16-bit types) of a 16-byte vector, as float.
template <class ST>
__device__ __forceinline__ float elem(const uint4& v, int e);

template <>
__device__ __forceinline__ float elem<F32>(const uint4& v, int e) {
  const uint32_t w = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
  return __uint_as_float(w);
}
template <>
__device__ __forceinline__ float elem<BF16>(const uint4& v, int e) {
  const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}
template <>
__device__ __forceinline__ float elem<F16>(const uint4& v, int e) {
  const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  const uint16_t h = (e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
  return (float)__builtin_bit_cast(_Float16, h);
}

// ---- 16-byte partial dot product ------------------------------------------------
// sum over the vector's elements of k[e] * q[e], added to acc (fp32 accumulate).
template <class ST>
__device__ __forceinline__ float dot16(const uint4& k, const uint4& q, float acc);

template <>
__device__ __forceinline__ float dot16<BF16>(const uint4& k, const uint4& q, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.x), __builtin_bit_cast(bf16x2_t, q.x), acc,
                                        false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.y), __builtin_bit_cast(bf16x2_t, q.y), acc,
                                        false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.z), __builtin_bit_cast(bf16x2_t, q.z), acc,
                                        false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.w), __builtin_bit_cast(bf16x2_t, q.w), acc,
                                        false);
  return acc;
}
template <>
__device__ __forceinline__ float dot16<F16>(const uint4& k, const uint4& q, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, k.x), __builtin_bit_cast(f16x2_t, q.x), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, k.y), __builtin_bit_cast(f16x2_t, q.y), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, k.z), __builtin_bit_cast(f16x2_t, q.z), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, k.w), __builtin_bit_cast(f16x2_t, q.w), acc, false);
  return acc;
}
template <>
__device__ __forceinline__ float dot16<F32>(const uint4& k, const uint4& q, float acc) {
  acc = fmaf(__uint_as_float(k.x), __uint_as_float(q.x), acc);
  acc = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), acc);
  acc = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), acc);
  acc = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), acc);
  return acc;
}

// ---- fp32 -> storage, round to nearest even ---------------------------------------
template <class ST>
__device__ __forceinline__ uint32_t to_storage(float x);

template <>
__device__ __forceinline__ uint32_t to_storage<F32>(float x) {
  return __float_as_uint(x);
}
template <>
__device__ __forceinline__ uint32_t to_storage<F16>(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);  // v_cvt_f16_f32 rounds to nearest even
}
template <>
__device__ __forceinline__ uint32_t to_storage<BF16>(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // NaN stays a quiet NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ---- cross-lane sums inside a group of lanes that shares one token row -------------
// DPP row controls (gfx9): row_mirror pairs lane i with 15-i, row_half_mirror pairs i
// with 7-i inside each half row, quad_perm [2,3,0,1] and [1,0,3,2] pair i with i^2
// and i^1.  Each is an involution; applied in this order they sum over 16 (resp. 8)
// lanes.  A 32-lane group first folds lane i with i^16 through ds_swizzle.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  // every control used here reads a lane of the same row, so bound_ctrl never matters;
  // setting it lets the compiler fold the move into the consuming v_add/v_max
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppQuadXor1 = 0xB1;

template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 8 || LANES == 16 || LANES == 32, "token-row group of 8, 16 or 32 lanes");
  if constexpr (LANES == 32)
    x += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));  // i ^ 16
  if constexpr (LANES >= 16) x += dpp<kDppRowMirror>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppQuadXor1>(x);
  return x;
}

// ---- lanes of one wave exchanging values through LDS -----------------------------
// A store by one lane and a load of the same LDS word by another lane of the same
// wave are unsynchronised in the language's memory model, so the compiler may move
// the load above the store (or forward a lane's own store).  This wavefront-scope
// release/acquire pair pins the order: everything stored before it is visible to
// every lane's loads after it.  No s_barrier is involved.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace pcache
