// mfma_common.h -- gfx950 building blocks shared by the matrix-core attention kernels
// (decode_mfma.hip, varlen.hip): MFMA wrappers for the q.k and P.V tiles, packing of
// probabilities into the 16-bit operand type, exact widening of OCP E4M3 codes,
// buffer resources for one K/V tile, scalar-cache loads of read-only data, and an
// LDS-only workgroup barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace pcache {
namespace {

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource, dword 3 for gfx9-family parts

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

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

// out^T tile += V^T tile . P^T tile (K = 16 tokens)
template <class ST>
__device__ __forceinline__ f32x4_t mfma_pv(const uint2& v, const uint2& p, f32x4_t c);
template <>
__device__ __forceinline__ f32x4_t mfma_pv<BF16>(const uint2& v, const uint2& p, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, v), __builtin_bit_cast(bf16x4_t, p),
                                                   c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4_t mfma_pv<F16>(const uint2& v, const uint2& p, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, v), __builtin_bit_cast(f16x4_t, p), c, 0, 0,
                                               0);
}

// two floats rounded to nearest-even into one dword of the storage type
template <class ST>
__device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <>
__device__ __forceinline__ uint32_t pack2<BF16>(float lo, float hi) {
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  const bf16x2_v v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
template <>
__device__ __forceinline__ uint32_t pack2<F16>(float lo, float hi) {
  typedef _Float16 f16x2_v __attribute__((ext_vector_type(2)));
  const f16x2_v v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// bf16 probabilities enter P.V as two operands, the value rounded to bf16 and the part
// that rounding drops (rounded to bf16 in turn), so that P.V sees each probability to
// about 2^-16 of its size rather than bf16's 2^-8: at outputs of 2 to 4, where rounding
// the output to bf16 already costs up to 2^-7, one rounding of the probabilities could take
// the result past 1e-2 of the exact value.  fp16 (2^-11) keeps a single operand.
template <class ST>
constexpr bool kSplitP = false;
template <>
constexpr bool kSplitP<BF16> = true;

// the residuals a - bf16(a), b - bf16(b) of a dword packed by pack2<BF16>(a, b), each
// exact in fp32 and rounded to bf16
__device__ __forceinline__ uint32_t residual2(uint32_t packed, float a, float b) {
  const float ha = __builtin_bit_cast(float, packed << 16);
  const float hb = __builtin_bit_cast(float, packed & 0xffff0000u);
  return pack2<BF16>(a - ha, b - hb);
}

// four E4M3 codes (one dword) widened exactly to two dwords of the 16-bit type
template <class ST>
__device__ __forceinline__ uint2 widen4(uint32_t codes);
template <>
__device__ __forceinline__ uint2 widen4<BF16>(uint32_t codes) {
  return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true)));
}
template <>
__device__ __forceinline__ uint2 widen4<F16>(uint32_t codes) {
  return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes, 1.0f, true)));
}

// a lane's slice of one V row: 8 (head_size 128) or 4 (64) 16-bit values
template <int N>
struct VRowOf;
template <>
struct VRowOf<8> {
  using type = uint4;
};
template <>
struct VRowOf<4> {
  using type = uint2;
};
__device__ __forceinline__ uint32_t vword(const uint4& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }
__device__ __forceinline__ uint32_t vword(const uint2& v, int i) { return i == 0 ? v.x : v.y; }

// the same slice as E4M3 codes: 8 bytes (head_size 128) or 4 (64)
template <int N>
struct VRow8Of;
template <>
struct VRow8Of<8> {
  using type = uint2;
};
template <>
struct VRow8Of<4> {
  using type = uint32_t;
};
__device__ __forceinline__ uint32_t vword(uint32_t v, int) { return v; }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-uniform reads of data the kernel never writes (lengths, block tables, slopes),
// through the scalar data cache: they count on their own counter, so waiting for one
// does not also wait for the vector loads issued before it.
template <class T>
__device__ __forceinline__ T uniform_load(const T* p, int64_t i) {
  typedef const __attribute__((address_space(4))) T cT;
  return ((cT*)p)[i];
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Barrier that orders LDS only: vector loads in flight stay in flight across it
// (__syncthreads() also waits for every outstanding global access of the wave).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Barrier whose workgroup-scope release/acquire covers global memory as well: a global
// store by one wave before it is visible to every wave's global loads after it, and the
// compiler may move no global access across it.  (It waits for the wave's outstanding
// vector memory accesses, loads included.)
__device__ __forceinline__ void global_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

}  // namespace
}  // namespace pcache
