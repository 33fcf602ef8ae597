// Matrix-core helpers shared by the gfx950 attention kernels that run their
// contractions as v_mfma_f32_32x32x16_{bf16,f16}: the MFMA call, packing of
// fp32 pairs to 16-bit operands, reductions across the two 32-lane halves
// of a wavefront, and the key order that lets a score accumulator feed the
// next contraction directly.
//
// Operand layout of the 32x32x16 instruction on a 64-lane wavefront: lane l
// holds row (l % 32) of A (column of B) and the 8 consecutive k-elements
// starting at 8 * (l / 32); the accumulator lane l holds column (l % 32) and
// rows 8j + 4(l / 32) + i for j, i in 0..3, element 4j + i.
#pragma once

#include "common.h"

namespace pa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <typename ST>
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c);
template <>
__device__ __forceinline__ f32x16 mfma32<BF16>(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<F16>(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}

// v_mfma_f32_16x16x32_{bf16,f16}: lane l holds row (l % 16) of A and column
// (l % 16) of B, each with the 8 consecutive k-elements starting at
// 8 * (l / 16); the accumulator lane l holds column (l % 16), rows
// 4 (l / 16) + i, element i (checked on gfx950 with an exact integer product).
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <typename ST>
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c);
template <>
__device__ __forceinline__ f32x4 mfma16<BF16>(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16<F16>(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}

// two fp32 -> one dword of two 16-bit values (round to nearest even)
template <typename ST>
__device__ __forceinline__ uint32_t pack2(float a, float b);
template <>
__device__ __forceinline__ uint32_t pack2<BF16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, bf16x2{static_cast<__bf16>(a), static_cast<__bf16>(b)});
}
template <>
__device__ __forceinline__ uint32_t pack2<F16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, f16x2{static_cast<_Float16>(a), static_cast<_Float16>(b)});
}

// Max / sum of x over lanes l and l ^ 32.  v_permlane32_swap exchanges the
// two 32-lane halves between its two operands; with x in both, every lane
// ends up holding its own value in one result and its partner's in the
// other (which one depends on the half), so both reductions are symmetric.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A-operand row m of a 32-key subtile holds key perm(m): bits 2 and 3 swapped.
__device__ __forceinline__ int key_perm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

}  // namespace pa
