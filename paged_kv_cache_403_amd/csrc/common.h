// Shared device helpers for the gfx950 kernels: storage types, 16-byte
// vector access, conversions, and cross-lane exchanges on a 64-lane
// wavefront built from DPP / ds_swizzle / ds_bpermute.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Storage types.  Elements are moved as raw bits; arithmetic is fp32.
struct F32 {
  using elem = float;
  static constexpr int bytes = 4;
};
struct F16 {
  using elem = _Float16;
  static constexpr int bytes = 2;
};
struct BF16 {
  using elem = __bf16;
  static constexpr int bytes = 2;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Widen the two elements packed in a dword (16-bit types) to fp32.
template <typename ST>
__device__ __forceinline__ void widen2(uint32_t w, float& a, float& b);
template <>
__device__ __forceinline__ void widen2<F16>(uint32_t w, float& a, float& b) {
  f16x2 h = __builtin_bit_cast(f16x2, w);
  a = static_cast<float>(h[0]);
  b = static_cast<float>(h[1]);
}
template <>
__device__ __forceinline__ void widen2<BF16>(uint32_t w, float& a, float& b) {
  a = bf16_lo(w);
  b = bf16_hi(w);
}

// Round fp32 to the storage type (round to nearest even).
template <typename ST>
__device__ __forceinline__ typename ST::elem narrow(float x) {
  return static_cast<typename ST::elem>(x);
}

// fp32 dot product of one 16-byte chunk of K with the matching q chunk, added
// to acc.  For 16-bit types q is kept packed (exact) and v_dot2 is used.
// Vector elements are copied to scalars before __builtin_bit_cast: the
// compiler mis-selects the element when it reinterprets an element lvalue.
template <typename ST>
__device__ __forceinline__ float dot16(const u32x4& qv, const u32x4& kv, float acc);
template <>
__device__ __forceinline__ float dot16<F16>(const u32x4& qv, const u32x4& kv, float acc) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t a = qv[c], b = kv[c];
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
  }
  return acc;
}
template <>
__device__ __forceinline__ float dot16<BF16>(const u32x4& qv, const u32x4& kv, float acc) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t a = qv[c], b = kv[c];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
  }
  return acc;
}
template <>
__device__ __forceinline__ float dot16<F32>(const u32x4& qv, const u32x4& kv, float acc) {
#pragma unroll
  for (int c = 0; c < 4; ++c) acc = __builtin_fmaf(__uint_as_float(qv[c]), __uint_as_float(kv[c]), acc);
  return acc;
}

// Widen a 16-byte chunk to fp32 values (VEC = 16 / bytes of them).
template <typename ST>
__device__ __forceinline__ void widen16(const u32x4& v, float* out) {
  if constexpr (ST::bytes == 4) {
#pragma unroll
    for (int c = 0; c < 4; ++c) out[c] = __uint_as_float(v[c]);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) widen2<ST>(v[c], out[2 * c], out[2 * c + 1]);
  }
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 load16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x & 63); }

// Value held by lane (lane ^ M) of the same wavefront.
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  int x = __float_as_int(v);
  if constexpr (M == 1) {
    x = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    x = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (M == 8) {
    x = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // row_ror:8 == xor 8 in a 16-lane row
  } else if constexpr (M == 4 || M == 16) {
    x = __builtin_amdgcn_ds_swizzle(x, 0x1F | (M << 10));  // bitmask mode, xor_mask = M
  } else {
    static_assert(M == 32, "xor mask");
    x = __builtin_amdgcn_ds_bpermute((lane_id() ^ 32) << 2, x);
  }
  return __int_as_float(x);
}

// Runtime-dispatched variant for masks known only as loop indices that the
// compiler fully unrolls.
template <int M>
struct XorLane {
  static __device__ __forceinline__ float get(float v) { return xor_lane<M>(v); }
};

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

}  // namespace pa
