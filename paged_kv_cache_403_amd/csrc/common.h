// Shared device helpers for the gfx950 kernels: storage types, 16-byte
// vector access, conversions, and cross-lane exchanges on a 64-lane
// wavefront built from DPP / ds_swizzle / ds_bpermute.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedattn.h"

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
// One-byte OCP E4M3 codes (FP8 KV pools); widened exactly by the gfx950
// conversion instructions.
struct FP8 {
  using elem = uint8_t;
  static constexpr int bytes = 1;
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
  if constexpr (ST::bytes == 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t w = v[c];
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);  // bytes 0, 1
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);   // bytes 2, 3
      out[4 * c] = lo[0];
      out[4 * c + 1] = lo[1];
      out[4 * c + 2] = hi[0];
      out[4 * c + 3] = hi[1];
    }
  } else if constexpr (ST::bytes == 4) {
#pragma unroll
    for (int c = 0; c < 4; ++c) out[c] = __uint_as_float(v[c]);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) widen2<ST>(v[c], out[2 * c], out[2 * c + 1]);
  }
}

// fp32 dot product of 16 E4M3 codes (one 16-byte chunk of K) with the
// matching 16 q values held as 8 packed 16-bit pairs (two 16-byte chunks):
// each code pair is widened exactly to the q type, then v_dot2.
template <typename AT>
__device__ __forceinline__ float dot_fp8(const u32x4* qv, const u32x4& kv, float acc);
template <>
__device__ __forceinline__ float dot_fp8<F16>(const u32x4* qv, const u32x4& kv, float acc) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t w = kv[c];
    const uint32_t q0 = qv[c / 2][2 * (c % 2)], q1 = qv[c / 2][2 * (c % 2) + 1];
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, q0), __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, false),
                                 acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, q1), __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, true),
                                 acc, false);
  }
  return acc;
}
template <>
__device__ __forceinline__ float dot_fp8<BF16>(const u32x4* qv, const u32x4& kv, float acc) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t w = kv[c];
    const uint32_t q0 = qv[c / 2][2 * (c % 2)], q1 = qv[c / 2][2 * (c % 2) + 1];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q0),
                                          __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q1),
                                          __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true), acc, false);
  }
  return acc;
}

// Two E4M3 codes of a dword (bytes 0-1, or 2-3 when HI) widened exactly to
// a packed pair of the 16-bit type.
template <typename ST, bool HI>
__device__ __forceinline__ uint32_t widen_fp8_pair(uint32_t w);
template <>
__device__ __forceinline__ uint32_t widen_fp8_pair<F16, false>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, false));
}
template <>
__device__ __forceinline__ uint32_t widen_fp8_pair<F16, true>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, true));
}
template <>
__device__ __forceinline__ uint32_t widen_fp8_pair<BF16, false>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false));
}
template <>
__device__ __forceinline__ uint32_t widen_fp8_pair<BF16, true>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true));
}

// fp32 -> E4M3 code: nearest value, ties to the even code, magnitudes past
// 448 saturate to +-448, NaN -> S.1111.111, the sign of zero kept.  Built
// from the format's fields (RNE of the fp32 significand to 3 bits for
// normals, of x * 2^9 to an integer below 2^-6).
__device__ __forceinline__ uint32_t to_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  if (x != x) return sign | 0x7Fu;
  const float a = fminf(fabsf(x), 448.f);
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.f));  // 8 is the smallest normal's code
  } else {
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);  // round the significand to 3 bits, ties to even
    const uint32_t e = (u >> 23) - 127u + 7u;
    code = (e << 3) | ((u >> 20) & 7u);
  }
  return sign | code;
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

// Checking build (PA_DEBUG): the kernels count the device metadata they
// clamp or skip (PA_DEBUG_COUNT, kinds pa_debug_kind; in the product build it
// expands to no code at all) in counters of their own translation
// unit -- the library is linked without relocatable device code, so each
// unit's code object holds its own copy -- and PA_DEBUG_UNIT(name) gives the
// unit a host function debug_counts_<name> that adds them into a host array
// and optionally clears them.
#ifdef PA_DEBUG
namespace dbg {
static __device__ unsigned long long counts[PA_DBG_KINDS];
}
#define PA_DEBUG_COUNT(kind, hit)                                 \
  do {                                                            \
    if (hit) atomicAdd(&::pa::dbg::counts[kind], 1ull);           \
  } while (0)
#define PA_DEBUG_UNIT(name)                                                                            \
  hipError_t debug_counts_##name(unsigned long long* acc, bool reset) {                               \
    unsigned long long v[PA_DBG_KINDS];                                                                \
    hipError_t e = hipMemcpyFromSymbol(v, HIP_SYMBOL(dbg::counts), sizeof(v), 0, hipMemcpyDeviceToHost); \
    if (e != hipSuccess) return e;                                                                     \
    for (int k = 0; k < PA_DBG_KINDS; ++k) acc[k] += v[k];                                             \
    if (!reset) return hipSuccess;                                                                     \
    const unsigned long long z[PA_DBG_KINDS] = {};                                                     \
    return hipMemcpyToSymbol(HIP_SYMBOL(dbg::counts), z, sizeof(z), 0, hipMemcpyHostToDevice);        \
  }
#else
#define PA_DEBUG_COUNT(kind, hit) \
  do {                            \
  } while (0)
#define PA_DEBUG_UNIT(name)
#endif

}  // namespace pa
