// Device helpers for the gfx950 kernels: vector types, FP8/bf16 conversions, MFMA
// wrappers and wave shuffles (the page-gather address code is in kv_addr.hpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.hpp"

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((vector_size(8)));
typedef int i32x2 __attribute__((vector_size(8)));

#define PA_LDS __attribute__((address_space(3)))

// ---- MFMA ----------------------------------------------------------------------
// 16x16x32: A lane l holds row l%16, K = 8*(l/16)..+7; B lane l holds column l%16,
// same K; C lane l holds rows 4*(l/16)..+3 of column l%16.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_fp8(long a, long b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

// ---- conversions ------------------------------------------------------------------
// 8 e4m3 codes (two dwords) -> 8 bf16, exactly (every e4m3 value is a bf16 value).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}
// 8 int8 codes (two dwords, byte k = code k) -> 8 bf16, exactly (|code| <= 128 fits the
// 8-bit significand of bf16).
__device__ __forceinline__ bf16x8 i8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  bf16x8 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    r[k] = (__bf16)(float)(int8_t)(lo >> (8 * k));
    r[4 + k] = (__bf16)(float)(int8_t)(hi >> (8 * k));
  }
  return r;
}
template <bool I8>
__device__ __forceinline__ bf16x8 codes8_to_bf16x8(uint32_t lo, uint32_t hi) {
  if constexpr (I8) return i8x8_to_bf16x8(lo, hi);
  else return fp8x8_to_bf16x8(lo, hi);
}
// Four floats -> four e4m3 codes packed in a dword (RNE; inputs must be within +-448).
__device__ __forceinline__ uint32_t f32x4_to_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
template <bool HI_WORD>
__device__ __forceinline__ f32x2 fp8x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI_WORD);
}

// Reductions over lanes {l, l^16, l^32, l^48}: the gfx950 row-swap moves exchange
// 32-lane halves and 16-lane rows of two registers in the VALU, with no LDS round trip.
// permlane32_swap(x, x) yields {x[l mod 32], x[(l mod 32) + 32]}; permlane16_swap(x, x)
// yields the even and the odd row of each row pair, so each step combines lane l with
// lane l^32 (then l^16).
__device__ __forceinline__ float swap32_combine_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap16_combine_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_max_xor_16_32(float x) { return swap16_combine_max(swap32_combine_max(x)); }
__device__ __forceinline__ float wave_sum_xor_16_32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
