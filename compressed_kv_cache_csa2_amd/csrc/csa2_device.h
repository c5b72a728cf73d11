// Device-side helpers shared by the CSA2 kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two E4M3 bytes (the low or high 16-bit half of `src`) -> two bf16, exactly: every E4M3
// value is a bf16 value. Element 0 comes from the lower byte.
template <bool HIGH_HALF>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t src) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, 1.0f, HIGH_HALF);
  return __builtin_bit_cast(uint32_t, r);
}

// Four E4M3 bytes -> four bf16 packed in two dwords (channel order kept).
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t src) {
  u32x2 r;
  r.x = e4m3x2_to_bf16x2<false>(src);
  r.y = e4m3x2_to_bf16x2<true>(src);
  return r;
}

// E4M3 scale byte -> float (OCP E4M3FN: bias 7, exponent 0 is subnormal m * 2^-9).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 0xF, m = b & 0x7;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return (b & 0x80) ? -v : v;
}

// E2M1 code (4 bits) -> float bits. Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6: for codes >= 2
// the exponent/mantissa fields are (code + 252) << 22; code 1 is 0.5.
__device__ __forceinline__ uint32_t e2m1_to_f32_bits(uint32_t c) {
  const uint32_t mag = c & 7u;
  uint32_t bits = mag >= 2u ? ((mag + 252u) << 22) : (mag ? 0x3F000000u : 0u);
  return bits | ((c & 8u) << 28);
}

// Eight E2M1 codes of one dword (low nibble first) times a scale -> eight bf16 packed in
// four dwords. The product of a 2-significant-bit code and a 4-significant-bit scale has
// at most 5 significant bits and lies in [2^-10, 2688], so truncating the float to its
// upper half is exact.
__device__ __forceinline__ u32x4 fp4x8_to_bf16x8(uint32_t codes, float scale) {
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v = __uint_as_float(e2m1_to_f32_bits((codes >> (4 * i)) & 0xFu)) * scale;
    h[i] = __float_as_uint(v) >> 16;
  }
  u32x4 r;
  r.x = h[0] | (h[1] << 16);
  r.y = h[2] | (h[3] << 16);
  r.z = h[4] | (h[5] << 16);
  r.w = h[6] | (h[7] << 16);
  return r;
}

// float -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Order-preserving key: a > b as floats <=> key(a) > key(b) as unsigned.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// A score takes part in a selection unless it is -inf or NaN.
__device__ __forceinline__ bool selectable(float f) { return f > -__builtin_inff(); }

}  // namespace csa2
