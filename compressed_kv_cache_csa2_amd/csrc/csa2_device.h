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
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

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

// Two E2M1 codes (byte BYTE of `codes`, low nibble first) -> two bf16, exactly. The
// conversion runs with a unit scale: the instruction applies only the exponent of its
// scale operand, so the E4M3 group scale is multiplied in separately.
template <int BYTE>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16x2(uint32_t codes) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, BYTE);
  return __builtin_bit_cast(uint32_t, r);
}

// Two bf16 (packed) times a float scale -> two bf16, by truncation. Exact when every
// product fits in bf16's 8 significant bits, which holds for an E2M1 value (<= 2
// significant bits) times an E4M3 scale (<= 4), in [2^-10, 2688].
__device__ __forceinline__ uint32_t bf16x2_scale_exact(uint32_t pair, float scale) {
  const float lo = __uint_as_float(pair << 16) * scale;
  const float hi = __uint_as_float(pair & 0xFFFF0000u) * scale;
  return (__float_as_uint(hi) & 0xFFFF0000u) | (__float_as_uint(lo) >> 16);
}

// Eight E2M1 codes of one dword (low nibble first) times a scale -> eight bf16 packed in
// four dwords, exactly.
__device__ __forceinline__ u32x4 fp4x8_to_bf16x8(uint32_t codes, float scale) {
  u32x4 r;
  r.x = bf16x2_scale_exact(e2m1x2_to_bf16x2<0>(codes), scale);
  r.y = bf16x2_scale_exact(e2m1x2_to_bf16x2<1>(codes), scale);
  r.z = bf16x2_scale_exact(e2m1x2_to_bf16x2<2>(codes), scale);
  r.w = bf16x2_scale_exact(e2m1x2_to_bf16x2<3>(codes), scale);
  return r;
}

// Eight E2M1 codes of one dword (low nibble first) times a power-of-two scale -> eight
// bf16 packed in four dwords. The conversion applies the exponent of `pow2` exactly, so an
// E8M0 scale 2^(e-127) passed as the float with exponent field e gives exact products while
// they stay in bf16's normal range.
__device__ __forceinline__ u32x4 fp4x8_to_bf16x8_pow2(uint32_t codes, float pow2) {
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2, 3));
  return r;
}

// Indexer score of the 32 positions of one wavefront step over E4M3 keys: lane (n, half)
// holds in raw the bytes 64*half .. +63 of position n's key row, a[kb] the A operand of
// k-block kb (head n, channels 64*half + 8*kb .. +7) and wr the head weights of its rows of
// the 32x32 accumulator. Eight v_mfma_f32_32x32x16_bf16 (exact E4M3 -> bf16 conversion),
// then ReLU, weights and the head sum; both half-waves return the score of position n.
// Every indexer path over E4M3 keys computes its scores with exactly these operations in
// this order, so a score recomputed elsewhere is bit-identical.
__device__ __forceinline__ float e4m3_step_score(const bf16x8 (&a)[8], const float (&wr)[16],
                                                 const u32x4 (&raw)[4]) {
  f32x16 acc = {};
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    const u32x2 lo = e4m3x4_to_bf16x4(raw[kb >> 1][(kb & 1) * 2]);
    const u32x2 hi = e4m3x4_to_bf16x4(raw[kb >> 1][(kb & 1) * 2 + 1]);
    const u32x4 bv = u32x4{lo.x, lo.y, hi.x, hi.y};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], __builtin_bit_cast(bf16x8, bv), acc, 0,
                                                  0, 0);
  }
  float part = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) part += wr[r] * fmaxf(acc[r], 0.f);
  part += __shfl_xor(part, 32);
  return part;
}

// The same over MXFP4 keys: lane (n, half) holds in raw[0..1] the code bytes 32*half .. +31
// of position n's row (channels 64*half .. +63) and in raw[2].x the row's four E8M0 scale
// bytes; k-block kb is code dword kb with the scale of group 2*half + kb/4. Every indexer
// path over MXFP4 keys with a bf16 query uses exactly these operations in this order.
__device__ __forceinline__ float mxfp4_step_score(const bf16x8 (&a)[8], const float (&wr)[16],
                                                  const u32x4 (&raw)[4], int half) {
  f32x16 acc = {};
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    const uint32_t d = raw[kb >> 2][kb & 3];
    const uint32_t e = (raw[2].x >> (8 * (2 * half + (kb >> 2)))) & 0xFFu;
    const u32x4 bv = fp4x8_to_bf16x8_pow2(d, __uint_as_float(e << 23));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], __builtin_bit_cast(bf16x8, bv), acc, 0,
                                                  0, 0);
  }
  float part = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) part += wr[r] * fmaxf(acc[r], 0.f);
  part += __shfl_xor(part, 32);
  return part;
}

// ---- fp16 forms (the attention works in fp16: every E2M1 x E4M3 product, and every E4M3
// value, is exact in fp16, and packed fp16 multiplies halve the conversion work) ----

// Two E2M1 codes (byte BYTE of `codes`, low nibble first) -> two fp16, exactly (unit scale).
template <int BYTE>
__device__ __forceinline__ f16x2 e2m1x2_to_f16x2(uint32_t codes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, BYTE);
}

// Two E4M3 bytes (low or high 16-bit half of `src`) -> two fp16, exactly.
template <bool HIGH_HALF>
__device__ __forceinline__ f16x2 e4m3x2_to_f16x2(uint32_t src) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src, 1.0f, HIGH_HALF);
}

// Eight E2M1 codes (low nibble first) times a scale held in both halves of `s2` ->
// eight fp16. Products have <= 6 significant bits and lie in [2^-10, 2688]: exact.
__device__ __forceinline__ u32x4 fp4x8_to_f16x8(uint32_t codes, f16x2 s2) {
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, e2m1x2_to_f16x2<0>(codes) * s2);
  r.y = __builtin_bit_cast(uint32_t, e2m1x2_to_f16x2<1>(codes) * s2);
  r.z = __builtin_bit_cast(uint32_t, e2m1x2_to_f16x2<2>(codes) * s2);
  r.w = __builtin_bit_cast(uint32_t, e2m1x2_to_f16x2<3>(codes) * s2);
  return r;
}

// Eight E4M3 bytes (two dwords, channel order kept) -> eight fp16, exactly.
__device__ __forceinline__ u32x4 fp8x8_to_f16x8(uint32_t a, uint32_t b) {
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, e4m3x2_to_f16x2<false>(a));
  r.y = __builtin_bit_cast(uint32_t, e4m3x2_to_f16x2<true>(a));
  r.z = __builtin_bit_cast(uint32_t, e4m3x2_to_f16x2<false>(b));
  r.w = __builtin_bit_cast(uint32_t, e4m3x2_to_f16x2<true>(b));
  return r;
}

// LDS transpose read (ds_read_b64_tr_b16): within each group of 16 lanes, output lane c
// receives, as item r, element c%4 of the 4 x 16-bit row that lane 4r + c/4 of the group
// addressed. `p` must point into LDS and be 8-byte aligned.
__device__ __forceinline__ u32x2 lds_read_tr16x4(const uint16_t* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// float -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// float32 -> E4M3 byte, nearest even, saturating at 448 (0x7E); sign kept.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {                 // >= 448
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {           // < 2^-6: multiples of 2^-9
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);   // exact scaling, then RNE
    code = (uint32_t)m;                   // 0..8 (8 is 2^-6, the first normal code)
  } else {
    const uint32_t e = a >> 23;           // biased exponent, 121..135
    const uint32_t mant = a & 0x7FFFFFu;
    uint32_t top = mant >> 20;            // 3 kept bits
    const uint32_t rest = mant & 0xFFFFFu;
    top += (rest > 0x80000u || (rest == 0x80000u && (top & 1u))) ? 1u : 0u;
    code = ((e - 120u) << 3) + top;       // a carry into the exponent is the right value
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// Order-preserving key: a > b as floats <=> key(a) > key(b) as unsigned.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// A score takes part in a selection unless it is -inf or NaN.
__device__ __forceinline__ bool selectable(float f) { return f > -__builtin_inff(); }

// Unsigned minimum / maximum (the device min/max overloads compare as signed int).
__device__ __forceinline__ uint32_t umin32(uint32_t a, uint32_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Block statistics of a Full pass beside each 8-slot block maximum: the block's argmax (the
// lowest slot holding the largest key) in bits 0..2 and, above them, the selection key of
// the largest score among its other seven slots (0 when none is selectable) rounded up to a
// multiple of 8, so the stored word is never below that key.
__device__ __forceinline__ uint32_t block_aux_word(uint32_t key2, uint32_t argmax) {
  return ((key2 + 7u) & ~7u) | argmax;
}

// Indexed ("structured") buffer loads: address = base + index * stride + offset. A load
// whose index is at or past the record count returns zeros without touching memory, so a
// gather can always issue the same loads and mark absent rows with an out-of-range index.
__device__ u32x4 sbuf_load_b128(__amdgpu_buffer_rsrc_t rsrc, int index, int offset, int soffset,
                                int aux) __asm("llvm.amdgcn.struct.ptr.buffer.load.v4i32");
__device__ u32x2 sbuf_load_b64(__amdgpu_buffer_rsrc_t rsrc, int index, int offset, int soffset,
                               int aux) __asm("llvm.amdgcn.struct.ptr.buffer.load.v2i32");
__device__ uint32_t sbuf_load_b32(__amdgpu_buffer_rsrc_t rsrc, int index, int offset, int soffset,
                                  int aux) __asm("llvm.amdgcn.struct.ptr.buffer.load.i32");

// Buffer descriptor over n_rows records of `stride` bytes (stride < 16,384) from `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rows_rsrc(const void* base, int stride,
                                                                 uint32_t n_rows) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)stride, (int)n_rows,
                                           0x00020000);
}

}  // namespace csa2
