// Cache writes on gfx950: quantise bf16 rows into the cache formats the read path reads
// ("DeepSeek-v4.1 Flash: Pushing the Limits of KV Cache Compression", 2.4.4: the main KV
// as E2M1 with one E4M3 scale per 16 channels and no global scale, quantised after RoPE;
// the sliding-window cache kept in FP8; the indexer cache in OCP MXFP4).
//
// Every rounding is to the nearest grid value with ties to the even code, saturating at
// the grid's largest value, decided on float32 values (bf16 inputs are exact in float32):
//   - E4M3: from the float32 bits, 3 mantissa bits kept with round-half-even; below 2^-6
//     the subnormal multiple of 2^-9 is rounded the same way; 448 is the largest value;
//   - E2M1 magnitude thresholds 0.25, 0.75, 1.25, 1.75, 2.5, 3.5 and 5 (the midpoints of
//     0, .5, 1, 1.5, 2, 3, 4, 6), a midpoint going to the even code;
//   - main KV: scale = E4M3(amax / 6) per 16 channels (a float32 division), codes = the
//     E2M1 rounding of the exact quotient x / scale (|x| against each midpoint times the
//     scale, products that are exact in float32), zero codes for a zero scale;
//   - MXFP4 keys: per 32 channels the exponent X = floor(log2 amax) - 2 stored as X + 127
//     kept in 1..254 (127 for an all-zero group), codes = E2M1(x * 2^-X).
// A destination row outside [0, n_rows) is skipped. Each wavefront lane handles eight
// consecutive channels; stores are whole dwords except the scale bytes.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

constexpr int CW_THREADS = 256;

// E4M3 byte (no NaN) -> float32.
__device__ __forceinline__ float e4m3_val(uint32_t b) { return e4m3_to_f32(b); }

// float32 -> E2M1 code (4 bits), nearest even, saturating at 6; no negative zero.
__device__ __forceinline__ uint32_t f32_to_e2m1_rne(float y) {
  const float a = fabsf(y);
  const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return m | ((y < 0.f && m != 0u) ? 8u : 0u);
}

// Eight bf16 (four dwords) -> eight floats.
__device__ __forceinline__ void bf16x8_to_f32(u32x4 v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

// Main-KV latent rows: lane l of a wavefront holds channels 8l .. 8l+7 of one row (half
// of scale group l/2).
__global__ __launch_bounds__(CW_THREADS) void latent_write_kernel(
    int n, const uint16_t* __restrict__ x, const int64_t* __restrict__ rows,
    uint8_t* __restrict__ kv_fp4, int64_t fp4_stride, uint8_t* __restrict__ kv_scale,
    int64_t sc_stride, int64_t n_entries) {
  const int r = blockIdx.x * (CW_THREADS / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= n) return;
  const int64_t dst = rows[r];
  if (dst < 0 || dst >= n_entries) return;
  float f[8];
  bf16x8_to_f32(*reinterpret_cast<const u32x4*>(x + (int64_t)r * 512 + 8 * lane), f);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  const uint32_t s_code = f32_to_e4m3_rne(__fdiv_rn(amax, 6.0f));
  const float s = e4m3_val(s_code);
  uint32_t packed = 0;
  if (s > 0.f) {
    // the exact quotient x / s against each grid midpoint: |x| against midpoint * s, exact
    const float t0 = 0.25f * s, t1 = 0.75f * s, t2 = 1.25f * s, t3 = 1.75f * s;
    const float t4 = 2.5f * s, t5 = 3.5f * s, t6 = 5.0f * s;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a = fabsf(f[i]);
      const uint32_t m = (uint32_t)(a > t0) + (uint32_t)(a >= t1) + (uint32_t)(a > t2) +
                         (uint32_t)(a >= t3) + (uint32_t)(a > t4) + (uint32_t)(a >= t5) +
                         (uint32_t)(a > t6);
      packed |= (m | ((f[i] < 0.f && m != 0u) ? 8u : 0u)) << (4 * i);
    }
  }
  *reinterpret_cast<uint32_t*>(kv_fp4 + dst * fp4_stride + 4 * lane) = packed;
  if ((lane & 1) == 0) kv_scale[dst * sc_stride + (lane >> 1)] = (uint8_t)s_code;
}

// E4M3 rows of d channels (the window rows, d = 512, or E4M3 indexer keys, d = 128): a
// wavefront covers 512 / d rows, lane l channels 8(l % (d/8)) .. +7.
__global__ __launch_bounds__(CW_THREADS) void e4m3_write_kernel(
    int n, int d, const uint16_t* __restrict__ x, const int64_t* __restrict__ rows,
    uint8_t* __restrict__ dst_rows, int64_t dst_stride, int64_t n_rows) {
  const int lanes_per_row = d / 8;
  const int gid = blockIdx.x * CW_THREADS + threadIdx.x;
  const int r = gid / lanes_per_row;
  const int c = gid % lanes_per_row;
  if (r >= n) return;
  const int64_t dst = rows[r];
  if (dst < 0 || dst >= n_rows) return;
  float f[8];
  bf16x8_to_f32(*reinterpret_cast<const u32x4*>(x + (int64_t)r * d + 8 * c), f);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= f32_to_e4m3_rne(f[i]) << (8 * i);
    hi |= f32_to_e4m3_rne(f[4 + i]) << (8 * i);
  }
  *reinterpret_cast<u32x2*>(dst_rows + dst * dst_stride + 8 * c) = u32x2{lo, hi};
}

// MXFP4 indexer keys: 16 lanes per row, lane l (of its row) channels 8l .. +7, four lanes
// per 32-channel scale group.
__global__ __launch_bounds__(CW_THREADS) void mxfp4_key_write_kernel(
    int n, const uint16_t* __restrict__ x, const int64_t* __restrict__ rows,
    uint8_t* __restrict__ k_codes, uint8_t* __restrict__ k_scales, int64_t n_entries) {
  const int gid = blockIdx.x * CW_THREADS + threadIdx.x;
  const int r = gid >> 4;
  const int c = gid & 15;
  // Every lane of the wavefront takes part in the shuffles; rows past n only skip stores.
  float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (r < n) bf16x8_to_f32(*reinterpret_cast<const u32x4*>(x + (int64_t)r * 128 + 8 * c), f);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  int code_s = 127;
  if (amax > 0.f) {
    int e;
    (void)frexpf(amax, &e);                 // amax = m * 2^e, m in [0.5, 1): floor(log2) = e - 1
    code_s = e - 1 - 2 + 127;
    code_s = code_s < 1 ? 1 : (code_s > 254 ? 254 : code_s);
  }
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) packed |= f32_to_e2m1_rne(ldexpf(f[i], 127 - code_s)) << (4 * i);
  if (r >= n) return;
  const int64_t dst = rows[r];
  if (dst < 0 || dst >= n_entries) return;
  *reinterpret_cast<uint32_t*>(k_codes + dst * 64 + 4 * c) = packed;
  if ((c & 3) == 0) k_scales[dst * 4 + (c >> 2)] = (uint8_t)code_s;
}

// ---------------------------------------------------------------------------------------
// Compressor: main-KV entries by gated pooling of m adjacent tokens ("DeepSeek-V4.1-Flash -
// Architecture", section 1: the KV content C and compression weights Z are projections of
// the hidden state; "DeepSeek-v4.1 Flash: Pushing the Limits of KV Cache Compression",
// 3.3.2: gated pooling that is a per-token projection at m = 1, and 2.3.1: no overlap and
// no absolute position embedding). Entry j, channel c = sum over tokens i = jm .. jm+m-1 of
// softmax_i(Z[i, c]) * C[i, c], in float32, stored as bf16 (nearest even). One lane per 8
// channels of one entry.
__global__ __launch_bounds__(CW_THREADS) void compress_kernel(
    int m, int n_out, const uint16_t* __restrict__ c, const uint16_t* __restrict__ z,
    int64_t ld_in, uint16_t* __restrict__ out, int64_t ld_out) {
  const int64_t gid = (int64_t)blockIdx.x * CW_THREADS + threadIdx.x;
  const int64_t j = gid >> 6;
  const int lane = (int)(gid & 63);
  if (j >= n_out) return;
  float zmax[8], den[8], num[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    zmax[k] = -__builtin_inff();
    den[k] = 0.f;
    num[k] = 0.f;
  }
  for (int i = 0; i < m; ++i) {
    float zf[8];
    bf16x8_to_f32(*reinterpret_cast<const u32x4*>(z + (j * m + i) * ld_in + 8 * lane), zf);
#pragma unroll
    for (int k = 0; k < 8; ++k) zmax[k] = fmaxf(zmax[k], zf[k]);
  }
  for (int i = 0; i < m; ++i) {
    float zf[8], cf[8];
    bf16x8_to_f32(*reinterpret_cast<const u32x4*>(z + (j * m + i) * ld_in + 8 * lane), zf);
    bf16x8_to_f32(*reinterpret_cast<const u32x4*>(c + (j * m + i) * ld_in + 8 * lane), cf);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float g = expf(zf[k] - zmax[k]);
      den[k] += g;
      num[k] += g * cf[k];
    }
  }
  u32x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float lo = num[2 * k] / den[2 * k];
    const float hi = num[2 * k + 1] / den[2 * k + 1];
    o[k] = f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
  }
  *reinterpret_cast<u32x4*>(out + j * ld_out + 8 * lane) = o;
}

// Indexer keys as a projection of main-KV entries ("DeepSeek-v4.1 Flash: Pushing the Limits
// of KV Cache Compression", 2.3.1): k[r, o] = sum_c e[r, c] * W[o, c] with W bf16
// [128, 512] (output channel major), fp32 accumulation on v_mfma_f32_32x32x16_bf16, bf16
// output (nearest even). A wavefront computes 32 rows x all 128 outputs as four 32 x 32
// tiles (four independent accumulation chains sharing each A operand); a workgroup 128
// rows. A operand: lane l holds row l%32, channels k0 + 8(l/32) .. +7; B of tile q: output
// 32q + l%32, the same channels; each is one 16-byte load (W stays in cache).
constexpr int PJ_ROWS = 32 * (CW_THREADS / 64);

__global__ __launch_bounds__(CW_THREADS) void project_kernel(
    int n, const uint16_t* __restrict__ e, int64_t ld_e, const uint16_t* __restrict__ wk,
    uint16_t* __restrict__ out, int64_t ld_out) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int64_t row0 = (int64_t)blockIdx.x * PJ_ROWS + 32 * wave;
  if (row0 >= n) return;
  const int64_t my_row = row0 + (lane & 31);
  const uint16_t* arow = e + (my_row < n ? my_row : row0) * ld_e + 8 * half;
  const uint16_t* brow = wk + (int64_t)(lane & 31) * 512 + 8 * half;
  f32x16 acc[4] = {};
#pragma unroll 4
  for (int k0 = 0; k0 < 512; k0 += 16) {
    const bf16x8 av = *reinterpret_cast<const bf16x8*>(arow + k0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(brow + 32 * 512 * q + k0);
      acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[q], 0, 0, 0);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int o = 32 * q + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = row0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (row < n) out[row * ld_out + o] = (uint16_t)f32_to_bf16_rne(acc[q][r]);
    }
  }
}

hipError_t launch_compress(int m, int n_out, const uint16_t* c, const uint16_t* z, int64_t ld_in,
                           uint16_t* out, int64_t ld_out, hipStream_t stream) {
  const int64_t threads = (int64_t)n_out * 64;
  hipLaunchKernelGGL(compress_kernel, dim3((unsigned)((threads + CW_THREADS - 1) / CW_THREADS)),
                     dim3(CW_THREADS), 0, stream, m, n_out, c, z, ld_in, out, ld_out);
  return hipGetLastError();
}

hipError_t launch_project_index_key(int n, const uint16_t* e, int64_t ld_e, const uint16_t* wk,
                                    uint16_t* out, int64_t ld_out, hipStream_t stream) {
  hipLaunchKernelGGL(project_kernel, dim3((unsigned)((n + PJ_ROWS - 1) / PJ_ROWS)), dim3(CW_THREADS),
                     0, stream,
                     n, e, ld_e, wk, out, ld_out);
  return hipGetLastError();
}

hipError_t launch_latent_write(int n, const uint16_t* x, const int64_t* rows, uint8_t* kv_fp4,
                               int64_t fp4_stride, uint8_t* kv_scale, int64_t sc_stride,
                               int64_t n_entries, hipStream_t stream) {
  const int per_block = CW_THREADS / 64;
  hipLaunchKernelGGL(latent_write_kernel, dim3((n + per_block - 1) / per_block), dim3(CW_THREADS),
                     0, stream, n, x, rows, kv_fp4, fp4_stride, kv_scale, sc_stride, n_entries);
  return hipGetLastError();
}

hipError_t launch_e4m3_write(int n, int d, const uint16_t* x, const int64_t* rows,
                             uint8_t* dst, int64_t dst_stride, int64_t n_rows,
                             hipStream_t stream) {
  const int64_t threads = (int64_t)n * (d / 8);
  hipLaunchKernelGGL(e4m3_write_kernel, dim3((unsigned)((threads + CW_THREADS - 1) / CW_THREADS)),
                     dim3(CW_THREADS), 0, stream, n, d, x, rows, dst, dst_stride, n_rows);
  return hipGetLastError();
}

hipError_t launch_mxfp4_key_write(int n, const uint16_t* x, const int64_t* rows, uint8_t* k_codes,
                                  uint8_t* k_scales, int64_t n_entries, hipStream_t stream) {
  const int64_t threads = (int64_t)n * 16;
  hipLaunchKernelGGL(mxfp4_key_write_kernel,
                     dim3((unsigned)((threads + CW_THREADS - 1) / CW_THREADS)), dim3(CW_THREADS),
                     0, stream, n, x, rows, k_codes, k_scales, n_entries);
  return hipGetLastError();
}

}  // namespace csa2
