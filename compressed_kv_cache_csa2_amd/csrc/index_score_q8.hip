// Lightning-indexer score with an MXFP8 query over MXFP4 keys, on gfx950's scaled
// f8f6f4 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// The pages' V4 lineage runs the indexer in low precision ("DeepSeek-v4.1 Flash: Pushing
// the Limits of KV Cache Compression", 2.4.4 and 3.1: FP4 indexer keys in OCP MXFP4). Here
// the query is quantised too, to OCP MXFP8 (E4M3 elements, one E8M0 scale per 32
// channels), so both operands go to the matrix core as they are stored and the hardware
// applies both scales: no conversion instructions in the stream, two MFMAs per 32
// positions instead of eight. Every product (E4M3 x E2M1 x two powers of two) is exact in
// fp32; only the accumulation rounds.
//
// Operand layout of the 32x32x64 scaled MFMA on gfx950 (established with an in-bounds lane
// probe): for lane l, row/column l % 32 and half h = l / 32,
//   A (fp8, 32 bytes): byte j < 16 holds k = 16h + j, byte j >= 16 holds k = 32 + 16h + j - 16;
//   B (fp4, 16 bytes, low nibble first): nibble q holds k = 32h + q;
//   the A and B scale bytes of lane l cover k-block h (k = 32h .. 32h + 31) of its row or
//   column; D as in the bf16 32x32 products (row 8(r/4) + 4h + r%4, column l % 32).
// For MFMA i (channels 64i .. 64i+63) a key lane (position n, half h) therefore holds code
// bytes 32i + 16h .. +15 of its row (channels 64i + 32h .. +31, one 16-byte load) with
// scale byte 2i + h, and a query lane (head m, half h) holds E4M3 bytes 64i + 16h .. +15
// and 64i + 32 + 16h .. +15 of its head with the head's scale byte 2i + h.
// E4M3 keys take the fp8 B form, which is laid out as the fp8 A operand (checked through
// the scores against the oracle): a key lane holds bytes 64i + 16h .. +15 and
// 64i + 32 + 16h .. +15 of its row, with the unit scale byte 127.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int Q8_THREADS = 256;
// 32-position steps per wavefront: 2,048 slots per Full workgroup, 512 per Reindex one (the
// pool is 16,384 slots per query, so smaller tiles keep every CU busy)
constexpr int Q8_STEPS_FULL = 16;
constexpr int Q8_STEPS_REINDEX = 4;

template <bool REINDEX, bool FP4K>
__global__ __launch_bounds__(Q8_THREADS) void index_score_q8_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales,
    const float* __restrict__ w, const uint8_t* __restrict__ k_codes,
    const uint8_t* __restrict__ k_scales, int64_t n_entries, const int64_t* __restrict__ kv_start,
    const int32_t* __restrict__ n_visible, const int32_t* __restrict__ pool_blocks, int n_pool,
    float* __restrict__ scores, int64_t ld, float* __restrict__ block_max, int64_t ld_bm) {
  constexpr int Q8_STEPS = REINDEX ? Q8_STEPS_REINDEX : Q8_STEPS_FULL;
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 31;
  const int half = lane >> 5;

  // A operands (head n) and their scale bytes for the two MFMAs.
  i32x8 a[2];
  uint32_t sa[2];
  {
    const uint8_t* qrow = q_codes + ((int64_t)t * 32 + n) * 128;
    const uint32_t qs = *reinterpret_cast<const uint32_t*>(q_scales + ((int64_t)t * 32 + n) * 4);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(qrow + 64 * i + 16 * half);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(qrow + 64 * i + 32 + 16 * half);
      a[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      sa[i] = (qs >> (8 * (2 * i + half))) & 0xFFu;
    }
  }
  float wr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) wr[r] = w[(int64_t)t * 32 + 8 * (r >> 2) + 4 * half + (r & 3)];

  const int64_t base = kv_start[t];
  const int64_t nv = n_visible[t];
  constexpr int TILE = (Q8_THREADS / 64) * Q8_STEPS * 32;
  const int64_t tile0 = (int64_t)blockIdx.x * TILE + (int64_t)wave * 32;
  auto slot_at = [&](int step) -> int64_t {
    return tile0 + (int64_t)step * (Q8_THREADS / 64) * 32 + n;
  };
  // The cache row of this lane's slot in a step, -1 when absent; Reindex slots map
  // through the pool (slot s is position 8 * pool[s / 8] + s % 8).
  auto row_of = [&](int step) -> int64_t {
    const int64_t slot = slot_at(step);
    if (slot >= ld) return -1;
    int64_t pos = slot;
    if (REINDEX) {
      const int64_t pb = slot >> 3;
      const int b = pb < n_pool ? pool_blocks[(int64_t)t * n_pool + pb] : -1;
      if (b < 0) return -1;
      pos = (int64_t)b * 8 + (slot & 7);
    }
    if (pos >= nv) return -1;
    const int64_t row = base + pos;
    return (row >= 0 && row < n_entries) ? row : -1;
  };
  int64_t rows[Q8_STEPS];
#pragma unroll
  for (int st = 0; st < Q8_STEPS; ++st) rows[st] = row_of(st);
  auto row_at = [&](int step) -> int64_t { return rows[step]; };
  bool any = nv > 0 && base >= 0 && base < n_entries;
  if (REINDEX) {
    // A wavefront whose slots are all absent (past a compacted candidate list) loads and
    // multiplies nothing; its slots score -inf.
    bool mine = false;
#pragma unroll
    for (int st = 0; st < Q8_STEPS; ++st) mine |= rows[st] >= 0;
    any = any && __ballot(mine) != 0ull;
  }
  // Per step and lane, MXFP4: code bytes 16h .. +15 and 32 + 16h .. +15 of its row and the
  // scale word; E4M3: bytes 64i + 16h .. +15 and 64i + 32 + 16h .. +15 for i = 0, 1.
  constexpr int NKB = FP4K ? 2 : 4;
  u32x4 kb[2][NKB];
  uint32_t ks[2];
  auto load_step = [&](int step, int b) {
    const int64_t r = row_at(step);
    const int64_t rr = r >= 0 ? r : base;
    if constexpr (FP4K) {
      const uint8_t* row = k_codes + rr * 64;
      kb[b][0] = *reinterpret_cast<const u32x4*>(row + 16 * half);
      kb[b][1] = *reinterpret_cast<const u32x4*>(row + 32 + 16 * half);
      ks[b] = *reinterpret_cast<const uint32_t*>(k_scales + rr * 4);
    } else {
      const uint8_t* row = k_codes + rr * 128;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        kb[b][2 * i] = *reinterpret_cast<const u32x4*>(row + 64 * i + 16 * half);
        kb[b][2 * i + 1] = *reinterpret_cast<const u32x4*>(row + 64 * i + 32 + 16 * half);
      }
      ks[b] = 0x7F7F7F7Fu;
    }
  };
  float sc[Q8_STEPS];
  if (any) load_step(0, 0);
#pragma unroll
  for (int step = 0; step < Q8_STEPS; ++step) {
    float sv = -__builtin_inff();
    if (any) {
      const int b = step & 1;
      if (step + 1 < Q8_STEPS) load_step(step + 1, b ^ 1);
      f32x16 acc = {};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t sb = (ks[b] >> (8 * (2 * i + half))) & 0xFFu;
        if constexpr (FP4K) {
          const u32x4 c = kb[b][i];
          const i32x8 bv = i32x8{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
          // A format 0 (fp8 E4M3), B format 4 (fp4 E2M1)
          acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], bv, acc, 0, 4, 0,
                                                                (int)sa[i], 0, (int)sb);
        } else {
          const u32x4 c0 = kb[b][2 * i], c1 = kb[b][2 * i + 1];
          const i32x8 bv = i32x8{(int)c0.x, (int)c0.y, (int)c0.z, (int)c0.w,
                                 (int)c1.x, (int)c1.y, (int)c1.z, (int)c1.w};
          // A and B format 0 (fp8 E4M3)
          acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], bv, acc, 0, 0, 0,
                                                                (int)sa[i], 0, (int)sb);
        }
      }
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) part += wr[r] * fmaxf(acc[r], 0.f);
      part += __shfl_xor(part, 32);
      if (row_at(step) >= 0) sv = part;
    }
    sc[step] = sv;
  }
#pragma unroll
  for (int step = 0; step < Q8_STEPS; ++step) {
    const int64_t slot = slot_at(step);
    const float sv = sc[step];
    if (scores != nullptr && slot < ld && half == 0) scores[(int64_t)t * ld + slot] = sv;
    if (block_max != nullptr) {
      float m = sv;
      m = fmaxf(m, __shfl_xor(m, 1));
      m = fmaxf(m, __shfl_xor(m, 2));
      m = fmaxf(m, __shfl_xor(m, 4));
      if (half == 0 && (n & 7) == 0 && slot < ld) block_max[(int64_t)t * ld_bm + (slot >> 3)] = m;
    }
  }
}

// Queries that share one sequence (chunked prefill), MXFP8 query over E4M3 keys: a
// workgroup scores SQ8_QT queries (four per wavefront, operands and scales in registers)
// against one 4,096-row tile. Per 32-row step each wavefront loads one 16-byte quarter of
// every row's B operand straight into an LDS buffer in operand order (the keys need no
// conversion: the matrix core takes the E4M3 bytes), one barrier per step, then every
// wavefront reads the step's two operands and runs its queries' two MFMAs each. The
// products and their order are those of index_score_q8_kernel: identical scores.
constexpr int SQ8_QW = 4;
constexpr int SQ8_QT = (Q8_THREADS / 64) * SQ8_QW;
constexpr int SQ8_TILE = 4096;
constexpr int SQ8_PF = 16;   // steps whose rows are in flight (they come mostly from cache)

__global__ __launch_bounds__(Q8_THREADS) void index_score_shared_q8_kernel(
    int n_q, const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales,
    const float* __restrict__ w, const uint8_t* __restrict__ k_cache, int64_t n_entries,
    int64_t kv_start, const int32_t* __restrict__ n_visible, float* __restrict__ scores,
    int64_t ld, float* __restrict__ block_max, int64_t ld_bm) {
  // bsh[buf][2i + part][lane]: bytes 64i + 32 part + 16h .. +15 of row lane % 32
  __shared__ u32x4 bsh[2][4][64];
  __shared__ int nv_sh[SQ8_QT];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int half = lane >> 5;
  const int t0 = blockIdx.y * SQ8_QT;

  i32x8 a[SQ8_QW][2];
  uint32_t sa[SQ8_QW][2];
  float wr[SQ8_QW][16];
  int nvq[SQ8_QW];
#pragma unroll
  for (int j = 0; j < SQ8_QW; ++j) {
    const int t = t0 + SQ8_QW * wave + j;
    const bool ok = t < n_q;
    const int64_t tq = ok ? t : 0;
    const uint8_t* qrow = q_codes + (tq * 32 + n) * 128;
    const uint32_t qs = *reinterpret_cast<const uint32_t*>(q_scales + (tq * 32 + n) * 4);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(qrow + 64 * i + 16 * half);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(qrow + 64 * i + 32 + 16 * half);
      a[j][i] = ok ? i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                           (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w}
                   : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      sa[j][i] = (qs >> (8 * (2 * i + half))) & 0xFFu;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
      wr[j][r] = ok ? w[tq * 32 + 8 * (r >> 2) + 4 * half + (r & 3)] : 0.f;
    nvq[j] = ok ? n_visible[t] : 0;
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < SQ8_QW; ++j) nv_sh[SQ8_QW * wave + j] = nvq[j];
  }
  __syncthreads();
  int nv_max = 0;
#pragma unroll
  for (int q = 0; q < SQ8_QT; ++q) nv_max = max(nv_max, nv_sh[q]);

  const int64_t tile0 = (int64_t)blockIdx.x * SQ8_TILE;
  constexpr int STEPS = SQ8_TILE / 32;
  const bool any = nv_max > 0 && kv_start >= 0 && kv_start < n_entries;
  auto row_at = [&](int step) -> int64_t {
    const int64_t slot = tile0 + (int64_t)step * 32 + n;
    if (slot >= ld || slot >= nv_max) return -1;
    const int64_t row = kv_start + slot;
    return (row >= 0 && row < n_entries) ? row : -1;
  };
  // wavefront w loads operand part (w % 2) of MFMA w / 2: bytes 64(w/2) + 32(w%2) + 16h .. +15
  const int boff = 64 * (wave >> 1) + 32 * (wave & 1) + 16 * half;
  u32x4 raw[SQ8_PF];
  auto load = [&](int step) -> u32x4 {
    const int64_t r = row_at(step);
    return *reinterpret_cast<const u32x4*>(k_cache + (r >= 0 ? r : kv_start) * 128 + boff);
  };
  if (any) {
#pragma unroll
    for (int i = 0; i < SQ8_PF; ++i) raw[i] = load(i);
  }
#pragma unroll 1
  for (int step0 = 0; step0 < STEPS; step0 += SQ8_PF) {
#pragma unroll
    for (int i = 0; i < SQ8_PF; ++i) {
      const int step = step0 + i;
      const int buf = step & 1;
      const int64_t slot = tile0 + (int64_t)step * 32 + n;
      const bool row_ok = any && row_at(step) >= 0;
      if (any) {
        bsh[buf][wave][lane] = raw[i];
        if (step + SQ8_PF < STEPS) raw[i] = load(step + SQ8_PF);
      }
      __syncthreads();
      i32x8 b[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const u32x4 lo = bsh[buf][2 * m][lane], hi = bsh[buf][2 * m + 1][lane];
        b[m] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < SQ8_QW; ++j) {
        const int t = t0 + SQ8_QW * wave + j;
        float sv = -__builtin_inff();
        if (any) {
          f32x16 acc = {};
#pragma unroll
          for (int m = 0; m < 2; ++m)
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j][m], b[m], acc, 0, 0, 0,
                                                                  (int)sa[j][m], 0, 127);
          float part = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) part += wr[j][r] * fmaxf(acc[r], 0.f);
          part += __shfl_xor(part, 32);
          if (row_ok && slot < nvq[j]) sv = part;
        }
        if (t < n_q && slot < ld && half == 0) scores[(int64_t)t * ld + slot] = sv;
        if (block_max != nullptr) {
          float mm = sv;
          mm = fmaxf(mm, __shfl_xor(mm, 1));
          mm = fmaxf(mm, __shfl_xor(mm, 2));
          mm = fmaxf(mm, __shfl_xor(mm, 4));
          if (t < n_q && half == 0 && (n & 7) == 0 && slot < ld)
            block_max[(int64_t)t * ld_bm + (slot >> 3)] = mm;
        }
      }
    }
  }
}

hipError_t launch_index_score_shared_q8(int n_q, const uint8_t* q_codes, const uint8_t* q_scales,
                                        const float* w, const uint8_t* k_cache,
                                        int64_t n_entries, int64_t kv_start,
                                        const int32_t* n_visible, float* scores, int64_t ld,
                                        float* block_max, int64_t ld_bm, hipStream_t stream) {
  dim3 grid((unsigned)((ld + SQ8_TILE - 1) / SQ8_TILE), (unsigned)((n_q + SQ8_QT - 1) / SQ8_QT));
  hipLaunchKernelGGL(index_score_shared_q8_kernel, grid, dim3(Q8_THREADS), 0, stream, n_q,
                     q_codes, q_scales, w, k_cache, n_entries, kv_start, n_visible, scores, ld,
                     block_max, ld_bm);
  return hipGetLastError();
}

// MXFP8 quantisation of bf16 rows of 128 channels (the OCP microscaling recipe): per 32
// channels the exponent X = floor(log2 amax) - 8 (8 = E4M3's largest exponent), stored
// as X + 127 kept in 1..254 (127 for an all-zero group), codes E4M3(x * 2^-X), nearest
// even, saturating at 448. 16 lanes per row, lane c channels 8c .. 8c+7.
__global__ __launch_bounds__(Q8_THREADS) void mxfp8_quantize_kernel(
    int n_rows, const uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  const int64_t gid = (int64_t)blockIdx.x * Q8_THREADS + threadIdx.x;
  const int64_t r = gid >> 4;
  const int c = (int)(gid & 15);
  // Every lane takes part in the shuffles; rows past n_rows only skip the stores.
  float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (r < n_rows) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(x + r * 128 + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  // floor(log2 amax) is the exponent field minus 127 (a subnormal amax gives a field of 0
  // and clamps to scale byte 1 either way); bf16 inputs keep the byte within 1..246
  int code_s = 127;
  if (amax > 0.f) {
    code_s = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 8;
    code_s = code_s < 1 ? 1 : (code_s > 254 ? 254 : code_s);
  }
  // 2^(127 - code_s) as a float (exponent field 254 - code_s, in 8 .. 253 for bytes up to
  // 246): multiplying by it is exact, as ldexpf would be
  const float inv = __uint_as_float((uint32_t)(254 - code_s) << 23);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= f32_to_e4m3_rne(f[i] * inv) << (8 * i);
    hi |= f32_to_e4m3_rne(f[4 + i] * inv) << (8 * i);
  }
  if (r >= n_rows) return;
  *reinterpret_cast<u32x2*>(codes + r * 128 + 8 * c) = u32x2{lo, hi};
  if ((c & 3) == 0) scales[r * 4 + (c >> 2)] = (uint8_t)code_s;
}

hipError_t launch_index_score_q8(bool reindex, bool fp4k, int n_q, const uint8_t* q_codes,
                                 const uint8_t* q_scales, const float* w, const uint8_t* k_codes,
                                 const uint8_t* k_scales, int64_t n_entries,
                                 const int64_t* kv_start, const int32_t* n_visible,
                                 const int32_t* pool_blocks, int n_pool, float* scores,
                                 int64_t ld, float* block_max, int64_t ld_bm,
                                 hipStream_t stream) {
  const int tile = (Q8_THREADS / 64) * (reindex ? Q8_STEPS_REINDEX : Q8_STEPS_FULL) * 32;
  dim3 grid((unsigned)((ld + tile - 1) / tile), (unsigned)n_q);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(Q8_THREADS), 0, stream, q_codes, q_scales, w, k_codes,
                       k_scales, n_entries, kv_start, n_visible, pool_blocks, n_pool, scores, ld,
                       block_max, ld_bm);
  };
  if (fp4k)
    reindex ? go(index_score_q8_kernel<true, true>) : go(index_score_q8_kernel<false, true>);
  else
    reindex ? go(index_score_q8_kernel<true, false>) : go(index_score_q8_kernel<false, false>);
  return hipGetLastError();
}

hipError_t launch_mxfp8_quantize(int n_rows, const uint16_t* x, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream) {
  const int64_t threads = (int64_t)n_rows * 16;
  hipLaunchKernelGGL(mxfp8_quantize_kernel,
                     dim3((unsigned)((threads + Q8_THREADS - 1) / Q8_THREADS)), dim3(Q8_THREADS),
                     0, stream, n_rows, x, codes, scales);
  return hipGetLastError();
}

}  // namespace csa2
