// Lightning-indexer score on gfx950 MFMA.
//
// Score of cache position j for query t (the indexer of "DeepSeek-v4.1 Flash: Pushing the
// Limits of KV Cache Compression", 2.3.1 and 3.3.2, with 32 indexer heads of dim 128 per
// "DeepSeek-V4.1-Flash - Architecture", section 2):
//     s[t,j] = sum_h w[t,h] * ReLU(q_idx[t,h,:] . k_idx[row(t,j),:])
//
// One wavefront scores 32 positions per step with eight v_mfma_f32_32x32x16_bf16: the
// 32 indexer heads are the M dimension, the 32 positions the N dimension and the 128
// channels the K dimension. Lane l (n = l%32, half = l/32) streams bytes
// [64*half, 64*half + 64) of row n straight from HBM (four 16-byte loads; a wave reads
// 32 whole rows = 4 KiB), converts the E4M3 bytes to bf16 in registers (exact) and feeds
// them as the B operand; the A operand holds q_idx with the same channel assignment, so
// the K-sum is the plain dot product. The 32x32 fp32 result sits in 16 registers per
// lane (row = 8*(r/4) + 4*half + r%4, column = l%32); ReLU, the per-head weight and the
// sum over heads happen in registers plus one cross-half shuffle. Scores and optional
// 8-slot block maxima are kept in registers and written with coalesced stores after the
// workgroup's rows have been read; a Full pass may write the block maxima alone (the 4-byte
// score stores cost about a tenth of the pass's time against 3% of its bytes).
//
// Indexer keys come in one of three formats: E4M3 rows of 128 bytes, MXFP4 rows (the
// OCP microscaling format the pages name for the indexer cache, "DeepSeek-v4.1 Flash:
// Pushing the Limits of KV Cache Compression", 2.4.4 and 3.1): 64 bytes of E2M1 codes
// (channel 2m in the low nibble of byte m) and 4 E8M0 scale bytes, one per 32 channels.
// An MXFP4 lane reads 32 bytes of codes (its 64 channels) and the row's scale word (a Full
// pass reads whole rows per lane instead, in index_score_full_wide_fp4_kernel below), and
// converts with the hardware E2M1 -> bf16 conversion whose scale operand is the E8M0
// scale as a power of two: exact while the products stay in bf16's normal range; or bf16
// rows of 256 bytes (the block-mean keys of the two-stage filter, fed to the MFMA as they
// are). Work per step is 8,192 flops per position against 128 bytes read (E4M3): HBM-bound
// at 64 flop/B.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

constexpr int IS_THREADS = 256;
// Steps of 32 slots per wave: a Full-layer workgroup scores 4 x 16 x 32 = 2,048 slots;
// a Reindex workgroup 512 (the pool is only 16,384 slots per query, so smaller tiles keep
// every CU busy).
constexpr int IS_STEPS_FULL = 16;
constexpr int IS_STEPS_REINDEX = 4;
constexpr int IS_PREFETCH = 1;   // steps whose rows are in flight while one is multiplied
constexpr int FULL_PF_STAGED = 2;   // the same for the Full E4M3 pass without a score row
constexpr int RE_PF = 1;           // the same for the coalesced E4M3 Reindex pass

// Indexer-key formats: E4M3 rows of 128 bytes, MXFP4 rows (64 code bytes + 4 E8M0 scale
// bytes in a separate array) and bf16 rows of 256 bytes (the block-mean keys of the
// two-stage filter).
enum { KF_E4M3 = 0, KF_MXFP4 = 1, KF_BF16 = 2 };

// Integer key of a float whose signed order is the float order (negative floats have their
// magnitude bits flipped); the map is its own inverse on the key.
__device__ __forceinline__ int order_key(float v) {
  const int k = __float_as_int(v);
  return k ^ ((k >> 31) & 0x7FFFFFFF);
}

// Largest key over each aligned group of 8 lanes, in every lane of the group: quad swaps of
// 1 and 2 lanes, then the mirror within 8 lanes (lane i reads lane 7 - i), as DPP moves.
__device__ __forceinline__ int group8_max_all(int k) {
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0xB1, 0xF, 0xF, false));
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0x4E, 0xF, 0xF, false));
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0x141, 0xF, 0xF, false));
  return k;
}

template <bool REINDEX, int KF>
__global__ __launch_bounds__(IS_THREADS) void index_score_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_cache, const uint8_t* __restrict__ k_scales, int64_t n_entries,
    const int64_t* __restrict__ kv_start, const int32_t* __restrict__ n_visible,
    const int32_t* __restrict__ pool_blocks, int n_pool,
    float* __restrict__ scores, int64_t ld, float* __restrict__ block_max, int64_t ld_bm) {
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 31;
  const int half = lane >> 5;

  // A operand: head n, channels 64*half + 8*kb + (0..7) for k-block kb.
  bf16x8 a[8];
  const uint16_t* qrow = q_idx + ((int64_t)t * 32 + n) * 128 + 64 * half;
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) a[kb] = *reinterpret_cast<const bf16x8*>(qrow + 8 * kb);
  float wr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) wr[r] = w[(int64_t)t * 32 + 8 * (r >> 2) + 4 * half + (r & 3)];

  const int64_t base = kv_start[t];
  const int64_t nv = n_visible[t];
  constexpr int IS_STEPS_PER_WAVE = REINDEX ? IS_STEPS_REINDEX : IS_STEPS_FULL;
  constexpr int IS_TILE = (IS_THREADS / 64) * IS_STEPS_PER_WAVE * 32;
  const int64_t tile0 = (int64_t)blockIdx.x * IS_TILE + (int64_t)wave * 32;

  // Resolve the cache row of this lane's slot for a step; -1 when absent.
  auto row_of = [&](int step, int64_t& slot) -> int64_t {
    slot = tile0 + (int64_t)step * (IS_THREADS / 64) * 32 + n;
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
  // Rows are loaded unconditionally (an absent slot loads the query's first row, which
  // exists, and is masked afterwards) into buffers that rotate over the unrolled steps, so
  // no load waits on another. A query with no visible row in the cache loads nothing.
  // Reindex rows come through the pool and are resolved before streaming.
  constexpr int NB = IS_PREFETCH + 1;
  bool any = nv > 0 && base >= 0 && base < n_entries;
  int64_t rows[REINDEX ? IS_STEPS_PER_WAVE : 1];
  int64_t slots_unused;
  if (REINDEX) {
    bool mine = false;
#pragma unroll
    for (int st = 0; st < IS_STEPS_PER_WAVE; ++st) {
      rows[st] = row_of(st, slots_unused);
      mine |= rows[st] >= 0;
    }
    // A wavefront whose slots are all absent (past a compacted candidate list) loads and
    // multiplies nothing; its slots score -inf.
    any = any && __ballot(mine) != 0ull;
  }
  auto row_at = [&](int step) -> int64_t {
    int64_t sl;
    return REINDEX ? rows[REINDEX ? step : 0] : row_of(step, sl);
  };
  auto slot_at = [&](int step) -> int64_t { return tile0 + (int64_t)step * (IS_THREADS / 64) * 32 + n; };
  // E4M3: raw[0..3] = bytes 64*half .. +63 of the row. MXFP4: raw[0..1] = code bytes
  // 32*half .. +31 (channels 64*half .. +63) and raw[2].x = the row's four scale bytes.
  // bf16: raw[0..7] = channels 64*half .. +63.
  constexpr int NR = KF == KF_BF16 ? 8 : 4;
  u32x4 buf[NB][NR];
  float sc[IS_STEPS_PER_WAVE];
  auto load_step = [&](int step, u32x4 (&raw)[NR]) {
    const int64_t r = row_at(step);
    const int64_t rr = r >= 0 ? r : base;
    if constexpr (KF == KF_BF16) {
      const u32x4* p = reinterpret_cast<const u32x4*>(k_cache + rr * 256 + 128 * half);
#pragma unroll
      for (int i = 0; i < 8; ++i) raw[i] = p[i];
    } else if constexpr (KF == KF_MXFP4) {
      const u32x4* p = reinterpret_cast<const u32x4*>(k_cache + rr * 64 + 32 * half);
      raw[0] = p[0];
      raw[1] = p[1];
      raw[2].x = *reinterpret_cast<const uint32_t*>(k_scales + rr * 4);
    } else {
      const u32x4* p = reinterpret_cast<const u32x4*>(k_cache + rr * 128 + 64 * half);
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[i] = p[i];
    }
  };
  if (any) {
#pragma unroll
    for (int st = 0; st < IS_PREFETCH && st < IS_STEPS_PER_WAVE; ++st) load_step(st, buf[st % NB]);
  }
#pragma unroll
  for (int step = 0; step < IS_STEPS_PER_WAVE; ++step) {
    float sv = -__builtin_inff();
    if (any) {
      if (step + IS_PREFETCH < IS_STEPS_PER_WAVE)
        load_step(step + IS_PREFETCH, buf[(step + IS_PREFETCH) % NB]);
      u32x4 (&raw)[NR] = buf[step % NB];
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        u32x4 bv;
        if constexpr (KF == KF_BF16) {
          bv = raw[kb];
        } else if constexpr (KF == KF_MXFP4) {
          // channels 64*half + 8*kb .. +7: code dword kb, scale group 2*half + kb/4
          const uint32_t d = raw[kb >> 2][kb & 3];
          const uint32_t e = (raw[2].x >> (8 * (2 * half + (kb >> 2)))) & 0xFFu;
          bv = fp4x8_to_bf16x8_pow2(d, __uint_as_float(e << 23));
        } else {
          const u32x2 lo = e4m3x4_to_bf16x4(raw[kb >> 1][(kb & 1) * 2]);
          const u32x2 hi = e4m3x4_to_bf16x4(raw[kb >> 1][(kb & 1) * 2 + 1]);
          bv = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], __builtin_bit_cast(bf16x8, bv), acc,
                                                      0, 0, 0);
      }
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) part += wr[r] * fmaxf(acc[r], 0.f);
      part += __shfl_xor(part, 32);
      if (row_at(step) >= 0) sv = part;
    }
    sc[step] = sv;
  }
  // Scores and block maxima go out once the tile has been streamed: small stores
  // interleaved with the row reads cost read bandwidth.
#pragma unroll
  for (int step = 0; step < IS_STEPS_PER_WAVE; ++step) {
    const int64_t slot = slot_at(step);
    const float sv = sc[step];
    if (scores != nullptr && slot < ld && half == 0) scores[(int64_t)t * ld + slot] = sv;
    if (block_max != nullptr) {
      float m = sv;
      m = fmaxf(m, __shfl_xor(m, 1));
      m = fmaxf(m, __shfl_xor(m, 2));
      m = fmaxf(m, __shfl_xor(m, 4));
      if (half == 0 && (n & 7) == 0 && slot < ld)
        block_max[(int64_t)t * ld_bm + (slot >> 3)] = m;
    }
  }
}


// Full-mode scoring of E4M3 keys with coalesced row loads. A wavefront step still covers
// 32 consecutive slots (4 KiB of rows), but each load instruction reads 1 KiB of them
// contiguously: instruction i gives lane l the 16 bytes 16*(l%8) .. +15 of row 8i + l/8.
// The pieces go through a per-wavefront LDS buffer (piece c of row r at r*128 +
// ((c ^ (r%8)) * 16): eight lanes writing one row, or reading one piece of eight rows,
// cover all banks) and come back as the operand layout of index_score_kernel: lane (n,
// half) holds bytes 64*half .. +63 of row n. Conversion, products, their order and the
// epilogue are that kernel's, so every score is bit-identical to it (and to the Reindex
// form, which rescoring relies on). The row loads run one step ahead.
// Four wavefronts per SIMD (128 registers each) keep enough rows in flight.
template <int MODE>
__global__ __launch_bounds__(IS_THREADS) void index_score_full_e4m3_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_cache, int64_t n_entries, const int64_t* __restrict__ kv_start,
    const int32_t* __restrict__ n_visible, float* __restrict__ scores, int64_t ld,
    float* __restrict__ block_max, int64_t ld_bm, uint32_t* __restrict__ block_aux) {
  __shared__ u32x4 stage[IS_THREADS / 64][2][256];   // 8 KiB per wavefront
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 31;
  const int half = lane >> 5;
  bf16x8 a[8];
  const uint16_t* qrow = q_idx + ((int64_t)t * 32 + n) * 128 + 64 * half;
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) a[kb] = *reinterpret_cast<const bf16x8*>(qrow + 8 * kb);
  float wr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) wr[r] = w[(int64_t)t * 32 + 8 * (r >> 2) + 4 * half + (r & 3)];
  const int64_t base = kv_start[t];
  const int64_t nv = n_visible[t];
  constexpr int STEPS = IS_STEPS_FULL;
  constexpr int TILE = (IS_THREADS / 64) * STEPS * 32;
  const int64_t tile0 = (int64_t)blockIdx.x * TILE + (int64_t)wave * 32;
  const bool any = nv > 0 && base >= 0 && base < n_entries;
  // Slots below `lim` have a row (visible, inside the row width and the cache); an absent
  // row's piece is read from row `base`, which exists, and masked.
  int64_t lim = ld < nv ? ld : nv;
  if (any && n_entries - base < lim) lim = n_entries - base;
  auto slot_at = [&](int step) -> int64_t { return tile0 + (int64_t)step * (IS_THREADS / 64) * 32 + n; };
  const int piece = lane & 7;
  auto load_step = [&](int step, u32x4 (&g)[4]) {
    const int64_t s0 = tile0 + (int64_t)step * (IS_THREADS / 64) * 32 + (lane >> 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t slot = s0 + 8 * i;
      g[i] = *reinterpret_cast<const u32x4*>(k_cache + (base + (slot < lim ? slot : 0)) * 128 +
                                             16 * piece);
    }
  };
  // Rows of PF steps are in flight while a step is multiplied (more for the staged modes,
  // which keep no score array).
  constexpr int PF = MODE != 0 ? FULL_PF_STAGED : 1;
  u32x4 g[PF][4];
  // MODE 0: scores and maxima go out after the tile (the score row is the bulk of the
  // writes); MODE 1: block maxima only, reduced as each step completes and staged in LDS;
  // MODE 2: as 1, plus the block statistics (scores, if asked, stored as each step ends).
  constexpr bool AUX = MODE == 2;
  constexpr bool STAGED = MODE != 0;
  float sc[STAGED ? 1 : STEPS];
  float sv_prev = 0.f;   // statistics: the previous step's score
  static_assert(STEPS % 2 == 0, "block statistics pair the steps");
  __shared__ float bm_st[STAGED ? TILE / 8 : 1];    // block maxima of the tile
  __shared__ uint32_t aux_st[AUX ? TILE / 8 : 1];   // block statistics of the tile
  if (any) {
#pragma unroll
    for (int p0 = 0; p0 < PF; ++p0) load_step(p0, g[p0]);
  }
#pragma unroll
  for (int step = 0; step < STEPS; ++step) {
    float sv = -__builtin_inff();
    if (any) {
      u32x4* buf = stage[wave][step & 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + (lane >> 3);
        buf[r * 8 + (piece ^ (r & 7))] = g[step % PF][i];
      }
      if (step + PF < STEPS) load_step(step + PF, g[step % PF]);
      // LDS operations of one wavefront complete in order; the fences keep the compiler
      // from moving the reads above the writes.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      u32x4 raw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[i] = buf[n * 8 + ((4 * half + i) ^ (n & 7))];
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const u32x2 lo = e4m3x4_to_bf16x4(raw[kb >> 1][(kb & 1) * 2]);
        const u32x2 hi = e4m3x4_to_bf16x4(raw[kb >> 1][(kb & 1) * 2 + 1]);
        const u32x4 bv = u32x4{lo.x, lo.y, hi.x, hi.y};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], __builtin_bit_cast(bf16x8, bv), acc,
                                                      0, 0, 0);
      }
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) part += wr[r] * fmaxf(acc[r], 0.f);
      part += __shfl_xor(part, 32);
      if (slot_at(step) < lim) sv = part;
    }
    if constexpr (MODE == 1) {
      // Block maxima as each step completes, two steps at a time (both half-waves hold every
      // score of a step: half 0 takes the previous step's slots, half 1 this step's), on
      // integer keys whose signed order is the float order with DPP lane moves (equal to the
      // fmaxf reduction: scores are never -0).
      if (step & 1) {
        const int m = group8_max_all(order_key(half ? sv : sv_prev));
        if ((n & 7) == 0)
          bm_st[16 * (step - 1 + half) + 4 * wave + (n >> 3)] =
              __int_as_float(m ^ ((m >> 31) & 0x7FFFFFFF));
      } else {
        sv_prev = sv;
      }
    } else if constexpr (AUX) {
      // Block statistics, two steps at a time (both half-waves hold every score of a step,
      // so half 0 takes the previous step's slots and half 1 this step's; no score array is
      // kept): on integer keys whose signed order is the float order, with DPP lane moves,
      // every lane of a block gets its maximum (equal to the fmaxf reduction: scores are
      // never -0); the argmax is the lowest lane holding it (a ballot), the second key the
      // largest of the others.
      const int64_t slot = slot_at(step);
      if (scores != nullptr && slot < ld && half == 0) scores[(int64_t)t * ld + slot] = sv;
      if (step & 1) {
        const int k = order_key(half ? sv : sv_prev);
        const int m = group8_max_all(k);
        const uint64_t hit = __ballot(k == m);
        const uint32_t am = (uint32_t)__builtin_ctzll((hit >> (lane & 56)) | 0x100ull);
        const int k2 = group8_max_all((uint32_t)(n & 7) == am ? INT32_MIN : k);
        const uint32_t key2 = k2 <= order_key(-__builtin_inff()) ? 0u : (uint32_t)k2 ^ 0x80000000u;
        if ((n & 7) == 0) {
          const int blk = 16 * (step - 1 + half) + 4 * wave + (n >> 3);
          bm_st[blk] = __int_as_float(m ^ ((m >> 31) & 0x7FFFFFFF));
          aux_st[blk] = block_aux_word(key2, am);
        }
      } else {
        sv_prev = sv;
      }
    } else {
      sc[step] = sv;
    }
  }
  if constexpr (STAGED) {
    // one coalesced store per thread: thread i writes block i of the tile (small stores
    // after every step measured slower)
    __syncthreads();
    const int64_t b = (int64_t)blockIdx.x * (TILE / 8) + threadIdx.x;
    if (threadIdx.x < TILE / 8 && b * 8 < ld) {
      block_max[(int64_t)t * ld_bm + b] = bm_st[threadIdx.x];
      if constexpr (AUX) block_aux[(int64_t)t * ld_bm + b] = aux_st[threadIdx.x];
    }
    return;
  }
#pragma unroll
  for (int step = 0; step < STEPS; ++step) {
    const int64_t slot = slot_at(step);
    const float sv = sc[STAGED ? 0 : step];
    if (scores != nullptr && slot < ld && half == 0) scores[(int64_t)t * ld + slot] = sv;
    if (block_max != nullptr) {
      float m = sv;
      m = fmaxf(m, __shfl_xor(m, 1));
      m = fmaxf(m, __shfl_xor(m, 2));
      m = fmaxf(m, __shfl_xor(m, 4));
      if (half == 0 && (n & 7) == 0 && slot < ld)
        block_max[(int64_t)t * ld_bm + (slot >> 3)] = m;
    }
  }
}


// Reindex-mode scoring of E4M3 keys with coalesced row loads. A pool block is eight
// consecutive cache rows (1 KiB), and a wavefront step covers 32 slots, i.e. four pool
// blocks: load instruction i reads block i of the step whole (lane l: the 16 bytes
// 16*(l%8) .. +15 of the block's row l/8), and the pieces go through the per-wavefront LDS
// buffer of index_score_full_e4m3_kernel into index_score_kernel's operand layout. The
// block ids are wavefront-uniform, so a step whose four blocks are all absent (a compacted
// candidate list's -1 tail) loads and multiplies nothing. Conversion, products, their
// order and the epilogue are index_score_kernel's: identical scores. Rows of PF steps are
// in flight while a step is multiplied; scores and block maxima go out after the tile.
template <int STEPS, int PF>
__global__ __launch_bounds__(IS_THREADS) void index_score_reindex_e4m3_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_cache, int64_t n_entries, const int64_t* __restrict__ kv_start,
    const int32_t* __restrict__ n_visible, const int32_t* __restrict__ pool_blocks, int n_pool,
    float* __restrict__ scores, int64_t ld, float* __restrict__ block_max, int64_t ld_bm) {
  static_assert(PF >= 1 && PF <= STEPS, "prefetch depth");
  __shared__ u32x4 stage[IS_THREADS / 64][2][256];   // 8 KiB per wavefront
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int half = lane >> 5;
  bf16x8 a[8];
  const uint16_t* qrow = q_idx + ((int64_t)t * 32 + n) * 128 + 64 * half;
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) a[kb] = *reinterpret_cast<const bf16x8*>(qrow + 8 * kb);
  float wr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) wr[r] = w[(int64_t)t * 32 + 8 * (r >> 2) + 4 * half + (r & 3)];
  const int64_t base = kv_start[t];
  const int64_t nv = n_visible[t];
  constexpr int TILE = (IS_THREADS / 64) * STEPS * 32;
  const int64_t tile0 = (int64_t)blockIdx.x * TILE + (int64_t)wave * 32;
  const bool any = nv > 0 && base >= 0 && base < n_entries;
  // A slot has a row when its position is below lim (visible and inside the cache).
  int64_t lim = nv;
  if (any && n_entries - base < lim) lim = n_entries - base;
  // Block ids of each step's four blocks (-1: absent), the same in every lane.
  int bid[STEPS][4];
  bool live[STEPS];
#pragma unroll
  for (int step = 0; step < STEPS; ++step) {
    const int64_t pb0 = (tile0 + (int64_t)step * (IS_THREADS / 64) * 32) >> 3;
    bool l = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t pb = pb0 + i;
      const int b = pb < n_pool ? pool_blocks[(int64_t)t * n_pool + pb] : -1;
      bid[step][i] = b;
      l |= b >= 0;
    }
    live[step] = any && l;
  }
  auto slot_at = [&](int step) -> int64_t {
    return tile0 + (int64_t)step * (IS_THREADS / 64) * 32 + n;
  };
  const int piece = lane & 7;
  const int rin = lane >> 3;   // row of the block this lane loads
  auto load_step = [&](int step, u32x4 (&g)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = bid[step][i];
      const int64_t pos = (int64_t)b * 8 + rin;
      const bool ok = b >= 0 && pos < lim;
      g[i] = *reinterpret_cast<const u32x4*>(k_cache + (base + (ok ? pos : 0)) * 128 +
                                             16 * piece);
    }
  };
  u32x4 g[PF][4];
  float sc[STEPS];
#pragma unroll
  for (int p0 = 0; p0 < PF; ++p0)
    if (live[p0]) load_step(p0, g[p0]);
#pragma unroll
  for (int step = 0; step < STEPS; ++step) {
    float sv = -__builtin_inff();
    if (live[step]) {
      u32x4* buf = stage[wave][step & 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + rin;
        buf[r * 8 + (piece ^ (r & 7))] = g[step % PF][i];
      }
      if (step + PF < STEPS && live[step + PF]) load_step(step + PF, g[step % PF]);
      // LDS operations of one wavefront complete in order; the fences keep the compiler
      // from moving the reads above the writes.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      u32x4 raw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[i] = buf[n * 8 + ((4 * half + i) ^ (n & 7))];
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const u32x2 lo = e4m3x4_to_bf16x4(raw[kb >> 1][(kb & 1) * 2]);
        const u32x2 hi = e4m3x4_to_bf16x4(raw[kb >> 1][(kb & 1) * 2 + 1]);
        const u32x4 bv = u32x4{lo.x, lo.y, hi.x, hi.y};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], __builtin_bit_cast(bf16x8, bv), acc,
                                                      0, 0, 0);
      }
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) part += wr[r] * fmaxf(acc[r], 0.f);
      part += __shfl_xor(part, 32);
      const int j = n >> 3;
      const int b = j == 0 ? bid[step][0] : j == 1 ? bid[step][1] : j == 2 ? bid[step][2]
                                                                           : bid[step][3];
      if (b >= 0 && (int64_t)b * 8 + (n & 7) < lim) sv = part;
    } else if (step + PF < STEPS && live[step + PF]) {
      load_step(step + PF, g[step % PF]);
    }
    sc[step] = sv;
  }
#pragma unroll
  for (int step = 0; step < STEPS; ++step) {
    const int64_t slot = slot_at(step);
    const float sv = sc[step];
    if (scores != nullptr && slot < ld && half == 0) scores[(int64_t)t * ld + slot] = sv;
    if (block_max != nullptr) {
      float m = sv;
      m = fmaxf(m, __shfl_xor(m, 1));
      m = fmaxf(m, __shfl_xor(m, 2));
      m = fmaxf(m, __shfl_xor(m, 4));
      if (half == 0 && (n & 7) == 0 && slot < ld)
        block_max[(int64_t)t * ld_bm + (slot >> 3)] = m;
    }
  }
}

// Full-mode scoring of MXFP4 keys with whole rows per lane: a wavefront step covers 64
// slots, lane l loading row l of the step (its 64 code bytes as four 16-byte loads, and its
// scale word). The MFMA B operand wants, for columns n = 0..31, channels 8kb..+7 of row n in
// lane n and channels 64+8kb..+7 of row n in lane 32+n: one v_permlane32_swap per code
// dword exchanges the upper half-wave's low channels with the lower half-wave's high
// channels (and one swap of the scale word gives each lane the scales of the row it now
// holds), after which code dwords 0..7 are the operands of rows 0..31 and dwords 8..15
// those of rows 32..63. Twice the bytes per load instruction of index_score_kernel's MXFP4
// path and the same products in the same order: identical scores, about 10% faster.
// AUX: the block maxima and block statistics (as the E4M3 pass's mode 2 writes them) are
// reduced as each step completes, staged in LDS and written once per workgroup; scores, if
// asked, go out as each step ends.
constexpr int IW_STEPS = IS_STEPS_FULL / 2;   // 64-slot steps per wavefront (same tile)
constexpr int IW_PF = 3;                      // steps whose rows are in flight

template <bool AUX>
__global__ __launch_bounds__(IS_THREADS) void index_score_full_wide_fp4_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales, int64_t n_entries,
    const int64_t* __restrict__ kv_start, const int32_t* __restrict__ n_visible,
    float* __restrict__ scores, int64_t ld, float* __restrict__ block_max, int64_t ld_bm,
    uint32_t* __restrict__ block_aux) {
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 31;
  const int half = lane >> 5;
  bf16x8 a[8];
  const uint16_t* qrow = q_idx + ((int64_t)t * 32 + n) * 128 + 64 * half;
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) a[kb] = *reinterpret_cast<const bf16x8*>(qrow + 8 * kb);
  float wr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) wr[r] = w[(int64_t)t * 32 + 8 * (r >> 2) + 4 * half + (r & 3)];
  const int64_t base = kv_start[t];
  const int64_t nv = n_visible[t];
  constexpr int TILE = (IS_THREADS / 64) * IW_STEPS * 64;
  const int64_t tile0 = (int64_t)blockIdx.x * TILE + (int64_t)wave * 64;
  auto slot_at = [&](int step) -> int64_t {
    return tile0 + (int64_t)step * (IS_THREADS / 64) * 64 + lane;
  };
  auto row_at = [&](int step) -> int64_t {
    const int64_t slot = slot_at(step);
    if (slot >= ld || slot >= nv) return -1;
    const int64_t row = base + slot;
    return (row >= 0 && row < n_entries) ? row : -1;
  };
  const bool any = nv > 0 && base >= 0 && base < n_entries;
  constexpr int NB = IW_PF + 1;
  u32x4 buf[NB][4];
  uint32_t sbuf[NB];
  auto load_step = [&](int step, u32x4 (&raw)[4], uint32_t& sw) {
    const int64_t r = row_at(step);
    const int64_t rr = r >= 0 ? r : base;
    const u32x4* p = reinterpret_cast<const u32x4*>(k_codes + rr * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = p[i];
    sw = *reinterpret_cast<const uint32_t*>(k_scales + rr * 4);
  };
  float sc[AUX ? 1 : IW_STEPS];
  __shared__ float bm_st[AUX ? TILE / 8 : 1];       // block maxima of the tile
  __shared__ uint32_t aux_st[AUX ? TILE / 8 : 1];   // block statistics of the tile
  if (any) {
#pragma unroll
    for (int p0 = 0; p0 < IW_PF; ++p0) load_step(p0, buf[p0], sbuf[p0]);
  }
#pragma unroll
  for (int step = 0; step < IW_STEPS; ++step) {
    float sv = -__builtin_inff();
    if (any) {
      if (step + IW_PF < IW_STEPS)
        load_step(step + IW_PF, buf[(step + IW_PF) % NB], sbuf[(step + IW_PF) % NB]);
      u32x4 (&raw)[4] = buf[step % NB];
      // code dword d holds channels 8d .. 8d+7; dwords kb and 8+kb swap half-waves
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const auto s = __builtin_amdgcn_permlane32_swap(raw[d >> 2][d & 3],
                                                        raw[2 + (d >> 2)][d & 3], false, false);
        raw[d >> 2][d & 3] = s[0];
        raw[2 + (d >> 2)][d & 3] = s[1];
      }
      const auto ss = __builtin_amdgcn_permlane32_swap(sbuf[step % NB], sbuf[step % NB], false, false);
      const uint32_t scw[2] = {ss[0], ss[1]};
      float part[2];
#pragma unroll
      for (int set = 0; set < 2; ++set) {
        f32x16 acc = {};
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
          const int d = 8 * set + kb;
          const uint32_t code = raw[d >> 2][d & 3];
          const uint32_t e = (scw[set] >> (8 * (2 * half + (kb >> 2)))) & 0xFFu;
          const u32x4 bv = fp4x8_to_bf16x8_pow2(code, __uint_as_float(e << 23));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], __builtin_bit_cast(bf16x8, bv),
                                                        acc, 0, 0, 0);
        }
        float p = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) p += wr[r] * fmaxf(acc[r], 0.f);
        p += __shfl_xor(p, 32);
        part[set] = p;
      }
      // lane l owns slot l of the step: rows 0..31 are set 0, rows 32..63 set 1
      const float mine = half ? part[1] : part[0];
      if (row_at(step) >= 0) sv = mine;
    }
    if constexpr (AUX) {
      // The block of 8 consecutive slots lies in 8 consecutive lanes: maximum, argmax (the
      // lowest lane holding it) and the largest other key, on order-preserving integer
      // keys with DPP lane moves, as in the E4M3 pass.
      const int64_t slot = slot_at(step);
      if (scores != nullptr && slot < ld) scores[(int64_t)t * ld + slot] = sv;
      const int k = order_key(sv);
      const int m = group8_max_all(k);
      const uint64_t hit = __ballot(k == m);
      const uint32_t am = (uint32_t)__builtin_ctzll((hit >> (lane & 56)) | 0x100ull);
      const int k2 = group8_max_all((uint32_t)(lane & 7) == am ? INT32_MIN : k);
      const uint32_t key2 = k2 <= order_key(-__builtin_inff()) ? 0u : (uint32_t)k2 ^ 0x80000000u;
      if ((lane & 7) == 0) {
        const int blk = 32 * step + 8 * wave + (lane >> 3);
        bm_st[blk] = __int_as_float(m ^ ((m >> 31) & 0x7FFFFFFF));
        aux_st[blk] = block_aux_word(key2, am);
      }
    } else {
      sc[step] = sv;
    }
  }
  if constexpr (AUX) {
    // one coalesced store per thread: thread i writes block i of the tile
    __syncthreads();
    const int64_t b = (int64_t)blockIdx.x * (TILE / 8) + threadIdx.x;
    if (threadIdx.x < TILE / 8 && b * 8 < ld) {
      block_max[(int64_t)t * ld_bm + b] = bm_st[threadIdx.x];
      block_aux[(int64_t)t * ld_bm + b] = aux_st[threadIdx.x];
    }
    return;
  }
#pragma unroll
  for (int step = 0; step < IW_STEPS; ++step) {
    const int64_t slot = slot_at(step);
    const float sv = sc[AUX ? 0 : step];
    if (scores != nullptr && slot < ld) scores[(int64_t)t * ld + slot] = sv;
    if (block_max != nullptr) {
      float m = sv;
      m = fmaxf(m, __shfl_xor(m, 1));
      m = fmaxf(m, __shfl_xor(m, 2));
      m = fmaxf(m, __shfl_xor(m, 4));
      if ((lane & 7) == 0 && slot < ld) block_max[(int64_t)t * ld_bm + (slot >> 3)] = m;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Queries that share one sequence (chunked prefill: every query reads the same cache rows
// from kv_start, each up to its own causal n_visible). A workgroup scores SQ2_QT queries
// (SQ2_QW per wavefront, their MFMA operands and head weights held in registers) against
// one 4,096-row tile; rows are read and converted once per SQ2_QT queries.
// SS steps of 32 rows are staged per LDS buffer (double-buffered), so one barrier serves
// SS * QW * 8 products per wavefront. Wavefront w loads and converts k-blocks
// 2w and 2w+1 of every row of a stage (bytes 64*half + 16*w .. +15 of row n), one stage
// ahead of its use. Per step the QW product chains are issued one query after another, each
// together with the previous query's epilogue (ReLU, head weights, head sum, stores), so
// the epilogues run while products are in the matrix core; scheduling fences keep the
// compiler from merging the chains back into one interleaved block. Products, their order
// and the epilogue arithmetic are those of the per-query kernel: identical scores.
constexpr int SQ2_QW = 3;
constexpr int SQ2_SS = 4;
constexpr int SQ2_QT = (IS_THREADS / 64) * SQ2_QW;
constexpr int SQ2_TILE = 4096;

// max(x, 0) in one integer instruction: a float with the sign bit set (negative, or -0) is
// a negative integer and becomes +0, anything else is kept. For every finite x the value
// is fmaxf(x, 0) up to the sign of a zero, which leaves the weighted head sum unchanged.
__device__ __forceinline__ float relu1(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Largest of v over the 8 lanes of each aligned group of 8 (valid in each group's first
// lane): two quad exchanges and one rotation by 12 within a 16-lane row (lane i reads lane
// i + 4), taken on integer keys whose signed order is the float order (so the maxima need
// no NaN canonicalisation); equal to the fmaxf reduction for scores, which are never -0.
__device__ __forceinline__ float group8_max(float v) {
  int k = __float_as_int(v);
  k ^= (k >> 31) & 0x7FFFFFFF;
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0xB1, 0xF, 0xF, false));
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0x4E, 0xF, 0xF, false));
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0x12C, 0xF, 0xF, false));
  k ^= (k >> 31) & 0x7FFFFFFF;
  return __int_as_float(k);
}

template <int QW, int SS, bool BM>
__global__ __launch_bounds__(IS_THREADS, 2) void index_score_shared2_kernel(
    int n_q, const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint8_t* __restrict__ k_cache, int64_t n_entries, int64_t kv_start,
    const int32_t* __restrict__ n_visible, float* __restrict__ scores, int64_t ld,
    float* __restrict__ block_max, int64_t ld_bm) {
  constexpr int QT = (IS_THREADS / 64) * QW;
  __shared__ u32x4 bsh[2][SS][8][64];   // converted rows of a stage: step, k-block, lane
  __shared__ int nv_sh[QT];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int half = lane >> 5;
  const int t0 = blockIdx.y * QT;

  bf16x8 a[QW][8];
  float wr[QW][16];
  int nvq[QW];
#pragma unroll
  for (int j = 0; j < QW; ++j) {
    const int t = t0 + QW * wave + j;
    const bool ok = t < n_q;
    const uint16_t* qrow = q_idx + ((int64_t)(ok ? t : 0) * 32 + n) * 128 + 64 * half;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 8 * kb);
      a[j][kb] = ok ? v : bf16x8{};
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
      wr[j][r] = ok ? w[(int64_t)t * 32 + 8 * (r >> 2) + 4 * half + (r & 3)] : 0.f;
    nvq[j] = ok ? n_visible[t] : 0;
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < QW; ++j) nv_sh[QW * wave + j] = nvq[j];
  }
  __syncthreads();
  int nv_max = 0;
#pragma unroll
  for (int q = 0; q < QT; ++q) nv_max = max(nv_max, nv_sh[q]);

  const int64_t tile0 = (int64_t)blockIdx.x * SQ2_TILE;
  constexpr int STAGES = SQ2_TILE / (32 * SS);
  // Slots below lim have a row that some query of the group sees; each query masks its own.
  int64_t lim = ld < nv_max ? ld : nv_max;
  if (n_entries - kv_start < lim) lim = n_entries - kv_start;
  const bool any = nv_max > 0 && kv_start >= 0 && kv_start < n_entries && lim > tile0;
  // Stores through buffer descriptors over this tile's part of each query's score and
  // block-maximum rows: a lane with nothing to store (the upper half-wave, a lane that is
  // not first of its 8-slot block, a slot past the row or a query past n_q) uses an offset
  // past the descriptor's end, which the hardware drops, so no store is predicated.
  constexpr uint32_t DROP = 0xFFFFFFFFu;
  const int64_t tile_slots = ld - tile0 < SQ2_TILE ? ld - tile0 : SQ2_TILE;   // > 0
  __amdgpu_buffer_rsrc_t rs_s[QW], rs_b[QW];
#pragma unroll
  for (int j = 0; j < QW; ++j) {
    const int t = t0 + QW * wave + j;
    const bool ok = t < n_q;
    rs_s[j] = __builtin_amdgcn_make_buffer_rsrc(scores + (int64_t)(ok ? t : 0) * ld + tile0,
                                                (short)0, ok ? (int)(tile_slots * 4) : 0,
                                                0x00020000);
    rs_b[j] = __builtin_amdgcn_make_buffer_rsrc(
        block_max + (block_max != nullptr ? (int64_t)(ok ? t : 0) * ld_bm + (tile0 >> 3) : 0),
        (short)0, (ok && block_max != nullptr) ? (int)(((tile_slots + 7) >> 3) * 4) : 0,
        0x00020000);
  }
  auto store = [&](int j, int64_t slot, float sv) {
    const uint32_t rel = (uint32_t)(slot - tile0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sv), rs_s[j],
                                          half == 0 ? 4u * rel : DROP, 0, 0);
    if constexpr (BM) {
      const float m = group8_max(sv);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), rs_b[j],
                                            (half == 0 && (n & 7) == 0) ? 4u * (rel >> 3) : DROP,
                                            0, 0);
    }
  };
  if (!any) {   // no row of this tile is visible to the group: every slot scores -inf
    for (int step = 0; step < SQ2_TILE / 32; ++step)
#pragma unroll
      for (int j = 0; j < QW; ++j) store(j, tile0 + (int64_t)step * 32 + n, -__builtin_inff());
    return;
  }
  // Visible limits relative to the tile, clamped to [0, tile]: slot < x <=> rel < x_rel.
  auto rel_of = [&](int64_t x) -> int {
    const int64_t r = x - tile0;
    return r < 0 ? 0 : (r > SQ2_TILE ? SQ2_TILE : (int)r);
  };
  const int lim_rel = rel_of(lim);
  int nvq_rel[QW];
#pragma unroll
  for (int j = 0; j < QW; ++j) nvq_rel[j] = rel_of(nvq[j]);
  u32x4 raw[SS];
  auto load = [&](int stage) {
#pragma unroll
    for (int s = 0; s < SS; ++s) {
      const int64_t slot = tile0 + (int64_t)(stage * SS + s) * 32 + n;
      raw[s] = *reinterpret_cast<const u32x4*>(k_cache + (kv_start + (slot < lim ? slot : 0)) * 128 +
                                               64 * half + 16 * wave);
    }
  };
  load(0);
#pragma unroll 1
  for (int stage = 0; stage < STAGES; ++stage) {
    const int buf = stage & 1;
#pragma unroll
    for (int s = 0; s < SS; ++s) {
      const u32x4 v = raw[s];
      const u32x2 l0 = e4m3x4_to_bf16x4(v.x), h0 = e4m3x4_to_bf16x4(v.y);
      const u32x2 l1 = e4m3x4_to_bf16x4(v.z), h1 = e4m3x4_to_bf16x4(v.w);
      bsh[buf][s][2 * wave][lane] = u32x4{l0.x, l0.y, h0.x, h0.y};
      bsh[buf][s][2 * wave + 1][lane] = u32x4{l1.x, l1.y, h1.x, h1.y};
    }
    if (stage + 1 < STAGES) load(stage + 1);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < SS; ++s) {
      // slot - tile0 and the limits relative to the tile fit in 32 bits
      const int rel = (stage * SS + s) * 32 + n;
      const int64_t slot = tile0 + rel;
      const bool row_ok = rel < lim_rel;
      u32x4 b[8];
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) b[kb] = bsh[buf][s][kb][lane];
      f32x16 acc[QW];
#pragma unroll
      for (int j = 0; j < QW; ++j) acc[j] = f32x16{};
      // ReLU, head weights and head sum of query j, in the per-query kernel's order
      // (identical scores), then the stores.
      auto epilogue = [&](int j) {
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) part += wr[j][r] * relu1(acc[j][r]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part),
                                                         __float_as_uint(part), false, false);
        part += __uint_as_float(half ? sw[0] : sw[1]);   // the other half-wave's heads
        store(j, slot, (row_ok & (rel < nvq_rel[j])) ? part : -__builtin_inff());
      };
      // Query-major: query j's eight products run while query j-1's epilogue is computed
      // (scheduling fences keep each query's products and the previous epilogue together),
      // so only the last query's epilogue runs with no product of this wavefront in flight.
#pragma unroll
      for (int j = 0; j < QW; ++j) {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j][kb], __builtin_bit_cast(bf16x8, b[kb]),
                                                           acc[j], 0, 0, 0);
        if (j > 0) epilogue(j - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      epilogue(QW - 1);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Block-mean indexer keys for the two-stage (HISA-style) filter: block b of query t holds the
// mean of the E4M3 keys at positions 8b .. 8b+7 that are visible and in the cache, stored
// as bf16 (nearest even) at row km_start[t] + b; n_blocks[t] receives ceil(n_visible / 8).
// 16 lanes per block, lane c covering channels 8c .. 8c+7; sums of E4M3 values are exact
// in float32 and the mean is one float32 division by the count. With last_only, only the
// block holding position n_visible - 1 is recomputed (the one a newly appended token
// changes).
__global__ __launch_bounds__(IS_THREADS) void block_mean_keys_kernel(
    const uint8_t* __restrict__ k_cache, int64_t n_entries, const int64_t* __restrict__ kv_start,
    const int32_t* __restrict__ n_visible, uint16_t* __restrict__ km,
    const int64_t* __restrict__ km_start, int64_t n_km_rows, int64_t max_blocks,
    int32_t* __restrict__ n_blocks, int last_only) {
  const int t = blockIdx.y;
  const int64_t nv = n_visible[t] > 0 ? n_visible[t] : 0;
  const int64_t nb = (nv + 7) / 8;
  if (blockIdx.x == 0 && threadIdx.x == 0) n_blocks[t] = (int32_t)nb;
  if (last_only && (threadIdx.x >> 4) != 0) return;
  const int64_t b = last_only ? nb - 1 : (int64_t)blockIdx.x * (IS_THREADS / 16) + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  if (b < 0 || b >= nb || b >= max_blocks) return;
  const int64_t dst = km_start[t] + b;
  if (dst < 0 || dst >= n_km_rows) return;
  const int64_t base = kv_start[t];
  float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int count = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t pos = 8 * b + i;
    const int64_t row = base + pos;
    if (pos < nv && row >= 0 && row < n_entries) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(k_cache + row * 128 + 8 * c);
      const u32x2 lo = e4m3x4_to_bf16x4(v.x), hi = e4m3x4_to_bf16x4(v.y);
      const uint32_t d[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sum[2 * j] += __uint_as_float(d[j] << 16);
        sum[2 * j + 1] += __uint_as_float(d[j] & 0xFFFF0000u);
      }
      ++count;
    }
  }
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float m0 = count ? __fdiv_rn(sum[2 * j], (float)count) : 0.f;
    const float m1 = count ? __fdiv_rn(sum[2 * j + 1], (float)count) : 0.f;
    out[j] = f32_to_bf16_rne(m0) | (f32_to_bf16_rne(m1) << 16);
  }
  *reinterpret_cast<u32x4*>(km + dst * 128 + 8 * c) = out;
}

hipError_t launch_block_mean_keys(int n_q, const uint8_t* k_cache, int64_t n_entries,
                                  const int64_t* kv_start, const int32_t* n_visible, uint16_t* km,
                                  const int64_t* km_start, int64_t n_km_rows, int64_t max_blocks,
                                  int32_t* n_blocks, bool last_only, hipStream_t stream) {
  const int per_block = IS_THREADS / 16;
  dim3 grid(last_only ? 1u : (unsigned)((max_blocks + per_block - 1) / per_block), (unsigned)n_q);
  hipLaunchKernelGGL(block_mean_keys_kernel, grid, dim3(IS_THREADS), 0, stream, k_cache,
                     n_entries, kv_start, n_visible, km, km_start, n_km_rows, max_blocks, n_blocks,
                     last_only ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_index_score_shared(int n_q, const uint16_t* q_idx, const float* w,
                                     const uint8_t* k_cache, int64_t n_entries, int64_t kv_start,
                                     const int32_t* n_visible, float* scores, int64_t ld,
                                     float* block_max, int64_t ld_bm, hipStream_t stream) {
  dim3 grid((unsigned)((ld + SQ2_TILE - 1) / SQ2_TILE), (unsigned)((n_q + SQ2_QT - 1) / SQ2_QT));
  auto kernel = block_max != nullptr ? index_score_shared2_kernel<SQ2_QW, SQ2_SS, true>
                                     : index_score_shared2_kernel<SQ2_QW, SQ2_SS, false>;
  hipLaunchKernelGGL(kernel, grid, dim3(IS_THREADS), 0,
                     stream, n_q, q_idx, w, k_cache, n_entries, kv_start, n_visible, scores, ld,
                     block_max, ld_bm);
  return hipGetLastError();
}

hipError_t launch_index_score(bool reindex, int key_format, int n_q, const uint16_t* q_idx,
                              const float* w, const uint8_t* k_cache, const uint8_t* k_scales,
                              int64_t n_entries, const int64_t* kv_start,
                              const int32_t* n_visible, const int32_t* pool_blocks, int n_pool,
                              float* scores, int64_t ld, float* block_max, int64_t ld_bm,
                              uint32_t* block_aux, hipStream_t stream) {
  const int tile = (IS_THREADS / 64) * (reindex ? IS_STEPS_REINDEX : IS_STEPS_FULL) * 32;
  const int64_t tiles = (ld + tile - 1) / tile;
  dim3 grid((unsigned)tiles, (unsigned)n_q);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(IS_THREADS), 0, stream, q_idx, w, k_cache, k_scales,
                       n_entries, kv_start, n_visible, pool_blocks, n_pool, scores, ld, block_max,
                       ld_bm);
  };
  if (key_format == KF_BF16) {
    reindex ? go(index_score_kernel<true, KF_BF16>) : go(index_score_kernel<false, KF_BF16>);
  } else if (k_scales != nullptr) {
    if (reindex) {
      go(index_score_kernel<true, KF_MXFP4>);
    } else {
      auto wide = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, dim3(IS_THREADS), 0, stream, q_idx, w, k_cache,
                           k_scales, n_entries, kv_start, n_visible, scores, ld, block_max,
                           ld_bm, block_aux);
      };
      if (block_aux != nullptr)
        wide(index_score_full_wide_fp4_kernel<true>);
      else
        wide(index_score_full_wide_fp4_kernel<false>);
    }
  } else if (reindex) {
    constexpr int RT = (IS_THREADS / 64) * IS_STEPS_REINDEX * 32;
    hipLaunchKernelGGL((index_score_reindex_e4m3_kernel<IS_STEPS_REINDEX, RE_PF>),
                       dim3((unsigned)((ld + RT - 1) / RT), (unsigned)n_q), dim3(IS_THREADS), 0,
                       stream, q_idx, w, k_cache, n_entries, kv_start, n_visible, pool_blocks,
                       n_pool, scores, ld, block_max, ld_bm);
  } else {
    auto full = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, grid, dim3(IS_THREADS), 0, stream, q_idx, w, k_cache, n_entries,
                         kv_start, n_visible, scores, ld, block_max, ld_bm, block_aux);
    };
    if (block_aux != nullptr)
      full(index_score_full_e4m3_kernel<2>);
    else if (scores == nullptr && block_max != nullptr)
      full(index_score_full_e4m3_kernel<1>);
    else
      full(index_score_full_e4m3_kernel<0>);
  }
  return hipGetLastError();
}

}  // namespace csa2
