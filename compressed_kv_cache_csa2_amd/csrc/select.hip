// Exact Top-K and HSI block-pool selection on gfx950.
//
// Both selections keep the k largest values of a row under the order (value descending,
// index ascending), never keep -inf or NaN, and emit the kept indices in ascending
// order. That is the Top-512 of the indexer scores and the top-2,048 block maxima of the
// Hierarchical Sparse Indexer ("DeepSeek-v4.1 Flash: Pushing the Limits of KV Cache
// Compression", 2.3.4; "DeepSeek-V4.1-Flash - Architecture", section 3).
//
// One 1024-thread workgroup per query row. Values become order-preserving 32-bit keys
// (0 marks an element that cannot be selected); thread t owns 16 consecutive elements
// (rows up to 16,384) or 32 (longer rows, walked in segments of 32,768 past that) and
// keeps their keys in registers.
//   1. A block reduction gives the count, the smallest and the largest key.
//   2. Range refinement: the live key interval [A, B] is split into at most 2,048 equal
//      power-of-two bins, an LDS histogram of the keys inside [A, B] is taken, and the bin
//      holding the k-th largest key becomes the new interval. Bins follow the data's own
//      key range, so the first histogram spreads over many bins (few atomic collisions).
//   3. Once the interval holds at most 256 keys (usually after one pass) they are copied
//      to LDS and the k-th largest, tau, is the one key with fewer than `need` keys
//      above it and at least `need` at or above it; no further pass over the row.
//   4. Emission: every key > tau is kept, and of the keys == tau the lowest-indexed
//      (k - #greater). A block-wide prefix sum gives each thread its output offset (a
//      second one orders the ties when only some of them are kept); output is
//      deterministic and sorted by index.
//
// Block prefilter for Top-K: with maxima of 8-slot blocks, any threshold T such that at
// least k blocks have maximum >= T bounds the k-th largest score from below (each of those
// blocks holds a score >= T), so every winner lies in a block whose maximum is >= T. One
// or two refinement passes over the block maxima give such a T with few extra blocks;
// only those blocks' scores (typically ~600 blocks instead of the whole row) are then
// selected exactly. If more than 2,048 blocks tie at the threshold the full row is used.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int NBINS = 2048;
constexpr int BINS_PER_THREAD = NBINS / SEL_THREADS;
constexpr int CAND_BLOCKS_CAP = 2048;
constexpr int LIST_CAP = 256;          // an interval this small is finished by counting
constexpr uint32_t ALL_TIES = 0xFFFFFFFFu;

struct SelShared {
  uint32_t hist[NBINS];
  uint32_t wsum[SEL_WAVES];
  uint32_t wmin[SEL_WAVES];
  uint32_t wmax[SEL_WAVES];
  uint32_t scal[4];
  uint32_t list_n;
  uint32_t lkey[LIST_CAP];
  int32_t cblocks[CAND_BLOCKS_CAP];
};

// Unsigned minimum / maximum (the device min/max overloads compare as signed int).
__device__ __forceinline__ uint32_t umin32(uint32_t a, uint32_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Exclusive prefix sum over the block's threads; *total receives the block sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, SelShared& sh, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh.wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < SEL_WAVES; ++i) {
    const uint32_t s = sh.wsum[i];
    before += i < wave ? s : 0u;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// The keys of one row: thread tid holds elements seg*SEG + tid*R + r in keys[r]. Short
// rows use R = 16 so that every thread of the block holds keys.
template <class Src, int R>
struct KeyRow {
  static constexpr int SEG = SEL_THREADS * R;
  Src src;
  int64_t n;
  int nseg;
  uint32_t keys[R];
  int loaded;

  __device__ __forceinline__ KeyRow(const Src& s, int64_t n_) : src(s), n(n_), nseg((int)((n_ + SEG - 1) / SEG)), loaded(-1) {}

  __device__ __forceinline__ void load(int seg) {
    if (seg == loaded) return;
    const uint32_t base = (uint32_t)seg * SEG + threadIdx.x * R;
    src.template load<R>(base, (uint32_t)n, keys);
    loaded = seg;
  }
  static constexpr int per_thread() { return R; }
};

// One histogram pass over the keys in [A, B], which holds the need-th largest of them:
// [A, B] becomes the one of at most 2,048 equal power-of-two bins that holds it, and
// `need` the rank within the new interval. Bins follow the interval's own span, so the
// first pass spreads the keys over many bins (few atomic collisions) and each pass shrinks
// the interval by 2^11. Returns the number of keys in the new interval.
template <class Row>
__device__ __forceinline__ uint32_t hist_pass(Row& row, uint32_t& A, uint32_t& B, uint32_t& need,
                                              SelShared& sh) {
  constexpr int R = Row::per_thread();
  const int tid = threadIdx.x;
  const uint32_t span = B - A;
  const int bits = 32 - __clz(span);                 // span < 2^bits
  const int s = bits > 11 ? bits - 11 : 0;           // (span >> s) < 2048
#pragma unroll
  for (int j = 0; j < BINS_PER_THREAD; ++j) sh.hist[tid + j * SEL_THREADS] = 0;
  __syncthreads();
  for (int seg = 0; seg < row.nseg; ++seg) {
    row.load(seg);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t key = row.keys[r];
      if (key != 0u && key >= A && key <= B) atomicAdd(&sh.hist[(key - A) >> s], 1u);
    }
  }
  __syncthreads();
  // Thread tid owns bins BPT*tid .. BPT*tid + BPT-1.
  uint32_t h[BINS_PER_THREAD];
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < BINS_PER_THREAD; ++j) {
    h[j] = sh.hist[BINS_PER_THREAD * tid + j];
    local += h[j];
  }
  uint32_t total;
  const uint32_t excl = block_exclusive_scan(local, sh, &total);
  uint32_t above = total - excl - local;   // keys in bins above this thread's bins
#pragma unroll
  for (int j = BINS_PER_THREAD - 1; j >= 0; --j) {
    if (above < need && need <= above + h[j]) {
      sh.scal[0] = BINS_PER_THREAD * tid + j;
      sh.scal[1] = above;
      sh.scal[2] = h[j];
    }
    above += h[j];
  }
  __syncthreads();
  const uint32_t b = sh.scal[0];
  const uint32_t above_b = sh.scal[1];
  const uint32_t in_b = sh.scal[2];
  __syncthreads();
  const uint64_t lo = (uint64_t)A + ((uint64_t)b << s);
  const uint64_t hi = lo + (1ull << s) - 1;
  need -= above_b;
  A = (uint32_t)lo;
  B = hi < (uint64_t)B ? (uint32_t)hi : B;
  return in_b;
}

// Narrows [A, B] (holding the k-th largest key, with k - need keys above B) until A is
// the k-th largest key or, once at most cap keys are >= A, a lower bound of it.
template <class Row>
__device__ __forceinline__ void refine_cap(Row& row, uint32_t& A, uint32_t& B, uint32_t& need,
                                           uint32_t k, uint32_t cap, SelShared& sh) {
#pragma unroll 1
  while (A != B) {
    const uint32_t in_new = hist_pass(row, A, B, need, sh);
    if ((k - need) + in_new <= cap) break;   // keys >= the new A
  }
}

// The cnt <= LIST_CAP keys in [A, B] are gathered into LDS; the need-th largest of them
// is found by counting, for each, how many are greater and how many are at least as
// large. tau receives it and n_eq how many keys equal to tau are taken (ALL_TIES when
// every one of them is).
template <class Row>
__device__ __forceinline__ void rank_list(Row& row, uint32_t A, uint32_t B, uint32_t need,
                                          uint32_t cnt, SelShared& sh, uint32_t& tau,
                                          uint32_t& n_eq) {
  constexpr int R = Row::per_thread();
  const int tid = threadIdx.x;
  if (tid < LIST_CAP) sh.lkey[tid] = 0u;   // padding reads as "below every key"
  if (tid == 0) sh.list_n = 0u;
  __syncthreads();
  for (int seg = 0; seg < row.nseg; ++seg) {
    row.load(seg);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t key = row.keys[r];
      if (key != 0u && key >= A && key <= B) {
        const uint32_t slot = atomicAdd(&sh.list_n, 1u);
        if (slot < (uint32_t)LIST_CAP) sh.lkey[slot] = key;
      }
    }
  }
  __syncthreads();
  if ((uint32_t)tid < cnt) {
    const uint32_t ki = sh.lkey[tid];
    uint32_t gt = 0, ge = 0;
    const uint4* l4 = reinterpret_cast<const uint4*>(sh.lkey);
    for (uint32_t j = 0; j < (cnt + 3) / 4; ++j) {
      const uint4 v = l4[j];
      gt += (v.x > ki) + (v.y > ki) + (v.z > ki) + (v.w > ki);
      ge += (v.x >= ki) + (v.y >= ki) + (v.z >= ki) + (v.w >= ki);
    }
    if (gt < need && need <= ge) {   // every thread holding tau writes the same values
      sh.scal[0] = ki;
      sh.scal[1] = need - gt == ge - gt ? ALL_TIES : need - gt;
    }
  }
  __syncthreads();
  tau = sh.scal[0];
  n_eq = sh.scal[1];
  __syncthreads();
}

// Count / min / max of the valid keys of the row.
template <class Row>
__device__ __forceinline__ void row_stats(Row& row, uint32_t& count, uint32_t& kmin, uint32_t& kmax,
                          SelShared& sh) {
  constexpr int R = Row::per_thread();
  uint32_t c = 0, mn = 0xFFFFFFFFu, mx = 0u;
  for (int seg = 0; seg < row.nseg; ++seg) {
    row.load(seg);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t key = row.keys[r];
      c += key != 0u;
      mn = umin32(mn, key != 0u ? key : 0xFFFFFFFFu);
      mx = umax32(mx, key);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    c += __shfl_xor(c, off);
    mn = umin32(mn, (uint32_t)__shfl_xor(mn, off));
    mx = umax32(mx, (uint32_t)__shfl_xor(mx, off));
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sh.wsum[wave] = c;
    sh.wmin[wave] = mn;
    sh.wmax[wave] = mx;
  }
  __syncthreads();
  c = 0;
  mn = 0xFFFFFFFFu;
  mx = 0u;
#pragma unroll
  for (int i = 0; i < SEL_WAVES; ++i) {
    c += sh.wsum[i];
    mn = umin32(mn, sh.wmin[i]);
    mx = umax32(mx, sh.wmax[i]);
  }
  __syncthreads();
  count = c;
  kmin = mn;
  kmax = mx;
}

// Emit, in ascending index order, every key > tau and of the keys == tau the first n_eq
// (every one for ALL_TIES). emit(rank, index). Returns the count.
template <class Row, class Emit>
__device__ __forceinline__ uint32_t emit_ordered(Row& row, uint32_t tau, uint32_t n_eq, SelShared& sh,
                                 Emit emit) {
  constexpr int R = Row::per_thread();
  const bool split_ties = n_eq != 0u && n_eq != ALL_TIES;
  uint32_t eq_base = 0, out_base = 0;
  for (int seg = 0; seg < row.nseg; ++seg) {
    row.load(seg);
    uint32_t gt_mask = 0, eq_mask = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t key = row.keys[r];
      gt_mask |= (uint32_t)(key != 0u && key > tau) << r;
      eq_mask |= (uint32_t)(key != 0u && key == tau) << r;
    }
    uint32_t take = n_eq == ALL_TIES ? gt_mask | eq_mask : gt_mask;
    if (split_ties) {   // uniform: keep the first n_eq ties of the row
      const uint32_t n_e = __popc(eq_mask);
      uint32_t eq_total;
      const uint32_t eq_before = eq_base + block_exclusive_scan(n_e, sh, &eq_total);
      const uint32_t eq_keep = eq_before >= n_eq ? 0u : umin32(n_e, n_eq - eq_before);
      uint32_t seen = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t bit = (eq_mask >> r) & 1u;
        take |= (uint32_t)(bit != 0u && seen < eq_keep) << r;
        seen += bit;
      }
      eq_base += eq_total;
    }
    uint32_t take_total;
    uint32_t pos = out_base + block_exclusive_scan(__popc(take), sh, &take_total);
    const uint32_t base = (uint32_t)seg * Row::SEG + threadIdx.x * R;
    while (take != 0u) {
      const int r = __builtin_ctz(take);
      take &= take - 1u;
      emit(pos++, base + r);
    }
    out_base += take_total;
  }
  return out_base;
}

// Full exact selection of the k best keys of a row.
template <class Row, class Emit>
__device__ __forceinline__ uint32_t select_row(Row& row, uint32_t k, SelShared& sh, Emit emit) {
  uint32_t cnt, A, B;
  row_stats(row, cnt, A, B, sh);
  if (cnt <= k) return emit_ordered(row, 0u, 0u, sh, emit);
  // [A, B] holds cnt keys, of which the need-th largest is the k-th largest of the row.
  uint32_t need = k;
#pragma unroll 1
  while (A != B && cnt > (uint32_t)LIST_CAP) cnt = hist_pass(row, A, B, need, sh);
  uint32_t tau, n_eq;
  if (A == B) {
    tau = A;
    n_eq = need == cnt ? ALL_TIES : need;
  } else {
    rank_list(row, A, B, need, cnt, sh, tau, n_eq);
  }
  return emit_ordered(row, tau, n_eq, sh, emit);
}

// --------------------------------------------------------------------------- key sources

// Rows are 16-byte aligned with a leading dimension that is a multiple of 4 (checked by
// the C ABI), so a float4 starting below n never leaves its row. Every source issues all
// of a segment's loads before using any (an element past the end reads the row's first
// float4 and is masked afterwards), so a segment costs one memory round trip. Element
// indices of a row are below 2^31 + 2^15 (rows hold at most 2^31 elements), so they are
// kept in 32 bits.
__device__ __forceinline__ void keys4(float4 v, uint32_t i0, uint32_t n, uint32_t* k) {
  const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) k[j] = (i0 + j < n && selectable(f[j])) ? float_key(f[j]) : 0u;
}

// Scores of a row (float array), keys of slots i < n.
struct ScoreSrc {
  const float* row;
  template <int R>
  __device__ __forceinline__ void load(uint32_t base, uint32_t n, uint32_t (&keys)[R]) const {
    float4 v[R / 4];
#pragma unroll
    for (int q = 0; q < R / 4; ++q) {
      const uint32_t i0 = base + 4 * q;
      v[q] = *reinterpret_cast<const float4*>(row + (i0 < n ? i0 : 0u));
    }
#pragma unroll
    for (int q = 0; q < R / 4; ++q) keys4(v[q], base + 4 * q, n, &keys[4 * q]);
  }
};

// Block maxima with an override for one block (forced +inf for the pool, or a recomputed
// maximum for a partial last block in the Top-K prefilter; special = -1 for none).
struct BlockSrc {
  const float* bm;
  int64_t special;
  float special_value;
  template <int R>
  __device__ __forceinline__ void load(uint32_t base, uint32_t n, uint32_t (&keys)[R]) const {
    float4 v[R / 4];
#pragma unroll
    for (int q = 0; q < R / 4; ++q) {
      const uint32_t i0 = base + 4 * q;
      v[q] = *reinterpret_cast<const float4*>(bm + (i0 < n ? i0 : 0u));
    }
    const uint32_t sp = special < 0 ? 0xFFFFFFFFu : (uint32_t)special;
#pragma unroll
    for (int q = 0; q < R / 4; ++q) {
      const uint32_t i0 = base + 4 * q;
      const uint32_t j = sp - i0;   // < 4 only when the special block is in this float4
      if (j == 0u) v[q].x = special_value;
      if (j == 1u) v[q].y = special_value;
      if (j == 2u) v[q].z = special_value;
      if (j == 3u) v[q].w = special_value;
      keys4(v[q], i0, n, &keys[4 * q]);
    }
  }
};

// Scores of the candidate blocks' slots: element i is slot cblocks[i/8]*8 + i%8 (a
// negative block id, or a slot at or past n_slots, is absent).
struct CandSrc {
  const float* row;
  const int32_t* cblocks;   // LDS
  int64_t n_slots;          // slots >= n_slots are outside the selection
  template <int R>
  __device__ __forceinline__ void load(uint32_t base, uint32_t n, uint32_t (&keys)[R]) const {
    const uint32_t ns = (uint32_t)n_slots;
    float4 v[R / 4];
    uint32_t s0[R / 4];
#pragma unroll
    for (int q = 0; q < R / 4; ++q) {   // 4 consecutive elements of one block
      const uint32_t i0 = base + 4 * q;
      const int32_t b = i0 < n ? cblocks[i0 >> 3] : -1;
      s0[q] = b >= 0 ? (uint32_t)b * 8u + (i0 & 7u) : ns;   // absent block: masked
    }
#pragma unroll
    for (int q = 0; q < R / 4; ++q)
      v[q] = *reinterpret_cast<const float4*>(row + (s0[q] < ns ? s0[q] : 0u));
#pragma unroll
    for (int q = 0; q < R / 4; ++q) {
      const bool ok = s0[q] < ns;
      keys4(v[q], ok ? s0[q] : 0u, ok ? ns : 0u, &keys[4 * q]);
    }
  }
};

// --------------------------------------------------------------------------- kernels

// Rows of at most 16,384 elements hold 16 keys per thread, longer ones 32 (in segments
// of 32,768 when longer still).
template <class Src, class Emit>
__device__ __forceinline__ uint32_t select_any(const Src& src, int64_t n, uint32_t k, SelShared& sh,
                                               Emit emit) {
  if (n <= (int64_t)SEL_THREADS * 16) {
    KeyRow<Src, 16> row(src, n);
    return select_row(row, k, sh, emit);
  }
  KeyRow<Src, 32> row(src, n);
  return select_row(row, k, sh, emit);
}

__global__ __launch_bounds__(SEL_THREADS) void topk_kernel(
    const float* __restrict__ scores, int64_t ld, int64_t n_cols,
    const int32_t* __restrict__ n_valid, const float* __restrict__ block_max, int64_t ld_bm,
    int k, int pool_use, const int32_t* __restrict__ pool_blocks, int n_pool,
    int32_t* __restrict__ out, int64_t ld_idx) {
  __shared__ SelShared sh;
  const int t = blockIdx.x;
  const float* row = scores + (int64_t)t * ld;
  int64_t n = n_cols;
  if (n_valid != nullptr) {
    const int64_t v = n_valid[t];
    n = v < 0 ? 0 : (v < n ? v : n);
  }
  int32_t* orow = out + (int64_t)t * ld_idx;
  const uint32_t kk = (uint32_t)k;
  auto map = [&](int64_t slot) -> int32_t {
    if (pool_use != 1) return (int32_t)slot;
    const int64_t pb = slot >> 3;
    const int32_t b = pb < n_pool ? pool_blocks[(int64_t)t * n_pool + pb] : -1;
    return b < 0 ? -1 : (int32_t)((int64_t)b * 8 + (slot & 7));
  };
  uint32_t kept = 0;
  bool done = false;

  if (pool_use == 2) {
    // Candidates: the slots of the pool's blocks (ascending block ids, so the winners come
    // out in ascending position order; -1 entries are absent).
    const int32_t* prow = pool_blocks + (int64_t)t * n_pool;
    for (int i = threadIdx.x; i < n_pool; i += SEL_THREADS) sh.cblocks[i] = prow[i];
    __syncthreads();
    const CandSrc csrc{row, sh.cblocks, n};
    kept = select_any(csrc, (int64_t)n_pool * 8, kk, sh, [&](uint32_t rank, int64_t i) {
      if (rank < kk) orow[rank] = (int32_t)((int64_t)sh.cblocks[i >> 3] * 8 + (i & 7));
    });
    done = true;
  }
  if (!done && block_max != nullptr && n > (int64_t)CAND_BLOCKS_CAP * 8) {
    // Phase A: a threshold on block maxima leaving at most CAND_BLOCKS_CAP blocks.
    const int64_t nb = (n + 7) >> 3;
    const int64_t tail = n & 7;
    float tail_max = -__builtin_inff();
    if (tail) {
      for (int64_t s = (nb - 1) * 8; s < n; ++s) tail_max = fmaxf(tail_max, row[s]);
    }
    const BlockSrc bsrc{block_max + (int64_t)t * ld_bm, tail ? nb - 1 : -1, tail_max};
    KeyRow<BlockSrc, 32> brow(bsrc, nb);
    uint32_t count, A, B;
    row_stats(brow, count, A, B, sh);
    uint32_t thr = 0;   // keep blocks with key >= thr (0: every valid block)
    bool fits = count <= (uint32_t)CAND_BLOCKS_CAP;
    if (count > kk) {
      uint32_t need = kk;
      refine_cap(brow, A, B, need, kk, (uint32_t)CAND_BLOCKS_CAP, sh);
      thr = A;
      fits = true;
    }
    // Collect candidate blocks (ascending); count them to check the cap.
    const uint32_t n_cand = emit_ordered(brow, thr == 0u ? 0u : thr - 1u, 0u, sh,
                                         [&](uint32_t rank, int64_t b) {
                                           if (rank < CAND_BLOCKS_CAP) sh.cblocks[rank] = (int32_t)b;
                                         });
    __syncthreads();
    if (fits && n_cand <= (uint32_t)CAND_BLOCKS_CAP) {
      const CandSrc csrc{row, sh.cblocks, n};
      kept = select_any(csrc, (int64_t)n_cand * 8, kk, sh, [&](uint32_t rank, int64_t i) {
        if (rank < kk) orow[rank] = map((int64_t)sh.cblocks[i >> 3] * 8 + (i & 7));
      });
      done = true;
    }
  }
  if (!done) {
    const ScoreSrc ssrc{row};
    kept = select_any(ssrc, n, kk, sh, [&](uint32_t rank, int64_t i) {
      if (rank < kk) orow[rank] = map(i);
    });
  }
  for (int64_t r = kept + threadIdx.x; r < k; r += SEL_THREADS) orow[r] = -1;
}

__global__ __launch_bounds__(SEL_THREADS) void block_pool_kernel(
    const float* __restrict__ block_max, int64_t ld_bm, const int32_t* __restrict__ n_visible,
    int n_keep, int32_t* __restrict__ pool, int64_t ld_pool) {
  __shared__ SelShared sh;
  const int t = blockIdx.x;
  const int64_t nv = n_visible[t];
  int64_t nb = nv > 0 ? (nv + 7) >> 3 : 0;
  if (nb > ld_bm) nb = ld_bm;
  int32_t* prow = pool + (int64_t)t * ld_pool;
  const BlockSrc src{block_max + (int64_t)t * ld_bm, nb - 1, __builtin_inff()};
  const uint32_t kept = select_any(src, nb, (uint32_t)n_keep, sh, [&](uint32_t rank, int64_t b) {
    if (rank < (uint32_t)n_keep) prow[rank] = (int32_t)b;
  });
  for (int64_t r = kept + threadIdx.x; r < n_keep; r += SEL_THREADS) prow[r] = -1;
}

hipError_t launch_topk(int n_q, const float* scores, int64_t ld_scores, int64_t n_cols,
                       const int32_t* n_valid, const float* block_max, int64_t ld_bm, int k,
                       int pool_use, const int32_t* pool_blocks, int n_pool, int32_t* topk_idx,
                       int64_t ld_idx, hipStream_t stream) {
  hipLaunchKernelGGL(topk_kernel, dim3(n_q), dim3(SEL_THREADS), 0, stream, scores, ld_scores,
                     n_cols, n_valid, block_max, ld_bm, k, pool_use, pool_blocks, n_pool, topk_idx,
                     ld_idx);
  return hipGetLastError();
}

hipError_t launch_block_pool(int n_q, const float* block_max, int64_t ld_bm,
                             const int32_t* n_visible, int n_keep, int32_t* pool_blocks,
                             int64_t ld_pool, hipStream_t stream) {
  hipLaunchKernelGGL(block_pool_kernel, dim3(n_q), dim3(SEL_THREADS), 0, stream, block_max,
                     ld_bm, n_visible, n_keep, pool_blocks, ld_pool);
  return hipGetLastError();
}

}  // namespace csa2
