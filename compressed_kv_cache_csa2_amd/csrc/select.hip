// Exact Top-K and HSI block-pool selection on gfx950.
//
// Both selections keep the k largest values of a row under the order (value descending,
// index ascending), never keep -inf or NaN, and emit the kept indices in ascending
// order. That is the Top-512 of the indexer scores and the top-2,048 block maxima of the
// Hierarchical Sparse Indexer ("DeepSeek-v4.1 Flash: Pushing the Limits of KV Cache
// Compression", 2.3.4; "DeepSeek-V4.1-Flash - Architecture", section 3).
//
// One 1024-thread workgroup per query row. Values become order-preserving 32-bit keys
// (0 marks an element that cannot be selected) held in registers: R = 4, 8 or 16 keys per
// thread for rows up to 4,096, 8,192 or 16,384 elements, else R = 32 (walked in segments
// of 32,768 past that).
// Thread t holds the R/4 float4 groups starting at elements 4*(t + 1024*g), so each
// wavefront load reads 1 KiB of consecutive memory.
//   1. A block reduction gives the count, the smallest and the largest key.
//   2. Range refinement: the live key interval [A, B] is split into at most 2,048 equal
//      power-of-two bins, an LDS histogram of the keys inside [A, B] is taken, and the bin
//      holding the k-th largest key becomes the new interval. Bins follow the data's own
//      key range, so the first histogram spreads over many bins (few atomic collisions).
//   3. Once the interval holds at most 256 keys (usually after one pass) they are copied
//      to LDS and the k-th largest, tau, is the one key with fewer than `need` keys
//      above it and at least `need` at or above it; no further pass over the row.
//   4. Emission: every key > tau is kept, and of the keys == tau the lowest-indexed
//      (k - #greater). One block-wide prefix sum over the per-group counts (four 16-bit
//      fields per 64-bit word) gives every kept element its rank in index order (a second
//      one orders the ties when only some of them are kept). Ranks go to LDS and the
//      result is written out in one coalesced pass; output is sorted by index.
//
// Block prefilter for Top-K: with maxima of 8-slot blocks, any threshold T such that at
// least k blocks have maximum >= T bounds the k-th largest score from below (each of those
// blocks holds a score >= T), so every winner lies in a block whose maximum is >= T. One
// or two refinement passes over the block maxima give such a T with few extra blocks;
// only those blocks' scores (typically ~600 blocks instead of the whole row) are then
// selected exactly. If more than 2,048 blocks tie at the threshold the full row is used.
#include "csa2_device.h"
#include "csa2_launch.h"

#include <type_traits>

namespace csa2 {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int NBINS = 2048;
constexpr int BINS_PER_THREAD = NBINS / SEL_THREADS;
constexpr int CAND_BLOCKS_CAP = 2048;
constexpr int OUT_CAP = 2048;          // the largest k / n_keep
constexpr int LIST_CAP = 256;          // an interval this small is finished by counting
constexpr int FS_EARLY_WAVES = 4;      // full_select_kernel: wavefronts that load the indexer
                                       // operands before the candidate scan
constexpr uint32_t ALL_TIES = 0xFFFFFFFFu;
constexpr uint32_t INF_KEY = 0xFF800000u;   // float_key(+inf)

struct SelShared {
  uint32_t hist[NBINS];
  uint32_t wsum[SEL_WAVES];
  uint32_t wabove[SEL_WAVES];
  uint32_t wmin[SEL_WAVES];
  uint32_t wmax[SEL_WAVES];
  uint32_t wcnt[SEL_WAVES];
  uint32_t scal[4];
  uint32_t scal2[2];
  uint32_t list_n;
  uint32_t lkey[LIST_CAP];
  int32_t cblocks[CAND_BLOCKS_CAP];
  int32_t obuf[OUT_CAP];
  uint32_t gpos[8 * SEL_THREADS];      // per-group counts, then offsets, in index order
};


// Inclusive prefix sum over the 64 lanes of a wavefront with DPP lane moves: shifts by 1, 2,
// 4 and 8 within each row of 16 lanes (a lane with no source adds 0), then the last lane
// of row 0 added to row 1 and of row 2 to row 3 (row_bcast:15), and the last lane of row 1
// to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_inclusive_add(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return x;
}

// Exclusive prefix sum over the block's threads; *total receives the block sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, SelShared& sh, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_add(v);
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

// The keys of one row. keys[4g + j] is element seg*SEG + 4*(tid + SEL_THREADS*g) + j.
// A row of one segment is loaded once; a longer one (MULTI) is reloaded segment by
// segment in every pass.
template <class Src, int R, bool MULTI>
struct KeyRow {
  static constexpr int SEG = SEL_THREADS * R;
  Src src;
  uint32_t n;
  int nseg;
  uint32_t keys[R];

  __device__ __forceinline__ KeyRow(const Src& s, int64_t n_) : src(s), n((uint32_t)n_), nseg((int)((n_ + SEG - 1) / SEG)) {
    if (!MULTI) src.template load<R>(first(0), 4u * SEL_THREADS, n, keys);
  }
  __device__ __forceinline__ int segs() const { return MULTI ? nseg : 1; }
  __device__ __forceinline__ static uint32_t first(int seg) {
    return (uint32_t)seg * SEG + 4u * threadIdx.x;
  }
  __device__ __forceinline__ void load(int seg) {
    if (MULTI) src.template load<R>(first(seg), 4u * SEL_THREADS, n, keys);
  }
  static constexpr int per_thread() { return R; }
};

// The interval search. [A, B] is a key interval believed to hold the k-th largest key;
// one pass histograms the keys inside it into at most 2,048 equal power-of-two bins
// and counts the keys above B with a wave ballot. If the k-th largest key lies in [A, B], the interval narrows to the bin holding
// it (each pass divides the span by 2^11); otherwise the caller moves the interval.
struct Interval {
  uint32_t A, B;
  uint32_t need;   // rank of the k-th largest key within [A, B] (1 = the largest there)
  uint32_t cnt;    // keys in [A, B]
  uint32_t ge;     // keys >= A
  // Optional second rank k2 < k, answered by the first pass only: t2 becomes a key such
  // that every key ranked k2 or better is >= t2 and at most cap2 keys are (0: not found).
  uint32_t k2 = 0u, cap2 = 0u, t2 = 0u;
};

enum { PASS_NARROWED = 0, PASS_ABOVE = 1, PASS_BELOW = 2 };

template <class Row>
__device__ __forceinline__ int hist_pass(Row& row, uint32_t k, Interval& iv, SelShared& sh) {
  constexpr int R = Row::per_thread();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t A = iv.A, B = iv.B;
  const uint32_t span = B - A;
  const int bits = 32 - __clz(span);                 // span < 2^bits
  const int s = bits > 11 ? bits - 11 : 0;           // (span >> s) < 2048
#pragma unroll
  for (int j = 0; j < BINS_PER_THREAD; ++j) sh.hist[tid + j * SEL_THREADS] = 0;
  __syncthreads();
  uint32_t above = 0;   // wave-uniform
  for (int seg = 0; seg < row.segs(); ++seg) {
    row.load(seg);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t key = row.keys[r];
      const uint32_t d = key - A;                    // A >= 1, so key 0 wraps past span
      // only keys inside [A, B] touch LDS (an interval narrowed around the k-th key holds
      // few of them, and absent slots none)
      if (d <= span) atomicAdd(&sh.hist[d >> s], 1u);
      above += __popcll(__ballot(key > B));
    }
  }
  if (lane == 0) sh.wabove[wave] = above;
  __syncthreads();
  uint32_t n_above = 0;
#pragma unroll
  for (int i = 0; i < SEL_WAVES; ++i) n_above += sh.wabove[i];
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
  // The second rank (uniform values): its key lies above B, or in one of this pass's bins
  // (need2 > 0), whose lower edge is then the threshold.
  uint32_t need2 = 0u;
  if (iv.k2 != 0u) {
    if (n_above >= iv.k2) {
      iv.t2 = n_above <= iv.cap2 ? B + 1u : 0u;   // B < 0xFFFFFFFF: a key lies above it
    } else if (iv.k2 - n_above <= total) {
      need2 = iv.k2 - n_above;
    }
    iv.k2 = 0u;
  }
  const bool is_above = n_above >= k;
  const uint32_t need = is_above ? 0u : k - n_above;
  const bool is_below = !is_above && need > total;
  if ((is_above || is_below) && need2 == 0u) return is_above ? PASS_ABOVE : PASS_BELOW;   // uniform
  uint32_t hi_keys = total - excl - local;   // keys in bins above this thread's bins
#pragma unroll
  for (int j = BINS_PER_THREAD - 1; j >= 0; --j) {
    if (!is_above && !is_below && hi_keys < need && need <= hi_keys + h[j]) {
      sh.scal[0] = BINS_PER_THREAD * tid + j;
      sh.scal[1] = hi_keys;
      sh.scal[2] = h[j];
    }
    if (need2 != 0u && hi_keys < need2 && need2 <= hi_keys + h[j]) {
      sh.scal2[0] = BINS_PER_THREAD * tid + j;
      sh.scal2[1] = n_above + hi_keys + h[j];     // keys at or above the bin's lower edge
    }
    hi_keys += h[j];
  }
  __syncthreads();
  if (need2 != 0u) {
    const uint32_t ge2 = sh.scal2[1];
    iv.t2 = ge2 <= iv.cap2 ? (uint32_t)((uint64_t)A + ((uint64_t)sh.scal2[0] << s)) : 0u;
  }
  if (is_above || is_below) {
    __syncthreads();
    return is_above ? PASS_ABOVE : PASS_BELOW;
  }
  const uint32_t b = sh.scal[0];
  const uint32_t above_b = sh.scal[1];
  const uint32_t in_b = sh.scal[2];
  __syncthreads();
  const uint64_t lo = (uint64_t)A + ((uint64_t)b << s);
  const uint64_t hi = lo + (1ull << s) - 1;
  iv.A = (uint32_t)lo;
  iv.B = hi < (uint64_t)B ? (uint32_t)hi : B;
  iv.need = need - above_b;
  iv.cnt = in_b;
  iv.ge = n_above + above_b + in_b;
  return PASS_NARROWED;
}

// Narrows iv until [A, B] holds the k-th largest key and either A == B, or (cap_list)
// at most LIST_CAP keys lie in [A, B], or (cap_ge) at most cap_ge keys are >= A. A first
// interval that misses the k-th key is replaced by the part of the key range on its
// side, which holds it; the search then always narrows, so it ends within a few passes.
template <class Row>
__device__ __forceinline__ void locate(Row& row, uint32_t k, Interval& iv, uint32_t cap_list,
                                       uint32_t cap_ge, SelShared& sh) {
#pragma unroll 1
  for (int it = 0; it < 8; ++it) {
    const int r = hist_pass(row, k, iv, sh);
    if (r == PASS_ABOVE) {         // B < 0xFFFFFFFF here, since some key is above it
      iv.A = iv.B + 1u;
      iv.B = 0xFFFFFFFFu;
      continue;
    }
    if (r == PASS_BELOW) {         // A > 1 here, since some valid key is below it
      iv.B = iv.A - 1u;
      iv.A = 1u;
      continue;
    }
    if (iv.A == iv.B || iv.cnt <= cap_list || iv.ge <= cap_ge) return;
  }
}

// The cnt <= LIST_CAP keys in [A, B] are gathered into LDS; the need-th largest of them
// is found by counting, for each, how many are greater and how many are at least as
// large. tau receives it and n_eq how many keys equal to tau are taken (ALL_TIES when
// every one of them is).
template <class Row>
__device__ __forceinline__ void rank_list(Row& row, const Interval& iv, SelShared& sh, uint32_t& tau,
                                          uint32_t& n_eq) {
  constexpr int R = Row::per_thread();
  const int tid = threadIdx.x;
  if (tid < LIST_CAP) sh.lkey[tid] = 0u;   // padding reads as "below every key"
  if (tid == 0) sh.list_n = 0u;
  __syncthreads();
  const uint32_t A = iv.A, span = iv.B - iv.A, cnt = iv.cnt, need = iv.need;
  for (int seg = 0; seg < row.segs(); ++seg) {
    row.load(seg);
    uint32_t in = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) in |= (uint32_t)(row.keys[r] - A <= span) << r;
    while (in != 0u) {   // rare: only the few keys of the interval
      const int r = __builtin_ctz(in);
      in &= in - 1u;
      uint32_t key = 0;
#pragma unroll
      for (int q = 0; q < R; ++q) key = q == r ? row.keys[q] : key;
      const uint32_t slot = atomicAdd(&sh.list_n, 1u);
      if (slot < (uint32_t)LIST_CAP) sh.lkey[slot] = key;
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

// Count of the valid keys of the row, and a first interval: the smallest and largest
// finite key among each thread's first four (a 4,096-key sample of the first segment).
// +inf keys stay out of it (a forced +inf block would stretch the first histogram over
// the whole key range); a sample with no finite key gives the whole finite range.
template <class Row>
__device__ __forceinline__ void row_prepare(Row& row, uint32_t& count, Interval& iv, SelShared& sh) {
  constexpr int R = Row::per_thread();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t c = 0;   // wave-uniform
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int seg = 0; seg < row.segs(); ++seg) {
    row.load(seg);
#pragma unroll
    for (int r = 0; r < R; ++r) c += __popcll(__ballot(row.keys[r] != 0u));
    if (seg == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t key = row.keys[r];
        const bool fin = key != 0u && key != INF_KEY;
        mn = umin32(mn, fin ? key : 0xFFFFFFFFu);
        mx = umax32(mx, fin ? key : 0u);
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mn = umin32(mn, (uint32_t)__shfl_xor(mn, off));
    mx = umax32(mx, (uint32_t)__shfl_xor(mx, off));
  }
  if (lane == 0) {
    sh.wcnt[wave] = c;
    sh.wmin[wave] = mn;
    sh.wmax[wave] = mx;
  }
  __syncthreads();
  c = 0;
  mn = 0xFFFFFFFFu;
  mx = 0u;
#pragma unroll
  for (int i = 0; i < SEL_WAVES; ++i) {
    c += sh.wcnt[i];
    mn = umin32(mn, sh.wmin[i]);
    mx = umax32(mx, sh.wmax[i]);
  }
  __syncthreads();
  count = c;
  if (mx == 0u) {       // no finite key in the sample
    mn = 1u;
    mx = INF_KEY - 1u;
  }
  iv.A = mn;
  iv.B = mx;
}

// Rank offsets in index order for a per-thread R-bit mask whose bit 4g + j stands for
// element 4*(tid + SEL_THREADS*g) + j: index order runs over g, then tid, then j, so the
// per-group counts are laid out in LDS in that order, each thread sums NG consecutive
// ones, and one block scan turns them into offsets. Afterwards sh.gpos[g*SEL_THREADS +
// tid] is the rank of this thread's first element of group g; the caller synchronises
// before gpos is written again.
template <int NG>
__device__ __forceinline__ uint32_t group_offsets(uint32_t mask, SelShared& sh) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int g = 0; g < NG; ++g) sh.gpos[g * SEL_THREADS + tid] = __popc((mask >> (4 * g)) & 0xFu);
  __syncthreads();
  uint32_t e[NG];
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    e[i] = sh.gpos[NG * tid + i];
    local += e[i];
  }
  uint32_t total;
  uint32_t excl = block_exclusive_scan(local, sh, &total);
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    sh.gpos[NG * tid + i] = excl;
    excl += e[i];
  }
  __syncthreads();
  return total;
}

// Emit every key > tau and, of the keys == tau, the first n_eq in index order (every one
// for ALL_TIES). emit(rank, index) with rank = position in ascending index order, or
// emit(rank, index, flag) when the callback takes a third argument: flag = 1 when the
// key reaches t_flag. Returns the count.
template <class Row, class Emit>
__device__ __forceinline__ uint32_t emit_ordered(Row& row, uint32_t tau, uint32_t n_eq, SelShared& sh,
                                 Emit emit, uint32_t t_flag = 0u) {
  constexpr int R = Row::per_thread();
  constexpr int NG = R / 4;
  const int tid = threadIdx.x;
  const bool split_ties = n_eq != 0u && n_eq != ALL_TIES;
  uint32_t eq_base = 0, out_base = 0;
  for (int seg = 0; seg < row.segs(); ++seg) {
    row.load(seg);
    uint32_t take = 0, eq_mask = 0;
    if (n_eq == ALL_TIES) {   // uniform; tau is then a valid key, so key >= tau excludes key 0
#pragma unroll
      for (int r = 0; r < R; ++r) take |= (uint32_t)(row.keys[r] >= tau) << r;
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) take |= (uint32_t)(row.keys[r] > tau) << r;   // tau >= 0
    }
    if (split_ties) {   // uniform: keep the first n_eq ties of the row in index order
#pragma unroll
      for (int r = 0; r < R; ++r) eq_mask |= (uint32_t)(row.keys[r] == tau) << r;
      const uint32_t eq_total = group_offsets<NG>(eq_mask, sh);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        uint32_t rank = eq_base + sh.gpos[g * SEL_THREADS + tid];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * g + j;
          const uint32_t bit = (eq_mask >> r) & 1u;
          take |= (uint32_t)(bit != 0u && rank < n_eq) << r;
          rank += bit;
        }
      }
      eq_base += eq_total;
      __syncthreads();
    }
    const uint32_t take_total = group_offsets<NG>(take, sh);
    uint32_t fmask = 0u;
    if constexpr (std::is_invocable_v<Emit&, uint32_t, uint32_t, uint32_t>) {
#pragma unroll
      for (int r = 0; r < R; ++r) fmask |= (uint32_t)(row.keys[r] >= t_flag) << r;
    }
    // Recomputed here rather than kept from the loads: the opaque copy stops the compiler
    // from holding R element indices live through every pass.
    uint32_t first = Row::first(seg);
    asm volatile("" : "+v"(first));
    uint32_t rest = take;
    while (rest != 0u) {
      const int r = __builtin_ctz(rest);
      rest &= rest - 1u;
      const int g = r >> 2;
      const uint32_t before = __popc(take & ((1u << r) - 1u) & (0xFu << (4 * g)));
      const uint32_t rank = out_base + sh.gpos[g * SEL_THREADS + tid] + before;
      const uint32_t index = first + 4u * SEL_THREADS * (uint32_t)g + (uint32_t)(r & 3);
      if constexpr (std::is_invocable_v<Emit&, uint32_t, uint32_t, uint32_t>) {
        emit(rank, index, (fmask >> r) & 1u);
      } else {
        emit(rank, index);
      }
    }
    out_base += take_total;
    __syncthreads();
  }
  return out_base;
}

// Full exact selection of the k best keys of a row. With k2 > 0, *t2 receives a key
// threshold that every key ranked k2 or better reaches, reached by at most cap2 keys, taken
// from the first histogram pass (0 when that pass cannot give one, or every key is kept).
template <class Row, class Emit>
__device__ __forceinline__ uint32_t select_row(Row& row, uint32_t k, SelShared& sh, Emit emit,
                                               uint32_t k2 = 0u, uint32_t cap2 = 0u,
                                               uint32_t* t2 = nullptr) {
  uint32_t cnt;
  Interval iv;
  row_prepare(row, cnt, iv, sh);
  if (t2 != nullptr) *t2 = 0u;
  if (cnt <= k) return emit_ordered(row, 0u, 0u, sh, emit);
  iv.k2 = k2 < k ? k2 : 0u;
  iv.cap2 = cap2;
  locate(row, k, iv, (uint32_t)LIST_CAP, 0u, sh);
  if (t2 != nullptr) *t2 = iv.t2;
  uint32_t tau, n_eq;
  if (iv.A == iv.B) {
    tau = iv.A;
    n_eq = iv.need == iv.cnt ? ALL_TIES : iv.need;
  } else {
    rank_list(row, iv, sh, tau, n_eq);
  }
  return emit_ordered(row, tau, n_eq, sh, emit, iv.t2);
}

// --------------------------------------------------------------------------- key sources

// Rows are 16-byte aligned with a leading dimension that is a multiple of 4 (checked by
// the C ABI), so a float4 starting below n never leaves its row. Every source issues all
// of a segment's loads before using any (a group past the end reads the row's first
// float4 and is masked afterwards), so a segment costs one memory round trip. Element
// indices of a row stay below 2^31 + 2^15 (rows hold at most 2^31 elements), so they are
// kept in 32 bits. Group g of a thread starts at element first + g * stride.
__device__ __forceinline__ void keys4(float4 v, uint32_t i0, uint32_t n, uint32_t* k) {
  const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) k[j] = (i0 + j < n && selectable(f[j])) ? float_key(f[j]) : 0u;
}

// Scores of a row (float array), keys of slots i < n.
struct ScoreSrc {
  const float* row;
  template <int R>
  __device__ __forceinline__ void load(uint32_t first, uint32_t stride, uint32_t n,
                                       uint32_t (&keys)[R]) const {
    float4 v[R / 4];
#pragma unroll
    for (int g = 0; g < R / 4; ++g) {
      const uint32_t i0 = first + g * stride;
      v[g] = *reinterpret_cast<const float4*>(row + (i0 < n ? i0 : 0u));
    }
#pragma unroll
    for (int g = 0; g < R / 4; ++g) keys4(v[g], first + g * stride, n, &keys[4 * g]);
  }
};

// Block maxima with an override for one block (forced +inf for the pool, or a recomputed
// maximum for a partial last block in the Top-K prefilter; special = -1 for none).
struct BlockSrc {
  const float* bm;
  int64_t special;
  float special_value;
  template <int R>
  __device__ __forceinline__ void load(uint32_t first, uint32_t stride, uint32_t n,
                                       uint32_t (&keys)[R]) const {
    float4 v[R / 4];
#pragma unroll
    for (int g = 0; g < R / 4; ++g) {
      const uint32_t i0 = first + g * stride;
      v[g] = *reinterpret_cast<const float4*>(bm + (i0 < n ? i0 : 0u));
    }
    const uint32_t sp = special < 0 ? 0xFFFFFFFFu : (uint32_t)special;
#pragma unroll
    for (int g = 0; g < R / 4; ++g) {
      const uint32_t i0 = first + g * stride;
      const uint32_t j = sp - i0;   // < 4 only when the special block is in this float4
      if (j == 0u) v[g].x = special_value;
      if (j == 1u) v[g].y = special_value;
      if (j == 2u) v[g].z = special_value;
      if (j == 3u) v[g].w = special_value;
      keys4(v[g], i0, n, &keys[4 * g]);
    }
  }
};

// Key of one block maximum: the forced block reads special_value; a block at or past
// n_blocks is absent.
__device__ __forceinline__ uint32_t block_key(float v, uint32_t b, uint32_t special,
                                              float special_value, uint32_t n_blocks) {
  const float x = b == special ? special_value : v;
  return (b < n_blocks && selectable(x)) ? float_key(x) : 0u;
}

// Maxima of aligned groups of four blocks ("quads"): element q is the largest key of
// blocks 4q .. 4q+3, one float4 (0 when none is present). Loaded eight quads at a time to
// bound the registers in flight.
struct QuadSrc {
  const float* bm;
  uint32_t special;   // forced block, 0xFFFFFFFF for none
  float special_value;
  uint32_t n_blocks;
  template <int R>
  __device__ __forceinline__ void load(uint32_t first, uint32_t stride, uint32_t n,
                                       uint32_t (&keys)[R]) const {
#pragma unroll
    for (int c = 0; c < R / 8; ++c) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t q = first + (uint32_t)((8 * c + u) / 4) * stride + (uint32_t)(u % 4);
        v[u] = *reinterpret_cast<const float4*>(bm + 4u * (q < n ? q : 0u));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t q = first + (uint32_t)((8 * c + u) / 4) * stride + (uint32_t)(u % 4);
        const uint32_t b = 4u * q;
        uint32_t k = block_key(v[u].x, b, special, special_value, n_blocks);
        k = umax32(k, block_key(v[u].y, b + 1u, special, special_value, n_blocks));
        k = umax32(k, block_key(v[u].z, b + 2u, special, special_value, n_blocks));
        k = umax32(k, block_key(v[u].w, b + 3u, special, special_value, n_blocks));
        keys[8 * c + u] = q < n ? k : 0u;
      }
    }
  }
};

// The blocks of the candidate quads: element i is block cquads[i/4]*4 + i%4 (a negative
// quad id is absent).
struct QuadBlockSrc {
  const float* bm;
  const int32_t* cquads;   // LDS
  uint32_t special;
  float special_value;
  uint32_t n_blocks;
  template <int R>
  __device__ __forceinline__ void load(uint32_t first, uint32_t stride, uint32_t n,
                                       uint32_t (&keys)[R]) const {
    float4 v[R / 4];
    int32_t qd[R / 4];
#pragma unroll
    for (int g = 0; g < R / 4; ++g) {   // 4 consecutive elements = one quad
      const uint32_t i0 = first + g * stride;
      qd[g] = i0 < n ? cquads[i0 >> 2] : -1;
      v[g] = *reinterpret_cast<const float4*>(bm + 4u * (uint32_t)(qd[g] >= 0 ? qd[g] : 0));
    }
#pragma unroll
    for (int g = 0; g < R / 4; ++g) {
      const uint32_t b = 4u * (uint32_t)qd[g];
      const bool ok = qd[g] >= 0;
      keys[4 * g + 0] = ok ? block_key(v[g].x, b, special, special_value, n_blocks) : 0u;
      keys[4 * g + 1] = ok ? block_key(v[g].y, b + 1u, special, special_value, n_blocks) : 0u;
      keys[4 * g + 2] = ok ? block_key(v[g].z, b + 2u, special, special_value, n_blocks) : 0u;
      keys[4 * g + 3] = ok ? block_key(v[g].w, b + 3u, special, special_value, n_blocks) : 0u;
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
  __device__ __forceinline__ void load(uint32_t first, uint32_t stride, uint32_t n,
                                       uint32_t (&keys)[R]) const {
    const uint32_t ns = (uint32_t)n_slots;
    float4 v[R / 4];
    uint32_t s0[R / 4];
#pragma unroll
    for (int g = 0; g < R / 4; ++g) {   // 4 consecutive elements of one block
      const uint32_t i0 = first + g * stride;
      const int32_t b = i0 < n ? cblocks[i0 >> 3] : -1;
      s0[g] = b >= 0 ? (uint32_t)b * 8u + (i0 & 7u) : ns;   // absent block: masked
    }
#pragma unroll
    for (int g = 0; g < R / 4; ++g)
      v[g] = *reinterpret_cast<const float4*>(row + (s0[g] < ns ? s0[g] : 0u));
#pragma unroll
    for (int g = 0; g < R / 4; ++g) {
      const bool ok = s0[g] < ns;
      keys4(v[g], ok ? s0[g] : 0u, ok ? ns : 0u, &keys[4 * g]);
    }
  }
};

// --------------------------------------------------------------------------- kernels

// Rows hold the fewest keys per thread that cover them: 4 up to 4,096 elements, 8 up to
// 8,192, 16 up to 16,384, else 32 (in segments of 32,768 when longer still), so that a
// short row (the decoder Full layer's few hundred elements) costs few ballots, loads and
// emission steps per thread.
template <class Src, class Emit>
__device__ __forceinline__ uint32_t select_any(const Src& src, int64_t n, uint32_t k, SelShared& sh,
                                               Emit emit, uint32_t k2 = 0u, uint32_t cap2 = 0u,
                                               uint32_t* t2 = nullptr) {
  if (n <= (int64_t)SEL_THREADS * 4) {
    KeyRow<Src, 4, false> row(src, n);
    return select_row(row, k, sh, emit, k2, cap2, t2);
  }
  if (n <= (int64_t)SEL_THREADS * 8) {
    KeyRow<Src, 8, false> row(src, n);
    return select_row(row, k, sh, emit, k2, cap2, t2);
  }
  if (n <= (int64_t)SEL_THREADS * 16) {
    KeyRow<Src, 16, false> row(src, n);
    return select_row(row, k, sh, emit, k2, cap2, t2);
  }
  if (n <= (int64_t)SEL_THREADS * 32) {
    KeyRow<Src, 32, false> row(src, n);
    return select_row(row, k, sh, emit, k2, cap2, t2);
  }
  KeyRow<Src, 32, true> row(src, n);
  return select_row(row, k, sh, emit, k2, cap2, t2);
}

// The HSI pool of one query: the n_keep best of its nb block maxima (the forced block
// nb - 1 reads +inf) into sh.obuf in ascending block order; returns how many. With oflag,
// oflag[rank] = 1 marks the pool blocks whose key reaches *t2 (a nonzero *t2). Rows of more
// than 32,768 blocks first keep the n_keep best quads (aligned groups of four blocks,
// ranked by their largest block): a quad left out has n_keep quads ranked above it, each
// holding a block that outranks all of its blocks (ties go to the lower index at both
// levels), so every pool block lies in a kept quad; the pool is then selected among their
// blocks. This replaces several passes over the row by one.
__device__ __forceinline__ uint32_t select_pool(const float* bm_row, int64_t nb, int n_keep,
                                                SelShared& sh, uint32_t k2 = 0u,
                                                uint32_t* t2 = nullptr, uint32_t* oflag = nullptr) {
  const uint32_t kk = (uint32_t)n_keep;
  auto to_obuf = [&](uint32_t rank, uint32_t b, uint32_t f) {
    if (rank < kk) {
      sh.obuf[rank] = (int32_t)b;
      if (oflag != nullptr) oflag[rank] = f;
    }
  };
  if (nb <= (int64_t)SEL_THREADS * 32) {
    const BlockSrc src{bm_row, nb - 1, __builtin_inff()};
    return select_any(src, nb, kk, sh, to_obuf, k2, kk, t2);
  }
  const uint32_t nbu = (uint32_t)nb;
  const QuadSrc qsrc{bm_row, nbu - 1u, __builtin_inff(), nbu};
  const uint32_t n_cq = select_any(qsrc, (nb + 3) >> 2, kk, sh, [&](uint32_t rank, uint32_t q) {
    if (rank < kk) sh.cblocks[rank] = (int32_t)q;
  });
  __syncthreads();
  const QuadBlockSrc bsrc{bm_row, sh.cblocks, nbu - 1u, __builtin_inff(), nbu};
  const uint32_t n_c = n_cq < kk ? n_cq : kk;
  // Element i of the second row is block cblocks[i/4]*4 + i%4.
  return select_any(bsrc, (int64_t)n_c * 4, kk, sh, [&](uint32_t rank, uint32_t i, uint32_t f) {
    if (rank < kk) {
      sh.obuf[rank] = sh.cblocks[i >> 2] * 4 + (int32_t)(i & 3u);
      if (oflag != nullptr) oflag[rank] = f;
    }
  }, k2, kk, t2);
}

// The first min(kept, k) entries of sh.obuf go out, then -1 up to k.
__device__ __forceinline__ void write_out(const SelShared& sh, uint32_t kept, int k, int32_t* orow) {
  for (int r = threadIdx.x; r < k; r += SEL_THREADS) orow[r] = (uint32_t)r < kept ? sh.obuf[r] : -1;
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
  const uint32_t kk = (uint32_t)k;
  auto map = [&](uint32_t slot) -> int32_t {
    if (pool_use != 1) return (int32_t)slot;
    const uint32_t pb = slot >> 3;
    const int32_t b = pb < (uint32_t)n_pool ? pool_blocks[(int64_t)t * n_pool + pb] : -1;
    return b < 0 ? -1 : (int32_t)((uint32_t)b * 8u + (slot & 7u));
  };
  uint32_t kept = 0;
  bool done = false;

  if (pool_use == 1) {
    // Slots past the last live pool entry score nothing: the row ends there (a compacted
    // candidate list fills only its first part).
    const int32_t* prow = pool_blocks + (int64_t)t * n_pool;
    int last = -1;
    for (int i = threadIdx.x; i < n_pool; i += SEL_THREADS) last = prow[i] >= 0 ? i : last;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) last = max(last, __shfl_xor(last, off));
    if ((threadIdx.x & 63) == 0) sh.wmax[threadIdx.x >> 6] = (uint32_t)(last + 1);
    __syncthreads();
    uint32_t live = 0;
#pragma unroll
    for (int i = 0; i < SEL_WAVES; ++i) live = umax32(live, sh.wmax[i]);
    __syncthreads();
    if ((int64_t)live * 8 < n) n = (int64_t)live * 8;
  }
  if (pool_use == 2) {
    // Candidates: the slots of the pool's blocks (ascending block ids, so the winners come
    // out in ascending position order; -1 entries are absent).
    const int32_t* prow = pool_blocks + (int64_t)t * n_pool;
    for (int i = threadIdx.x; i < n_pool; i += SEL_THREADS) sh.cblocks[i] = prow[i];
    __syncthreads();
    const CandSrc csrc{row, sh.cblocks, n};
    kept = select_any(csrc, (int64_t)n_pool * 8, kk, sh, [&](uint32_t rank, uint32_t i) {
      if (rank < kk) sh.obuf[rank] = (int32_t)((uint32_t)sh.cblocks[i >> 3] * 8u + (i & 7u));
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
    auto phase_a = [&](auto& brow) {
      uint32_t count;
      Interval iv;
      row_prepare(brow, count, iv, sh);
      uint32_t thr = 0;   // keep blocks with key >= thr (0: every valid block)
      bool fits = count <= (uint32_t)CAND_BLOCKS_CAP;
      if (count > kk) {
        locate(brow, kk, iv, 0u, (uint32_t)CAND_BLOCKS_CAP, sh);
        thr = iv.A;
        fits = true;
      }
      // Collect candidate blocks (ascending); count them to check the cap.
      const uint32_t n_cand = emit_ordered(brow, thr == 0u ? 0u : thr - 1u, 0u, sh,
                                           [&](uint32_t rank, uint32_t b) {
                                             if (rank < CAND_BLOCKS_CAP) sh.cblocks[rank] = (int32_t)b;
                                           });
      __syncthreads();
      if (fits && n_cand <= (uint32_t)CAND_BLOCKS_CAP) {
        const CandSrc csrc{row, sh.cblocks, n};
        kept = select_any(csrc, (int64_t)n_cand * 8, kk, sh, [&](uint32_t rank, uint32_t i) {
          if (rank < kk) sh.obuf[rank] = map((uint32_t)sh.cblocks[i >> 3] * 8u + (i & 7u));
        });
        done = true;
      }
    };
    // The block maxima stay in registers while they fit (every pass of the threshold
    // search reads them again); longer rows are reloaded segment by segment.
    if (nb <= (int64_t)SEL_THREADS * 16) {
      KeyRow<BlockSrc, 16, false> brow(bsrc, nb);
      phase_a(brow);
    } else if (nb <= (int64_t)SEL_THREADS * 32) {
      KeyRow<BlockSrc, 32, false> brow(bsrc, nb);
      phase_a(brow);
    } else {
      KeyRow<BlockSrc, 32, true> brow(bsrc, nb);
      phase_a(brow);
    }
  }
  if (!done) {
    const ScoreSrc ssrc{row};
    kept = select_any(ssrc, n, kk, sh, [&](uint32_t rank, uint32_t i) {
      if (rank < kk) sh.obuf[rank] = map(i);
    });
  }
  __syncthreads();
  write_out(sh, kept, k, out + (int64_t)t * ld_idx);
}

__global__ __launch_bounds__(SEL_THREADS) void block_pool_kernel(
    const float* __restrict__ block_max, int64_t ld_bm, const int32_t* __restrict__ n_visible,
    int n_keep, int32_t* __restrict__ pool, int64_t ld_pool) {
  __shared__ SelShared sh;
  const int t = blockIdx.x;
  const int64_t nv = n_visible[t];
  int64_t nb = nv > 0 ? (nv + 7) >> 3 : 0;
  if (nb > ld_bm) nb = ld_bm;
  const uint32_t kept = select_pool(block_max + (int64_t)t * ld_bm, nb, n_keep, sh);
  __syncthreads();
  write_out(sh, kept, n_keep, pool + (int64_t)t * ld_pool);
}

// The HSI pool and the Top-K among its candidates in one workgroup per query: the pool is
// written out and kept in LDS, and the candidate selection reads its block list from there
// (the same results as block_pool_kernel followed by topk_kernel with pool_use 2).
__global__ __launch_bounds__(SEL_THREADS) void pool_topk_kernel(
    const float* __restrict__ block_max, int64_t ld_bm, const int32_t* __restrict__ n_visible,
    int n_keep, int32_t* __restrict__ pool, int64_t ld_pool, const float* __restrict__ scores,
    int64_t ld, int64_t n_cols, int k, int32_t* __restrict__ out, int64_t ld_idx) {
  __shared__ SelShared sh;
  const int t = blockIdx.x;
  const int64_t nv = n_visible[t];
  int64_t nb = nv > 0 ? (nv + 7) >> 3 : 0;
  if (nb > ld_bm) nb = ld_bm;
  const uint32_t kept_pool = select_pool(block_max + (int64_t)t * ld_bm, nb, n_keep, sh);
  __syncthreads();
  int32_t* prow = pool + (int64_t)t * ld_pool;
  for (int r = threadIdx.x; r < n_keep; r += SEL_THREADS) {
    const int32_t b = (uint32_t)r < kept_pool ? sh.obuf[r] : -1;
    prow[r] = b;
    sh.cblocks[r] = b;
  }
  __syncthreads();
  const int64_t n = nv < 0 ? 0 : (nv < n_cols ? nv : n_cols);
  const uint32_t kk = (uint32_t)k;
  const CandSrc csrc{scores + (int64_t)t * ld, sh.cblocks, n};
  const uint32_t kept = select_any(csrc, (int64_t)n_keep * 8, kk, sh, [&](uint32_t rank, uint32_t i) {
    if (rank < kk) sh.obuf[rank] = (int32_t)((uint32_t)sh.cblocks[i >> 3] * 8u + (i & 7u));
  });
  __syncthreads();
  write_out(sh, kept, k, out + (int64_t)t * ld_idx);
}

// The HSI pool and, for the Full layer of the same scores, its candidate blocks: the pool
// blocks whose maximum reaches a threshold that the (k+1)-th best block (the forced block
// counted first) reaches. A block holding one of the k best entries has fewer than k blocks
// ranked above it by (maximum desc, id asc), each of which holds a better entry of its own,
// so it is among the k best real blocks and reaches the threshold. The threshold comes from
// the pool selection's first histogram pass at no extra pass over the row; when that pass
// cannot give one, every pool block is a candidate. Candidates keep the pool's ascending
// order and are -1 padded like it.
__global__ __launch_bounds__(SEL_THREADS) void block_pool_cand_kernel(
    const float* __restrict__ block_max, int64_t ld_bm, const int32_t* __restrict__ n_visible,
    int n_keep, int32_t* __restrict__ pool, int64_t ld_pool, int k,
    int32_t* __restrict__ cand, int64_t ld_cand) {
  __shared__ SelShared sh;
  const int t = blockIdx.x;
  const int64_t nv = n_visible[t];
  int64_t nb = nv > 0 ? (nv + 7) >> 3 : 0;
  if (nb > ld_bm) nb = ld_bm;
  const float* bm_row = block_max + (int64_t)t * ld_bm;
  uint32_t t2 = 0u;
  const uint32_t kept = select_pool(bm_row, nb, n_keep, sh, (uint32_t)k + 1u, &t2);
  __syncthreads();
  int32_t* prow = pool + (int64_t)t * ld_pool;
  int32_t* crow = cand + (int64_t)t * ld_cand;
  if (t2 == 0u) {
    for (int r = threadIdx.x; r < n_keep; r += SEL_THREADS) {
      const int32_t b = (uint32_t)r < kept ? sh.obuf[r] : -1;
      prow[r] = b;
      crow[r] = b;
    }
    return;
  }
  // Thread tid flags the pool entries of ranks 2*tid and 2*tid + 1 (n_keep <= 2,048), so one
  // block scan in thread order keeps the candidates in ascending block order.
  const uint32_t forced = (uint32_t)nb - 1u;
  uint32_t f[2];
  int32_t bl[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t r = 2u * threadIdx.x + j;
    bl[j] = r < kept ? sh.obuf[r] : -1;
    const float v = bl[j] >= 0 ? bm_row[bl[j]] : 0.f;
    const uint32_t key = bl[j] < 0 ? 0u : block_key(v, (uint32_t)bl[j], forced, __builtin_inff(),
                                                    (uint32_t)nb);
    f[j] = key >= t2 ? 1u : 0u;
  }
  uint32_t total;
  const uint32_t excl = block_exclusive_scan(f[0] + f[1], sh, &total);
  if (f[0]) crow[excl] = bl[0];
  if (f[1]) crow[excl + f[0]] = bl[1];
  for (int r = threadIdx.x; r < n_keep; r += SEL_THREADS) {
    prow[r] = (uint32_t)r < kept ? sh.obuf[r] : -1;
    if ((uint32_t)r >= total) crow[r] = -1;
  }
}

// The decoder Full layer's whole selection in one workgroup per query: the HSI pool and
// its candidate blocks (as block_pool_cand_kernel), then the Top-K among the candidates'
// positions (as topk_kernel with pool_use 2 over their rescored slots would give it) from
// the Full pass's block statistics. A winner of the Top-K lies in a candidate block and is
// either the block's argmax, whose score is the block maximum, or another slot, whose score
// is at most the block's second score; and the k-th best score is at least the threshold t2
// that the candidates reach (k real blocks reach it, each through its own argmax). So each
// candidate block contributes its argmax with its maximum, except the few whose stored
// second key reaches t2: those are rescored, all 8 slots, with the layer's indexer query
// (e4m3_step_score or mxfp4_step_score, the Full pass's own arithmetic, so bit-identical
// scores; FP4K selects MXFP4 keys, codes in k_cache and scales in k_scales). The elements
// are laid out in ascending position order, so ties go to the lower position and the
// winners come out ascending, exactly as from the separate calls. Without a threshold, or
// with more elements than fit, every candidate block is rescored.
constexpr int FS_SLOTS = CAND_BLOCKS_CAP * 8;   // 16,384: every slot of every candidate
constexpr int FS_ELEMS = FS_SLOTS / 2;          // element scores and positions side by side

struct FullSelShared {
  SelShared sel;
  union {
    float cscore[FS_SLOTS];   // all rescored: score of candidate slot i
    struct {
      float escore[FS_ELEMS];   // element scores, ascending position order
      int32_t epos[FS_ELEMS];   // their positions
    } el;
  };
};

// Scores held in LDS, read as a key row.
struct LdsScoreSrc {
  const float* s;
  template <int R>
  __device__ __forceinline__ void load(uint32_t first, uint32_t stride, uint32_t n,
                                       uint32_t (&keys)[R]) const {
#pragma unroll
    for (int g = 0; g < R / 4; ++g) {
      const uint32_t i0 = first + g * stride;
      const float4 v = *reinterpret_cast<const float4*>(s + (i0 < n ? i0 : 0u));
      keys4(v, i0, n, &keys[4 * g]);
    }
  }
};

template <bool FP4K>
__global__ __launch_bounds__(SEL_THREADS) void full_select_kernel(
    const float* __restrict__ block_max, int64_t ld_bm, const int32_t* __restrict__ n_visible,
    int n_keep, int32_t* __restrict__ pool, int64_t ld_pool, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w, const uint8_t* __restrict__ k_cache,
    const uint8_t* __restrict__ k_scales, int64_t n_entries,
    const int64_t* __restrict__ kv_start, const uint32_t* __restrict__ block_aux, int k,
    int32_t* __restrict__ out, int64_t ld_idx) {
  __shared__ FullSelShared fs;
  SelShared& sh = fs.sel;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int half = lane >> 5;

  const int64_t nv = n_visible[t];
  const int64_t base = kv_start[t];
  int64_t nb = nv > 0 ? (nv + 7) >> 3 : 0;
  if (nb > ld_bm) nb = ld_bm;
  const float* bm_row = block_max + (int64_t)t * ld_bm;
  const uint32_t* aux_row = block_aux + (int64_t)t * ld_bm;
  uint32_t t2 = 0u;
  // The pool's candidate flags go to the element area, free until the elements are laid out.
  uint32_t* pflag = reinterpret_cast<uint32_t*>(fs.el.escore);
  const uint32_t kept = select_pool(bm_row, nb, n_keep, sh, (uint32_t)k + 1u, &t2, pflag);
  __syncthreads();

  // Indexer operands. Rescoring steps go to wavefronts 0, 1, 2, ... in turn and are usually
  // few (a handful of blocks), so only the first FS_EARLY_WAVES wavefronts load the operands
  // here, after the pool selection's registers are free (every wavefront loading them costs
  // the next phase thousands of cycles of memory-instruction issue); a later wavefront loads
  // them when it is given a step.
  bf16x8 a[8];
  float wr[16];
  auto load_operands = [&]() {
    const uint16_t* qrow = q_idx + ((int64_t)t * 32 + n) * 128 + 64 * half;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) a[kb] = *reinterpret_cast<const bf16x8*>(qrow + 8 * kb);
#pragma unroll
    for (int r = 0; r < 16; ++r) wr[r] = w[(int64_t)t * 32 + 8 * (r >> 2) + 4 * half + (r & 3)];
  };
  const bool early = wave < FS_EARLY_WAVES;   // uniform
  if (early) load_operands();

  // The pool goes out. Its candidate blocks (those whose key reaches t2, or all of it when
  // the first pass gave no threshold) stay in LDS in ascending order with their block
  // maxima and statistics words, whose loads are issued before the scan that places them.
  float* cval = reinterpret_cast<float*>(sh.gpos);  // candidate block maxima
  uint32_t* caux = sh.gpos + CAND_BLOCKS_CAP;       // candidate statistics words
  int32_t* prow = pool + (int64_t)t * ld_pool;
  uint32_t n_c;
  {
    uint32_t f[2], word[2];
    float val[2];
    int32_t bl[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t r = 2u * tid + j;
      bl[j] = r < kept && r < (uint32_t)n_keep ? sh.obuf[r] : -1;
      f[j] = bl[j] >= 0 && (t2 == 0u || pflag[r] != 0u) ? 1u : 0u;
      word[j] = f[j] ? aux_row[bl[j]] : 0u;
      val[j] = f[j] ? bm_row[bl[j]] : 0.f;
    }
    uint32_t total;
    const uint32_t excl = block_exclusive_scan(f[0] + f[1], sh, &total);
    for (int r = tid; r < n_keep; r += SEL_THREADS)
      prow[r] = (uint32_t)r < kept ? sh.obuf[r] : -1;
    uint32_t c = excl;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (f[j]) {
        sh.cblocks[c] = bl[j];
        cval[c] = val[j];
        caux[c] = word[j];
        ++c;
      }
    }
    n_c = total;
  }
  __syncthreads();

  // Elements: thread tid lays out candidate ranks 2*tid and 2*tid + 1. One scan gives the
  // element offsets (low 16 bits) and the rescored-block ranks (high 16 bits). A block that
  // is not rescored contributes its argmax with the block maximum.
  int32_t cb[2];
  uint32_t cnt[2], rs[2], amax[2];
  float cv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t r = 2u * tid + j;
    cb[j] = r < n_c ? sh.cblocks[r] : -1;
    const uint32_t word = cb[j] >= 0 ? caux[r] : 0u;
    cv[j] = cb[j] >= 0 ? cval[r] : 0.f;
    rs[j] = cb[j] >= 0 && (t2 == 0u || (word & ~7u) >= t2) ? 1u : 0u;
    cnt[j] = cb[j] < 0 ? 0u : (rs[j] ? 8u : 1u);
    amax[j] = word & 7u;   // the block's argmax slot
  }
  uint32_t total;
  const uint32_t excl = block_exclusive_scan((cnt[0] + cnt[1]) | ((rs[0] + rs[1]) << 16), sh,
                                             &total);
  const uint32_t n_el = total & 0xFFFFu;
  const uint32_t n_r = total >> 16;
  const bool mixed = n_el <= (uint32_t)FS_ELEMS;
  int32_t* rblk = sh.obuf;                               // rescored blocks (mixed layout)
  uint32_t* roff = sh.gpos + 2 * CAND_BLOCKS_CAP;        // their first element
  if (mixed) {
    uint32_t e = excl & 0xFFFFu;
    uint32_t rr = excl >> 16;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (cb[j] < 0) continue;
      if (rs[j]) {
        rblk[rr] = cb[j];
        roff[rr] = e;
        ++rr;
      } else {
        fs.el.escore[e] = cv[j];
        fs.el.epos[e] = cb[j] * 8 + (int32_t)amax[j];
      }
      e += cnt[j];
    }
  }
  __syncthreads();

  // Rescoring: 32-slot steps of four blocks (the rescored ones, or every candidate), taken
  // by the 16 wavefronts in turn, each loading its next step's rows while it multiplies the
  // current one.
  const uint32_t n_blk = mixed ? n_r : n_c;
  const int n_steps = (int)((n_blk + 3) / 4);
  const bool any = nv > 0 && base >= 0 && base < n_entries;
  auto block_of = [&](int step) -> int32_t {
    const uint32_t j = 4u * (uint32_t)step + (uint32_t)(n >> 3);
    if (j >= n_blk) return -1;
    return mixed ? rblk[j] : sh.cblocks[j];
  };
  auto row_of = [&](int32_t b) -> int64_t {
    if (b < 0) return -1;
    const int64_t pos = (int64_t)b * 8 + (n & 7);
    if (pos >= nv) return -1;
    const int64_t row = base + pos;
    return (row >= 0 && row < n_entries) ? row : -1;
  };
  auto load_rows = [&](int64_t r, u32x4 (&raw)[4]) {
    const int64_t rr = r >= 0 ? r : base;
    if constexpr (FP4K) {
      const u32x4* p = reinterpret_cast<const u32x4*>(k_cache + rr * 64 + 32 * half);
      raw[0] = p[0];
      raw[1] = p[1];
      raw[2].x = *reinterpret_cast<const uint32_t*>(k_scales + rr * 4);
      return;
    }
    const u32x4* p = reinterpret_cast<const u32x4*>(k_cache + rr * 128 + 64 * half);
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = p[i];
  };
  auto put = [&](int step, int32_t b, float sv) {
    const uint32_t j = 4u * (uint32_t)step + (uint32_t)(n >> 3);
    if (half != 0 || j >= n_blk) return;
    if (mixed) {
      const uint32_t e = roff[j] + (uint32_t)(n & 7);
      fs.el.escore[e] = sv;
      fs.el.epos[e] = b * 8 + (n & 7);
    } else {
      fs.cscore[8 * j + (uint32_t)(n & 7)] = sv;
    }
  };
  if (any) {
    if (!early && wave < n_steps) load_operands();
    u32x4 cur[4], nxt[4];
    int32_t bc = wave < n_steps ? block_of(wave) : -1;
    int64_t rc = row_of(bc);
    if (wave < n_steps) load_rows(rc, cur);
    for (int st = wave; st < n_steps; st += SEL_WAVES) {
      int32_t bn = -1;
      int64_t rn = -1;
      if (st + SEL_WAVES < n_steps) {
        bn = block_of(st + SEL_WAVES);
        rn = row_of(bn);
        load_rows(rn, nxt);
      }
      const float sv = FP4K ? mxfp4_step_score(a, wr, cur, half) : e4m3_step_score(a, wr, cur);
      put(st, bc, rc >= 0 ? sv : -__builtin_inff());
#pragma unroll
      for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
      bc = bn;
      rc = rn;
    }
  } else {
    for (int st = wave; st < n_steps; st += SEL_WAVES) put(st, block_of(st), -__builtin_inff());
  }
  __syncthreads();

  // The Top-K among the elements (ascending position order), emitted ascending.
  const uint32_t kk = (uint32_t)k;
  uint32_t kept_k;
  if (mixed) {
    const LdsScoreSrc src{fs.el.escore};
    kept_k = select_any(src, (int64_t)n_el, kk, sh, [&](uint32_t rank, uint32_t i) {
      if (rank < kk) sh.obuf[rank] = fs.el.epos[i];
    });
  } else {
    const LdsScoreSrc src{fs.cscore};
    kept_k = select_any(src, (int64_t)n_c * 8, kk, sh, [&](uint32_t rank, uint32_t i) {
      if (rank < kk) sh.obuf[rank] = (int32_t)((uint32_t)sh.cblocks[i >> 3] * 8u + (i & 7u));
    });
  }
  __syncthreads();
  write_out(sh, kept_k, k, out + (int64_t)t * ld_idx);
}

hipError_t launch_full_select(int n_q, const float* block_max, int64_t ld_bm,
                              const int32_t* n_visible, int n_keep, int32_t* pool_blocks,
                              int64_t ld_pool, const uint16_t* q_idx, const float* w,
                              const uint8_t* k_cache, const uint8_t* k_scales, int64_t n_entries,
                              const int64_t* kv_start, const uint32_t* block_aux, int k,
                              int32_t* topk_idx, int64_t ld_idx, hipStream_t stream) {
  if (k_scales != nullptr)
    hipLaunchKernelGGL(full_select_kernel<true>, dim3(n_q), dim3(SEL_THREADS), 0, stream,
                       block_max, ld_bm, n_visible, n_keep, pool_blocks, ld_pool, q_idx, w,
                       k_cache, k_scales, n_entries, kv_start, block_aux, k, topk_idx, ld_idx);
  else
    hipLaunchKernelGGL(full_select_kernel<false>, dim3(n_q), dim3(SEL_THREADS), 0, stream,
                       block_max, ld_bm, n_visible, n_keep, pool_blocks, ld_pool, q_idx, w,
                       k_cache, k_scales, n_entries, kv_start, block_aux, k, topk_idx, ld_idx);
  return hipGetLastError();
}

hipError_t launch_block_pool_cand(int n_q, const float* block_max, int64_t ld_bm,
                                  const int32_t* n_visible, int n_keep, int32_t* pool_blocks,
                                  int64_t ld_pool, int k, int32_t* cand_blocks, int64_t ld_cand,
                                  hipStream_t stream) {
  hipLaunchKernelGGL(block_pool_cand_kernel, dim3(n_q), dim3(SEL_THREADS), 0, stream, block_max,
                     ld_bm, n_visible, n_keep, pool_blocks, ld_pool, k, cand_blocks, ld_cand);
  return hipGetLastError();
}

hipError_t launch_pool_topk(int n_q, const float* block_max, int64_t ld_bm,
                            const int32_t* n_visible, int n_keep, int32_t* pool_blocks,
                            int64_t ld_pool, const float* scores, int64_t ld_scores,
                            int64_t n_cols, int k, int32_t* topk_idx, int64_t ld_idx,
                            hipStream_t stream) {
  hipLaunchKernelGGL(pool_topk_kernel, dim3(n_q), dim3(SEL_THREADS), 0, stream, block_max, ld_bm,
                     n_visible, n_keep, pool_blocks, ld_pool, scores, ld_scores, n_cols, k,
                     topk_idx, ld_idx);
  return hipGetLastError();
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
