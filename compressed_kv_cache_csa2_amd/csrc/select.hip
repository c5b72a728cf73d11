// Exact Top-K and HSI block-pool selection on gfx950.
//
// Both selections keep the k largest values of a row under the order (value descending,
// index ascending), never keep -inf or NaN, and emit the kept indices in ascending
// order. That is the Top-512 of the indexer scores and the top-2,048 block maxima of the
// Hierarchical Sparse Indexer ("DeepSeek-v4.1 Flash: Pushing the Limits of KV Cache
// Compression", 2.3.4; "DeepSeek-V4.1-Flash - Architecture", section 3).
//
// One 512-thread workgroup per query row. Values become order-preserving 32-bit keys
// (0 marks an element that cannot be selected); thread t owns 64 consecutive elements and
// keeps their keys in registers (rows longer than 32,768 are walked in segments).
//   1. A block reduction gives the count, the smallest and the largest key.
//   2. Range refinement: the live key interval [A, B] is split into at most 2,048 equal
//      power-of-two bins, an LDS histogram of the keys inside [A, B] is taken, and the bin
//      holding the k-th largest key becomes the new interval. Bins follow the data's own
//      key range, so the first histogram spreads over many bins (few atomic collisions);
//      the interval shrinks by 2^11 per pass, so three passes at most reach one key tau.
//   3. Emission: every key > tau is kept, and of the keys == tau the lowest-indexed
//      (k - #greater). Two block-wide prefix sums (ties, then kept) give each thread its
//      output offsets; output is deterministic and sorted by index.
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

constexpr int SEL_THREADS = 512;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_R = 64;                       // keys per thread per segment
constexpr int SEL_SEG = SEL_THREADS * SEL_R;    // 32,768 keys per segment
constexpr int NBINS = 2048;
constexpr int CAND_BLOCKS_CAP = 2048;
constexpr int BINS_PER_THREAD = NBINS / SEL_THREADS;

struct SelShared {
  uint32_t hist[NBINS];
  uint32_t wsum[SEL_WAVES];
  uint32_t wmin[SEL_WAVES];
  uint32_t wmax[SEL_WAVES];
  uint32_t scal[4];
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

// The keys of one row: thread tid holds elements seg*SEG + tid*R + r in keys[r].
template <class Src>
struct KeyRow {
  Src src;
  int64_t n;
  int nseg;
  uint32_t keys[SEL_R];
  int loaded;

  __device__ __forceinline__ KeyRow(const Src& s, int64_t n_) : src(s), n(n_), nseg((int)((n_ + SEL_SEG - 1) / SEL_SEG)), loaded(-1) {}

  __device__ __forceinline__ void load(int seg) {
    if (seg == loaded) return;
    const int64_t base = (int64_t)seg * SEL_SEG + (int64_t)threadIdx.x * SEL_R;
    src.load(base, n, keys);
    loaded = seg;
  }
};

// Refinement passes over [A, B], which holds the k-th largest key; `need` is how many
// keys to take from [A, B] (so k - need keys lie above B). Stops when A == B (then A is
// the k-th largest key and `need` keys equal to it are taken), or, when cap > 0, as soon
// as at most cap keys are >= A (A is then a lower bound of the k-th largest key).
template <class Row>
__device__ __forceinline__ void refine(Row& row, uint32_t& A, uint32_t& B, uint32_t& need, uint32_t k,
                       uint32_t cap, SelShared& sh) {
  const int tid = threadIdx.x;
#pragma unroll 1
  while (A != B) {
    const uint32_t span = B - A;
    const int bits = 32 - __clz(span);                 // span < 2^bits
    const int s = bits > 11 ? bits - 11 : 0;           // (span >> s) < 2048
#pragma unroll
    for (int j = 0; j < BINS_PER_THREAD; ++j) sh.hist[tid + j * SEL_THREADS] = 0;
    __syncthreads();
    for (int seg = 0; seg < row.nseg; ++seg) {
      row.load(seg);
#pragma unroll
      for (int r = 0; r < SEL_R; ++r) {
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
        sh.scal[2] = above + h[j];
      }
      above += h[j];
    }
    __syncthreads();
    const uint32_t b = sh.scal[0];
    const uint32_t above_b = sh.scal[1];
    const uint32_t through = sh.scal[2];
    __syncthreads();
    const uint64_t lo = (uint64_t)A + ((uint64_t)b << s);
    const uint64_t hi = lo + (1ull << s) - 1;
    const uint32_t ge = (k - need) + through;   // keys >= the new A
    need -= above_b;
    A = (uint32_t)lo;
    B = hi < (uint64_t)B ? (uint32_t)hi : B;
    if (cap != 0u && ge <= cap) break;
  }
}

// Count / min / max of the valid keys of the row.
template <class Row>
__device__ __forceinline__ void row_stats(Row& row, uint32_t& count, uint32_t& kmin, uint32_t& kmax,
                          SelShared& sh) {
  uint32_t c = 0, mn = 0xFFFFFFFFu, mx = 0u;
  for (int seg = 0; seg < row.nseg; ++seg) {
    row.load(seg);
#pragma unroll
    for (int r = 0; r < SEL_R; ++r) {
      const uint32_t key = row.keys[r];
      if (key != 0u) {
        ++c;
        mn = umin32(mn, key);
        mx = umax32(mx, key);
      }
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

// Emit, in ascending index order, every key > tau and the first n_eq keys == tau
// (tau = 0 with n_eq = 0 keeps every valid key). emit(rank, index). Returns the count.
template <class Row, class Emit>
__device__ __forceinline__ uint32_t emit_ordered(Row& row, uint32_t tau, uint32_t n_eq, SelShared& sh,
                                 Emit emit) {
  uint32_t eq_base = 0, out_base = 0;
  for (int seg = 0; seg < row.nseg; ++seg) {
    row.load(seg);
    uint64_t gt_mask = 0, eq_mask = 0;
#pragma unroll
    for (int r = 0; r < SEL_R; ++r) {
      const uint32_t key = row.keys[r];
      gt_mask |= (uint64_t)(key != 0u && key > tau) << r;
      eq_mask |= (uint64_t)(key != 0u && key == tau) << r;
    }
    const uint32_t n_e = __popcll(eq_mask);
    uint32_t eq_total;
    const uint32_t eq_before = eq_base + block_exclusive_scan(n_e, sh, &eq_total);
    // ties kept by this thread: ranks eq_before .. eq_before + n_e - 1 below n_eq
    const uint32_t eq_keep = eq_before >= n_eq ? 0u : umin32(n_e, n_eq - eq_before);
    // keep the first eq_keep set bits of eq_mask
    uint64_t take = gt_mask;
    uint32_t seen = 0;
#pragma unroll
    for (int r = 0; r < SEL_R; ++r) {
      const uint32_t bit = (uint32_t)(eq_mask >> r) & 1u;
      take |= (uint64_t)(bit != 0u && seen < eq_keep) << r;
      seen += bit;
    }
    uint32_t take_total;
    uint32_t pos = out_base + block_exclusive_scan(__popcll(take), sh, &take_total);
    const int64_t base = (int64_t)seg * SEL_SEG + (int64_t)threadIdx.x * SEL_R;
    while (take != 0ull) {
      const int r = __builtin_ctzll(take);
      take &= take - 1ull;
      emit(pos++, base + r);
    }
    eq_base += eq_total;
    out_base += take_total;
  }
  return out_base;
}

// Full exact selection of the k best keys of a row.
template <class Row, class Emit>
__device__ __forceinline__ uint32_t select_row(Row& row, uint32_t k, SelShared& sh, Emit emit) {
  uint32_t count, A, B;
  row_stats(row, count, A, B, sh);
  if (count <= k) return emit_ordered(row, 0u, 0u, sh, emit);
  uint32_t need = k;
  refine(row, A, B, need, k, 0u, sh);
  return emit_ordered(row, A, need, sh, emit);
}

// --------------------------------------------------------------------------- key sources

// Rows are 16-byte aligned with a leading dimension that is a multiple of 4 (checked by
// the C ABI), so a float4 starting below n never leaves its row. Every source issues all
// of a segment's loads before using any (an element past the end reads the row's first
// float4 and is masked afterwards), so a segment costs one memory round trip.
__device__ __forceinline__ void keys4(float4 v, int64_t i0, int64_t n, uint32_t* k) {
  const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) k[j] = (i0 + j < n && selectable(f[j])) ? float_key(f[j]) : 0u;
}

// Scores of a row (float array), keys of slots i < n.
struct ScoreSrc {
  const float* row;
  __device__ __forceinline__ void load(int64_t base, int64_t n, uint32_t (&keys)[SEL_R]) const {
    float4 v[SEL_R / 4];
#pragma unroll
    for (int q = 0; q < SEL_R / 4; ++q) {
      const int64_t i0 = base + 4 * q;
      v[q] = *reinterpret_cast<const float4*>(row + (i0 < n ? i0 : 0));
    }
#pragma unroll
    for (int q = 0; q < SEL_R / 4; ++q) keys4(v[q], base + 4 * q, n, &keys[4 * q]);
  }
};

// Block maxima with an override for one block (forced +inf for the pool, or a recomputed
// maximum for a partial last block in the Top-K prefilter).
struct BlockSrc {
  const float* bm;
  int64_t special;
  float special_value;
  __device__ __forceinline__ void load(int64_t base, int64_t n, uint32_t (&keys)[SEL_R]) const {
    float4 v[SEL_R / 4];
#pragma unroll
    for (int q = 0; q < SEL_R / 4; ++q) {
      const int64_t i0 = base + 4 * q;
      v[q] = *reinterpret_cast<const float4*>(bm + (i0 < n ? i0 : 0));
    }
#pragma unroll
    for (int q = 0; q < SEL_R / 4; ++q) {
      const int64_t i0 = base + 4 * q;
      if (special >= i0 && special < i0 + 4) {
        const int j = (int)(special - i0);
        if (j == 0) v[q].x = special_value;
        if (j == 1) v[q].y = special_value;
        if (j == 2) v[q].z = special_value;
        if (j == 3) v[q].w = special_value;
      }
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
  __device__ __forceinline__ void load(int64_t base, int64_t n, uint32_t (&keys)[SEL_R]) const {
    float4 v[SEL_R / 4];
    int64_t s0[SEL_R / 4];
#pragma unroll
    for (int q = 0; q < SEL_R / 4; ++q) {   // 4 consecutive elements of one block
      const int64_t i0 = base + 4 * q;
      const int32_t b = i0 < n ? cblocks[i0 >> 3] : -1;
      s0[q] = b >= 0 ? (int64_t)b * 8 + (i0 & 7) : n_slots;   // absent block: masked
    }
#pragma unroll
    for (int q = 0; q < SEL_R / 4; ++q)
      v[q] = *reinterpret_cast<const float4*>(row + (s0[q] < n_slots ? s0[q] : 0));
#pragma unroll
    for (int q = 0; q < SEL_R / 4; ++q) {
      const bool ok = s0[q] < n_slots;
      keys4(v[q], ok ? s0[q] : 0, ok ? n_slots : 0, &keys[4 * q]);
    }
  }
};

// --------------------------------------------------------------------------- kernels

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
    KeyRow<CandSrc> crow(csrc, (int64_t)n_pool * 8);
    kept = select_row(crow, kk, sh, [&](uint32_t rank, int64_t i) {
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
    KeyRow<BlockSrc> brow(bsrc, nb);
    uint32_t count, A, B;
    row_stats(brow, count, A, B, sh);
    uint32_t thr = 0;   // keep blocks with key >= thr (0: every valid block)
    bool fits = count <= (uint32_t)CAND_BLOCKS_CAP;
    if (count > kk) {
      uint32_t need = kk;
      refine(brow, A, B, need, kk, (uint32_t)CAND_BLOCKS_CAP, sh);
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
      KeyRow<CandSrc> crow(csrc, (int64_t)n_cand * 8);
      kept = select_row(crow, kk, sh, [&](uint32_t rank, int64_t i) {
        if (rank < kk) orow[rank] = map((int64_t)sh.cblocks[i >> 3] * 8 + (i & 7));
      });
      done = true;
    }
  }
  if (!done) {
    const ScoreSrc ssrc{row};
    KeyRow<ScoreSrc> srow(ssrc, n);
    kept = select_row(srow, kk, sh, [&](uint32_t rank, int64_t i) {
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
  KeyRow<BlockSrc> row(src, nb);
  const uint32_t kept = select_row(row, (uint32_t)n_keep, sh, [&](uint32_t rank, int64_t b) {
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
