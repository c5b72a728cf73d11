// Exact Top-K and HSI block-pool selection on gfx950.
//
// Both selections keep the k largest values of a row under the order (value descending,
// index ascending), never keep -inf or NaN, and emit the kept indices in ascending
// order. That is the Top-512 of the indexer scores and the top-2,048 block maxima of the
// Hierarchical Sparse Indexer ("DeepSeek-v4.1 Flash: Pushing the Limits of KV Cache
// Compression", 2.3.4; "DeepSeek-V4.1-Flash - Architecture", section 3).
//
// One 1024-thread workgroup per query row:
//   1. radix select on order-preserving 32-bit keys, three passes of 11/11/10 bits with
//      an LDS histogram each, finds the k-th largest key tau and how many keys exceed it;
//   2. one ordered pass keeps every key > tau and the first (k - #greater) keys == tau in
//      index order. Ranks come from wave ballots and a 16-wave prefix, so the output is
//      deterministic and already sorted.
// Rows that fit in LDS are staged there once; longer rows are streamed from global
// memory (L2/MALL-resident right after the indexer wrote them).
//
// Block prefilter for Top-K: if block maxima of 8-slot blocks are given, the k-th largest
// block maximum m_k bounds the k-th largest score from below (k blocks each hold a score
// >= m_k), so every winner lies in a block whose maximum is >= m_k. Only those blocks'
// scores are gathered (usually k*8 = 4,096 slots instead of the whole row) and selected
// exactly; ties at the threshold keep every tied block, and if more than 2,048 blocks
// tie the kernel falls back to the full row.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int KEYS_CAP = 16384;
constexpr int CAND_BLOCKS_CAP = 2048;

struct SelShared {
  uint32_t hist[2048];
  uint32_t keys[KEYS_CAP];
  int32_t cblocks[CAND_BLOCKS_CAP];
  uint32_t wsum[SEL_WAVES];
  uint32_t wsum2[SEL_WAVES];
  uint32_t scal[4];
};

// Inclusive prefix sum over the 1024 threads of the block; *total receives the sum.
__device__ uint32_t block_inclusive_scan(uint32_t v, SelShared& sh, uint32_t* total) {
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
  for (int i = 0; i < SEL_WAVES; ++i) {
    const uint32_t s = sh.wsum[i];
    before += i < wave ? s : 0u;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + x;
}

struct KthResult {
  uint32_t tau;     // k-th largest key (0 when total <= k: every valid key qualifies)
  uint32_t n_take_eq;  // how many keys equal to tau are kept
  uint32_t total;   // number of valid keys
};

// Key source: get(i, &key) returns false for an element that cannot be selected.
template <class Get>
__device__ KthResult radix_kth(Get get, int64_t n, uint32_t k, SelShared& sh) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0, need = k;
  KthResult res{0u, 0u, 0u};
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int width = pass == 2 ? 10 : 11;
    const uint32_t dmask = (1u << width) - 1u;
    sh.hist[tid] = 0;
    sh.hist[tid + SEL_THREADS] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += SEL_THREADS) {
      uint32_t key;
      if (get(i, key) && (key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    // Thread tid owns bins 2*tid and 2*tid+1 (bins beyond the digit range are zero).
    const uint32_t h0 = sh.hist[2 * tid], h1 = sh.hist[2 * tid + 1];
    uint32_t total;
    const uint32_t incl = block_inclusive_scan(h0 + h1, sh, &total);
    if (pass == 0) {
      res.total = total;
      if (total <= k) return res;  // every valid key is kept
    }
    const uint32_t above1 = total - incl;      // keys in bins above 2*tid+1
    const uint32_t above0 = above1 + h1;       // keys in bins above 2*tid
    if (above1 < need && need <= above1 + h1) {
      sh.scal[0] = 2 * tid + 1;
      sh.scal[1] = above1;
    } else if (above0 < need && need <= above0 + h0) {
      sh.scal[0] = 2 * tid;
      sh.scal[1] = above0;
    }
    __syncthreads();
    const uint32_t d = sh.scal[0];
    need -= sh.scal[1];
    prefix |= d << shift;
    mask |= dmask << shift;
    __syncthreads();
  }
  res.tau = prefix;
  res.n_take_eq = need;
  return res;
}

// Keeps keys > tau and the first n_take_eq keys == tau in index order; emit(rank, i) is
// called with consecutive ranks in ascending i. Returns the number kept. With
// take_all_eq every key >= tau is kept.
template <class Get, class Emit>
__device__ uint32_t collect_ordered(Get get, int64_t n, uint32_t tau, uint32_t n_take_eq,
                                    bool take_all_eq, SelShared& sh, Emit emit) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t eq_base = 0, out_base = 0;
#pragma unroll 1
  for (int64_t c0 = 0; c0 < n; c0 += SEL_THREADS) {
    const int64_t i = c0 + tid;
    uint32_t key = 0;
    const bool valid = i < n && get(i, key);
    const bool gt = valid && key > tau;
    const bool eq = valid && key == tau;
    const uint64_t m_eq = __ballot(eq);
    if (lane == 0) sh.wsum[wave] = __popcll(m_eq);
    __syncthreads();
    uint32_t eq_before = 0, eq_total = 0;
    for (int w = 0; w < SEL_WAVES; ++w) {
      const uint32_t s = sh.wsum[w];
      eq_before += w < wave ? s : 0u;
      eq_total += s;
    }
    const uint32_t eq_rank = eq_base + eq_before + __popcll(m_eq & lt_mask);
    const bool take = gt || (eq && (take_all_eq || eq_rank < n_take_eq));
    const uint64_t m_take = __ballot(take);
    if (lane == 0) sh.wsum2[wave] = __popcll(m_take);
    __syncthreads();
    uint32_t take_before = 0, take_total = 0;
    for (int w = 0; w < SEL_WAVES; ++w) {
      const uint32_t s = sh.wsum2[w];
      take_before += w < wave ? s : 0u;
      take_total += s;
    }
    if (take) emit(out_base + take_before + (uint32_t)__popcll(m_take & lt_mask), i);
    eq_base += eq_total;
    out_base += take_total;
    __syncthreads();
  }
  return out_base;
}

// Selects the k best of a row given by `get` and writes mapped indices in ascending order.
template <class Get, class Emit>
__device__ uint32_t select_row(Get get, int64_t n, uint32_t k, SelShared& sh, Emit emit) {
  const KthResult r = radix_kth(get, n, k, sh);
  if (r.total <= k) return collect_ordered(get, n, 0u, 0u, true, sh, emit);
  return collect_ordered(get, n, r.tau, r.n_take_eq, false, sh, emit);
}

__global__ __launch_bounds__(SEL_THREADS) void topk_kernel(
    const float* __restrict__ scores, int64_t ld, int64_t n_cols,
    const int32_t* __restrict__ n_valid, const float* __restrict__ block_max, int64_t ld_bm,
    int k, const int32_t* __restrict__ pool_blocks, int n_pool, int32_t* __restrict__ out,
    int64_t ld_idx) {
  __shared__ SelShared sh;
  const int t = blockIdx.x;
  const float* row = scores + (int64_t)t * ld;
  int64_t n = n_cols;
  if (n_valid != nullptr) {
    const int64_t v = n_valid[t];
    n = v < 0 ? 0 : (v < n ? v : n);
  }
  int32_t* orow = out + (int64_t)t * ld_idx;
  auto map = [&](int64_t slot) -> int32_t {
    if (pool_blocks == nullptr) return (int32_t)slot;
    const int64_t pb = slot >> 3;
    const int32_t b = pb < n_pool ? pool_blocks[(int64_t)t * n_pool + pb] : -1;
    return b < 0 ? -1 : (int32_t)((int64_t)b * 8 + (slot & 7));
  };
  uint32_t kept = 0;
  bool done = false;

  if (n <= KEYS_CAP) {
    for (int64_t i = threadIdx.x; i < n; i += SEL_THREADS) {
      const float v = row[i];
      sh.keys[i] = selectable(v) ? float_key(v) : 0u;
    }
    __syncthreads();
    auto get = [&](int64_t i, uint32_t& key) { key = sh.keys[i]; return key != 0u; };
    kept = select_row(get, n, (uint32_t)k, sh, [&](uint32_t rank, int64_t i) {
      if (rank < (uint32_t)k) orow[rank] = map(i);
    });
    done = true;
  } else if (block_max != nullptr) {
    // Phase A: threshold on block maxima. The last block may be partial (slots >= n are
    // outside this selection), so its maximum is recomputed from the scores.
    const int64_t nb = (n + 7) >> 3;
    const float* bmrow = block_max + (int64_t)t * ld_bm;
    const int64_t tail = n & 7;
    float tail_max = -__builtin_inff();
    if (tail) {
      for (int64_t s = (nb - 1) * 8; s < n; ++s) tail_max = fmaxf(tail_max, row[s]);
    }
    auto getb = [&](int64_t b, uint32_t& key) {
      const float v = (tail && b == nb - 1) ? tail_max : bmrow[b];
      key = float_key(v);
      return selectable(v);
    };
    const KthResult rb = radix_kth(getb, nb, (uint32_t)k, sh);
    const uint32_t tau_b = rb.total <= (uint32_t)k ? 0u : rb.tau;
    const uint32_t n_cand = collect_ordered(getb, nb, tau_b, 0u, true, sh,
                                            [&](uint32_t rank, int64_t b) {
                                              if (rank < CAND_BLOCKS_CAP) sh.cblocks[rank] = (int32_t)b;
                                            });
    if (n_cand <= CAND_BLOCKS_CAP) {
      // Phase B: exact selection over the candidate blocks' slots, in slot order.
      const int64_t nc = (int64_t)n_cand * 8;
      for (int64_t i = threadIdx.x; i < nc; i += SEL_THREADS) {
        const int64_t slot = (int64_t)sh.cblocks[i >> 3] * 8 + (i & 7);
        const float v = slot < n ? row[slot] : -__builtin_inff();
        sh.keys[i] = selectable(v) ? float_key(v) : 0u;
      }
      __syncthreads();
      auto get = [&](int64_t i, uint32_t& key) { key = sh.keys[i]; return key != 0u; };
      kept = select_row(get, nc, (uint32_t)k, sh, [&](uint32_t rank, int64_t i) {
        if (rank < (uint32_t)k) orow[rank] = map((int64_t)sh.cblocks[i >> 3] * 8 + (i & 7));
      });
      done = true;
    }
  }
  if (!done) {
    auto get = [&](int64_t i, uint32_t& key) {
      const float v = row[i];
      key = float_key(v);
      return selectable(v);
    };
    kept = select_row(get, n, (uint32_t)k, sh, [&](uint32_t rank, int64_t i) {
      if (rank < (uint32_t)k) orow[rank] = map(i);
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
  const float* bmrow = block_max + (int64_t)t * ld_bm;
  int32_t* prow = pool + (int64_t)t * ld_pool;
  auto emit = [&](uint32_t rank, int64_t b) {
    if (rank < (uint32_t)n_keep) prow[rank] = (int32_t)b;
  };
  uint32_t kept;
  if (nb <= KEYS_CAP) {
    for (int64_t b = threadIdx.x; b < nb; b += SEL_THREADS) {
      const float v = b == nb - 1 ? __builtin_inff() : bmrow[b];
      sh.keys[b] = selectable(v) ? float_key(v) : 0u;
    }
    __syncthreads();
    auto get = [&](int64_t i, uint32_t& key) { key = sh.keys[i]; return key != 0u; };
    kept = select_row(get, nb, (uint32_t)n_keep, sh, emit);
  } else {
    auto get = [&](int64_t b, uint32_t& key) {
      const float v = b == nb - 1 ? __builtin_inff() : bmrow[b];
      key = float_key(v);
      return selectable(v);
    };
    kept = select_row(get, nb, (uint32_t)n_keep, sh, emit);
  }
  for (int64_t r = kept + threadIdx.x; r < n_keep; r += SEL_THREADS) prow[r] = -1;
}

hipError_t launch_topk(int n_q, const float* scores, int64_t ld_scores, int64_t n_cols,
                       const int32_t* n_valid, const float* block_max, int64_t ld_bm, int k,
                       const int32_t* pool_blocks, int n_pool, int32_t* topk_idx, int64_t ld_idx,
                       hipStream_t stream) {
  hipLaunchKernelGGL(topk_kernel, dim3(n_q), dim3(SEL_THREADS), 0, stream, scores, ld_scores,
                     n_cols, n_valid, block_max, ld_bm, k, pool_blocks, n_pool, topk_idx, ld_idx);
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
