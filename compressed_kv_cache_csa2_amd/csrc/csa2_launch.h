// Host-side launchers of the CSA2 kernels. Arguments are assumed validated by the C ABI
// layer; each launcher only enqueues work on `stream` and reports the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

// k_scales: NULL for E4M3 indexer keys ([E,128]); the E8M0 scale rows ([E,4]) for MXFP4
// keys, whose codes ([E,64]) are then k_cache.
// key_format: 0 E4M3, 1 MXFP4 (k_scales non-NULL), 2 bf16 rows of 256 bytes.
hipError_t launch_index_score(bool reindex, int key_format, int n_q, const uint16_t* q_idx,
                              const float* w, const uint8_t* k_cache, const uint8_t* k_scales,
                              int64_t n_entries, const int64_t* kv_start,
                              const int32_t* n_visible, const int32_t* pool_blocks, int n_pool,
                              float* scores, int64_t ld, float* block_max, int64_t ld_bm,
                              uint32_t* block_aux, hipStream_t stream);

// Block-mean keys (bf16 [rows, 128]) of every visible 8-position block, and the block counts.
hipError_t launch_block_mean_keys(int n_q, const uint8_t* k_cache, int64_t n_entries,
                                  const int64_t* kv_start, const int32_t* n_visible, uint16_t* km,
                                  const int64_t* km_start, int64_t n_km_rows, int64_t max_blocks,
                                  int32_t* n_blocks, bool last_only, hipStream_t stream);

// Full-mode scores of queries that all read the cache rows from one kv_start.
hipError_t launch_index_score_shared(int n_q, const uint16_t* q_idx, const float* w,
                                     const uint8_t* k_cache, int64_t n_entries, int64_t kv_start,
                                     const int32_t* n_visible, float* scores, int64_t ld,
                                     float* block_max, int64_t ld_bm, hipStream_t stream);

hipError_t launch_block_pool(int n_q, const float* block_max, int64_t ld_bm,
                             const int32_t* n_visible, int n_keep, int32_t* pool_blocks,
                             int64_t ld_pool, hipStream_t stream);

// pool_use: 0 none, 1 scores indexed by pool slot, 2 pool blocks are the candidates.
hipError_t launch_topk(int n_q, const float* scores, int64_t ld_scores, int64_t n_cols,
                       const int32_t* n_valid, const float* block_max, int64_t ld_bm, int k,
                       int pool_use, const int32_t* pool_blocks, int n_pool, int32_t* topk_idx,
                       int64_t ld_idx, hipStream_t stream);

// block_pool then topk with the pool's blocks as candidates, in one kernel.
hipError_t launch_pool_topk(int n_q, const float* block_max, int64_t ld_bm,
                            const int32_t* n_visible, int n_keep, int32_t* pool_blocks,
                            int64_t ld_pool, const float* scores, int64_t ld_scores,
                            int64_t n_cols, int k, int32_t* topk_idx, int64_t ld_idx,
                            hipStream_t stream);

// The HSI pool plus the Full layer's candidate blocks (a subset of the pool holding every
// block with one of the k best entries), both ascending and -1 padded to n_keep.
hipError_t launch_block_pool_cand(int n_q, const float* block_max, int64_t ld_bm,
                                  const int32_t* n_visible, int n_keep, int32_t* pool_blocks,
                                  int64_t ld_pool, int k, int32_t* cand_blocks, int64_t ld_cand,
                                  hipStream_t stream);

// The decoder Full layer's selection in one kernel: the pool (as launch_block_pool_cand) and
// the Top-K among its candidates, from the Full pass's block statistics (block_aux) and the
// rescoring, with the layer's indexer query, of the few candidate blocks whose second score
// can reach it. k_scales: NULL for E4M3 keys ([E,128] in k_cache); the E8M0 scale rows
// ([E,4]) for MXFP4 keys, whose codes ([E,64]) are then k_cache.
hipError_t launch_full_select(int n_q, const float* block_max, int64_t ld_bm,
                              const int32_t* n_visible, int n_keep, int32_t* pool_blocks,
                              int64_t ld_pool, const uint16_t* q_idx, const float* w,
                              const uint8_t* k_cache, const uint8_t* k_scales, int64_t n_entries,
                              const int64_t* kv_start, const uint32_t* block_aux, int k,
                              int32_t* topk_idx, int64_t ld_idx, hipStream_t stream);

hipError_t launch_sparse_attn(int n_q, const uint16_t* q, const uint8_t* kv_fp4,
                              int64_t fp4_stride, const uint8_t* kv_scale, int64_t scale_stride,
                              int64_t n_entries, const int64_t* kv_start, const int32_t* topk_idx,
                              int64_t ld_idx, int k, const uint8_t* window_kv,
                              int64_t n_window_rows, const int64_t* swa_start,
                              const int32_t* n_swa, float softmax_scale, uint16_t* out,
                              float* lse, hipStream_t stream);

// Cache writes: quantise bf16 rows into the cache formats (destination rows outside
// [0, n_rows) are skipped).
// Full or Reindex scores of an MXFP8 indexer query over MXFP4 keys (scaled f8f6f4 MFMA).
// fp4k: MXFP4 keys (codes + scales), else E4M3 rows of 128 bytes (k_scales unused).
hipError_t launch_index_score_q8(bool reindex, bool fp4k, int n_q, const uint8_t* q_codes,
                                 const uint8_t* q_scales, const float* w, const uint8_t* k_codes,
                                 const uint8_t* k_scales, int64_t n_entries,
                                 const int64_t* kv_start, const int32_t* n_visible,
                                 const int32_t* pool_blocks, int n_pool, float* scores,
                                 int64_t ld, float* block_max, int64_t ld_bm,
                                 hipStream_t stream);
// Full-mode MXFP8-query scores over E4M3 keys for queries sharing one sequence.
hipError_t launch_index_score_shared_q8(int n_q, const uint8_t* q_codes, const uint8_t* q_scales,
                                        const float* w, const uint8_t* k_cache,
                                        int64_t n_entries, int64_t kv_start,
                                        const int32_t* n_visible, float* scores, int64_t ld,
                                        float* block_max, int64_t ld_bm, hipStream_t stream);
// MXFP8 quantisation of bf16 rows of 128 channels.
hipError_t launch_mxfp8_quantize(int n_rows, const uint16_t* x, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream);
// Gated-pooling compressor: n_out entries of 512 channels from m tokens each (bf16 in/out).
hipError_t launch_compress(int m, int n_out, const uint16_t* c, const uint16_t* z, int64_t ld_in,
                           uint16_t* out, int64_t ld_out, hipStream_t stream);
// Indexer keys [n, 128] = entries [n, 512] . W^T, W bf16 [128, 512].
hipError_t launch_project_index_key(int n, const uint16_t* e, int64_t ld_e, const uint16_t* wk,
                                    uint16_t* out, int64_t ld_out, hipStream_t stream);
hipError_t launch_latent_write(int n, const uint16_t* x, const int64_t* rows, uint8_t* kv_fp4,
                               int64_t fp4_stride, uint8_t* kv_scale, int64_t sc_stride,
                               int64_t n_entries, hipStream_t stream);
hipError_t launch_e4m3_write(int n, int d, const uint16_t* x, const int64_t* rows,
                             uint8_t* dst, int64_t dst_stride, int64_t n_rows, hipStream_t stream);
hipError_t launch_mxfp4_key_write(int n, const uint16_t* x, const int64_t* rows, uint8_t* k_codes,
                                  uint8_t* k_scales, int64_t n_entries, hipStream_t stream);

}  // namespace csa2
