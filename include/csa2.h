/*
 * csa2.h - C ABI of the CSA2 sparse-attention read path for AMD gfx950 (MI355X).
 *
 * The read path of one CSA2 attention layer, as the pages on DeepSeek-V4.1-Flash
 * describe it, is:
 *   1. the lightning indexer scores the shared compressed cache with a per-layer
 *      indexer query (32 heads x 128) and per-head weights;
 *   2. a Top-512 of those scores is taken;
 *   3. in the decoder's Full layer, the same scores are reduced to 8-position block
 *      maxima and the best 2,048 blocks form the candidate pool that later Reindex
 *      layers are restricted to (the Hierarchical Sparse Indexer);
 *   4. 64-head attention with head dim 512 runs over the selected entries of the
 *      shared FP4 latent together with the 128-entry FP8 sliding window, in one
 *      softmax, with key = value = the latent.
 * Sources, cited by page title and section:
 *   [V41F-ARCH]  "DeepSeek-V4.1-Flash - Architecture" (reading notes), sections
 *                2 (CSA2 modes, layer schedule, main attention settings),
 *                3 (Hierarchical Sparse Indexer) and 4 (KV cache formats).
 *   [V41F-BLOG]  "DeepSeek-v4.1 Flash: Pushing the Limits of KV Cache Compression",
 *                sections 2.3.1-2.3.4 (CSA2, modes, HSI), 2.4.4 (FP4 main KV),
 *                3.1 (cache entries), 3.3.2 (the readout of one layer).
 *
 * Conventions shared by every call
 *   - Every call is stateless and re-entrant and returns an int status (CSA2_OK = 0).
 *   - Tensor arguments are caller-owned DEVICE pointers. The library never allocates,
 *     frees or keeps them past the enqueued work. Calls that take a workspace accept a
 *     caller-owned device workspace of csa2_workspace_bytes(...) bytes; in this version
 *     that is 0 for every op, so NULL/0 may be passed.
 *   - Layouts are dense row-major with the leading dimensions given. bf16 values are
 *     passed as their 16-bit patterns; FP8 E4M3 and FP4 E2M1 as bytes.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Calls only
 *     enqueue work: buffers must stay alive until the stream has been synchronised.
 *   - All argument checks run on the host before any HIP call. On any error status
 *     nothing has been launched and no output has been written; csa2_last_error()
 *     returns a message (thread-local, valid until the next call on that thread).
 *   - Device-resident index arguments (kv_start, n_visible, pool blocks, Top-K
 *     indices, SWA rows) cannot be checked on the host. Kernels check every row they
 *     would touch against the row counts passed in; an entry whose row falls outside
 *     its cache is treated as absent (score -inf, never selected, not attended).
 *   - Inputs are finite by contract (the FP8 codes 0x7F/0xFF, NaN, are not expected).
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Model constants [V41F-ARCH] sections 2-4; the names follow the configuration keys the
 * blog page quotes (index_topk, sliding_window, head_dim, candidate_block_size,
 * candidate_topk_blocks). */
#define CSA2_N_HEADS 64                  /* main query heads */
#define CSA2_HEAD_DIM 512                /* latent width = head dim, key = value */
#define CSA2_IDX_HEADS 32                /* indexer query heads */
#define CSA2_IDX_DIM 128                 /* indexer head dim */
#define CSA2_INDEX_TOPK 512              /* entries selected per query */
#define CSA2_SLIDING_WINDOW 128          /* SWA entries per query */
#define CSA2_CANDIDATE_BLOCK_SIZE 8      /* positions per HSI block */
#define CSA2_CANDIDATE_TOPK_BLOCKS 2048  /* HSI pool blocks (16,384 positions) */
#define CSA2_FP4_ROW_BYTES 256           /* 512 E2M1 codes, two per byte */
#define CSA2_SCALE_ROW_BYTES 32          /* one E4M3 scale per 16 channels */
#define CSA2_KIDX_ROW_BYTES 128          /* 128 E4M3 indexer-K channels */
#define CSA2_SWA_ROW_BYTES 512           /* 512 E4M3 SWA channels */
#define CSA2_MAX_K 2048                  /* largest k / n_keep accepted */

typedef enum { CSA2_FULL = 0, CSA2_REINDEX = 1, CSA2_REUSE = 2 } csa2_mode_t;

enum {
  CSA2_OK = 0,
  CSA2_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad leading dim, alignment */
  CSA2_ERR_UNSUPPORTED = 2, /* a dimension other than the compiled constants */
  CSA2_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  CSA2_ERR_HIP = 4          /* a HIP launch failed (message names it) */
};

/* Workspace sizing. `op` is one of the CSA2_OP_* values; `n_q` queries, `max_cols` the
 * largest row length (scores columns or block count) and `k` the selection size the
 * call will be made with. Returns 0 when the op needs no workspace, which in this version
 * is every op. */
enum { CSA2_OP_INDEX_SCORE = 0, CSA2_OP_BLOCK_POOL = 1, CSA2_OP_TOPK = 2, CSA2_OP_SPARSE_ATTN = 3 };
size_t csa2_workspace_bytes(int op, int n_q, int64_t max_cols, int k);

/* Lightning-indexer score ([V41F-BLOG] 2.3.1 and 3.3.2; [V41F-ARCH] 2 and 3).
 * For query t the score of cache position j is
 *     s[t,j] = sum_{h<32} w[t,h] * ReLU( q_idx[t,h,:] . k_idx[kv_start[t]+j, :] )
 * (the indexer Q, the shared indexer K and a per-head weight; the unprinted scale
 * factor is omitted because selection is invariant to a positive scale).
 *   mode = CSA2_FULL: slot j in [0, ld_scores) holds s[t,j] for j < n_visible[t];
 *       every other slot holds -inf. pool_blocks must be NULL.
 *   mode = CSA2_REINDEX: slot r in [0, n_pool*block_size) holds the score of position
 *       p = pool_blocks[t*n_pool + r/block_size]*block_size + r%block_size, or -inf when
 *       that block id is negative or p >= n_visible[t]; slots >= n_pool*block_size
 *       hold -inf. Requires ld_scores >= n_pool*block_size.
 *   mode = CSA2_REUSE: rejected (CSA2_ERR_INVALID_ARG): a Reuse layer does no scoring.
 * Arguments
 *   n_q                 queries (rows of q_idx, w, scores); 0 is a no-op.
 *   n_heads, d_idx      must be 32 and 128.
 *   q_idx    [n_q,32,128] bf16, 16-byte aligned.        w [n_q,32] f32.
 *   k_cache  [n_entries,128] E4M3, 16-byte aligned rows of 128 bytes.
 *   kv_start [n_q] int64 first cache row of query t's sequence; n_visible [n_q] int32.
 *   pool_blocks [n_q,n_pool] int32 (REINDEX), block ids with -1 padding.
 *   block_size          must be 8.
 *   scores   [n_q,ld_scores] f32 output. May be NULL in FULL mode when block_max is
 *       given: only the block maxima are written (ld_scores still sets the slot range).
 *       A decoder Full layer needs no more: its Top-K lies inside the pool, whose slots
 *       a REINDEX call with the same q_idx and w scores bit-identically.
 *   block_max [n_q,ld_block_max] f32 output, may be NULL: block_max[t,b] is the max of
 *       scores[t, 8b .. 8b+7] over the slots that exist; requires
 *       ld_block_max >= ceil(ld_scores/8). These maxima are what csa2_block_pool ranks,
 *       and csa2_topk uses them to skip blocks that cannot hold a winner.
 *   block_aux [n_q,ld_block_max] uint32 output, may be NULL; FULL mode with block_max only:
 *       the block statistics csa2_full_select reads. Bits 0..2 hold the block's argmax (the
 *       lowest slot whose score equals block_max[t,b]); the bits above hold the selection
 *       key of the largest score among its other slots (the order-preserving image of the
 *       float: sign bit flipped for non-negative values, all bits flipped for negative
 *       ones; 0 when no other slot has a score other than -inf), rounded up to a multiple
 *       of 8, so the stored word, masked to its upper bits, is never below that key.
 * Errors: CSA2_ERR_INVALID_ARG for NULL scores outside that case, or block_aux outside
 *   it. */
int csa2_index_score(csa2_mode_t mode, int n_q, int n_heads, int d_idx,
                     const void* q_idx, const float* w,
                     const void* k_cache, int64_t n_entries,
                     const int64_t* kv_start, const int32_t* n_visible,
                     const int32_t* pool_blocks, int n_pool, int block_size,
                     float* scores, int64_t ld_scores,
                     float* block_max, int64_t ld_block_max, uint32_t* block_aux,
                     void* stream);

/* Lightning-indexer score, FULL mode, for queries that share one sequence (chunked
 * prefill: [V41F-BLOG] 2.3.1 and 3.3.2, with the causal visibility of each query's own
 * position). Identical to csa2_index_score(CSA2_FULL, ...) with kv_start[t] = kv_start for
 * every t: slot j < n_visible[t] of query t scores cache row kv_start + j; other slots
 * hold -inf; block_max as there (nullable). The queries are scored in groups against
 * each cache tile, so every row is read once per group instead of once per query.
 * Arguments as csa2_index_score; kv_start is a host value. n_q <= 2^22.
 * Errors: CSA2_ERR_INVALID_ARG, CSA2_ERR_UNSUPPORTED as csa2_index_score. */
int csa2_index_score_shared(int n_q, int n_heads, int d_idx, const void* q_idx, const float* w,
                            const void* k_cache, int64_t n_entries, int64_t kv_start,
                            const int32_t* n_visible, float* scores, int64_t ld_scores,
                            float* block_max, int64_t ld_block_max, void* stream);

/* Lightning-indexer score over MXFP4 indexer keys ([V41F-BLOG] 2.4.4: the indexer cache
 * is FP4 in the OCP MXFP4 format; 3.1: a 128-dimensional MXFP4 indexer K entry is its
 * E2M1 payload plus one scale byte per 32 channels). Identical to csa2_index_score (same
 * modes, slots, outputs, -inf rules and errors) except for the key rows:
 *   k_codes  [n_entries,64] uint8: channel 2m is the low nibble of byte m, 2m+1 the high
 *            nibble (E2M1: sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0);
 *            16-byte aligned.
 *   k_scales [n_entries,4] uint8 E8M0 (value 2^(e-127)); scale g covers channels
 *            32g .. 32g+31; 4-byte aligned.
 * Key value of channel c = E2M1(code c) * 2^(k_scales[c/32] - 127). Supported scale codes
 * are 1..254 with every product inside bf16's normal range (|x| in [2^-126, 2^127]);
 * 0xFF (NaN) is never passed. block_aux (FULL mode with block_max only, nullable) holds the
 * same block statistics as csa2_index_score's, here of the MXFP4 scores; csa2_full_select_mxfp4
 * reads them. Errors: as csa2_index_score, plus CSA2_ERR_INVALID_ARG for a NULL or
 * misaligned k_scales. */
int csa2_index_score_mxfp4(csa2_mode_t mode, int n_q, int n_heads, int d_idx,
                           const void* q_idx, const float* w,
                           const void* k_codes, const void* k_scales, int64_t n_entries,
                           const int64_t* kv_start, const int32_t* n_visible,
                           const int32_t* pool_blocks, int n_pool, int block_size,
                           float* scores, int64_t ld_scores,
                           float* block_max, int64_t ld_block_max, uint32_t* block_aux,
                           void* stream);

/* MXFP8 indexer query (reading R24: the pages' V4 lineage runs the indexer in low
 * precision; here the query is quantised with the OCP microscaling recipe so that both
 * operands of the indexer product go to gfx950's scaled f8f6f4 MFMA as stored).
 *   csa2_quantize_mxfp8: rows x [n_rows, d] bf16 -> codes [n_rows, d] E4M3 and scales
 *       [n_rows, d/32] E8M0: per 32 channels X = floor(log2 amax) - 8, scale byte X + 127
 *       kept in 1..254 (127 for an all-zero group), code = E4M3(x * 2^-X), nearest even,
 *       saturating at 448. d must be 128; x and codes 16-byte aligned, scales 4-byte.
 *   csa2_index_score_mxfp4_q8: as csa2_index_score_mxfp4 (FULL and REINDEX modes, same
 *       slots, pool mapping, -inf rules, block maxima, nullable FULL scores) with the query
 *       given as q_codes
 *       [n_q, 32, 128] E4M3 and q_scales [n_q, 32, 4] E8M0 (query value of head h, channel
 *       c = E4M3(q_codes[t,h,c]) * 2^(q_scales[t,h,c/32] - 127)). Products are exact; the
 *       accumulation is the matrix core's fp32 (not bit-identical to the bf16 path).
 * Errors: as csa2_index_score_mxfp4. */
int csa2_quantize_mxfp8(int n_rows, int d, const void* x, void* codes, void* scales,
                        void* stream);
/* csa2_index_score_shared_q8: csa2_index_score_shared (queries sharing one sequence, FULL
 * mode, kv_start a host value, n_q <= 2^22) with the MXFP8 query over E4M3 keys; scores
 * identical to csa2_index_score_q8's. */
int csa2_index_score_shared_q8(int n_q, int n_heads, int d_idx, const void* q_codes,
                               const void* q_scales, const float* w, const void* k_cache,
                               int64_t n_entries, int64_t kv_start, const int32_t* n_visible,
                               float* scores, int64_t ld_scores, float* block_max,
                               int64_t ld_block_max, void* stream);
/* csa2_index_score_q8: the same with E4M3 keys (k_cache [n_entries, 128], as
 * csa2_index_score reads them) instead of MXFP4 ones: the matrix core's fp8 B operand with
 * unit key scales. Arguments, modes and errors as csa2_index_score. */
int csa2_index_score_q8(csa2_mode_t mode, int n_q, int n_heads, int d_idx, const void* q_codes,
                        const void* q_scales, const float* w, const void* k_cache,
                        int64_t n_entries, const int64_t* kv_start, const int32_t* n_visible,
                        const int32_t* pool_blocks, int n_pool, int block_size, float* scores,
                        int64_t ld_scores, float* block_max, int64_t ld_block_max, void* stream);
int csa2_index_score_mxfp4_q8(csa2_mode_t mode, int n_q, int n_heads, int d_idx,
                              const void* q_codes, const void* q_scales, const float* w,
                              const void* k_codes, const void* k_scales, int64_t n_entries,
                              const int64_t* kv_start, const int32_t* n_visible,
                              const int32_t* pool_blocks, int n_pool, int block_size,
                              float* scores, int64_t ld_scores, float* block_max,
                              int64_t ld_block_max, void* stream);

/* The compressor: main-KV entries from the per-token projections of the hidden state
 * ([V41F-ARCH] 1: the KV content C = H W_KV and the compression weights Z = H W_Z;
 * [V41F-BLOG] 3.3.2: gated pooling that is a per-token projection at m = 1; 2.3.1: no
 * overlap between adjacent entries and no absolute position embedding). Reading R22:
 * entry j, channel c = sum over the tokens i = jm .. jm+m-1 of softmax_i(z[i, c]) *
 * c[i, c], evaluated in float32 (exp, one division per channel) and stored as bf16 (nearest
 * even); n_tokens / m entries (rounded down: an incomplete group gives no entry). At
 * m = 1 the entry is c itself.
 *   m in 1..8 (the pages use 1 in the decoder and 2 in the encoder); d must be 512.
 *   c, z [n_tokens, ld_in] bf16, 16-byte aligned; out [n_tokens / m, ld_out] bf16.
 *   ld_in, ld_out >= 512, multiples of 8.
 * The entries are what csa2_write_latent quantises (after RoPE, which is applied by the
 * caller) and what csa2_project_index_key projects.
 * Errors: CSA2_ERR_INVALID_ARG (null pointer, bad size or alignment), CSA2_ERR_UNSUPPORTED
 * (m or d). */
int csa2_compress_kv(int m, int n_tokens, int d, const void* c, const void* z, int64_t ld_in,
                     void* out, int64_t ld_out, void* stream);

/* Indexer keys as a projection of main-KV entries ([V41F-BLOG] 2.3.1: CSA2 projects the
 * main KV entries to get the indexer K). Reading R23: out[r, o] = sum_c entries[r, c] *
 * w_ik[o, c], fp32 accumulation, bf16 output (nearest even).
 *   d_in must be 512 and d_out 128. entries [n, ld_entries] bf16 (ld_entries >= 512, a
 *   multiple of 8), 16-byte aligned; w_ik [128, 512] bf16 (output channel major),
 *   16-byte aligned; out [n, ld_out] bf16, ld_out >= 128.
 * The keys are what csa2_write_e4m3 (d = 128) or csa2_write_mxfp4_key store.
 * Errors: CSA2_ERR_INVALID_ARG, CSA2_ERR_UNSUPPORTED (d_in, d_out). */
int csa2_project_index_key(int n, int d_in, int d_out, const void* entries, int64_t ld_entries,
                           const void* w_ik, void* out, int64_t ld_out, void* stream);

/* Block-mean indexer keys for a HISA-style two-stage filter (the alternative
 * [V41F-BLOG] 2.3.4 sets beside HSI: the prefix is cut into blocks of consecutive
 * positions, each block keeps the mean of its indexer keys, a first stage scores those
 * means with the same query and weights, the best blocks are expanded to their positions
 * and a second stage scores them with the original keys). Block size 8 and bf16 storage
 * are readings (R20); the pages fix neither.
 * For query t with n = n_visible[t] (clipped below at 0), nb = ceil(n/8) and
 * n_blocks[t] = nb. For b < min(nb, max_blocks), km[km_start[t] + b, c] = bf16 (nearest
 * even) of the float32 quotient (sum over the visible positions p in 8b .. 8b+7 whose
 * row kv_start[t] + p lies in [0, n_entries) of E4M3 value k_cache[row, c]) / (count of
 * such positions); 0 when there are none. The sums are exact in float32.
 *   d_idx must be 128, block_size 8. k_cache [n_entries,128] E4M3, 8-byte aligned;
 *   kv_start [n_q] int64; n_visible [n_q] int32; km [n_km_rows,128] bf16 output,
 *   16-byte aligned; km_start [n_q] int64 first km row of query t (a destination row
 *   outside [0, n_km_rows) is skipped); 1 <= max_blocks <= 2^28 bounds the blocks
 *   written per query; n_blocks [n_q] int32 output. Queries that share a sequence may
 *   share km rows (the same values are written).
 *   last_only nonzero: only block nb - 1 (the one holding position n - 1) is recomputed,
 *   for the decoder's append of one token per query (the pages: a new token changes one
 *   block and completed blocks keep their summary); other km rows are left as they are.
 * The block means are what csa2_index_score_bf16 (FULL mode, n_visible = n_blocks,
 * kv_start = km_start) scores; those block scores, passed to csa2_block_pool as its
 * block_max with the position count n_visible, give the HISA pool.
 * Errors: CSA2_ERR_INVALID_ARG (null pointer, bad size or alignment),
 * CSA2_ERR_UNSUPPORTED (d_idx or block_size). */
int csa2_block_mean_keys(int n_q, int d_idx, int block_size, const void* k_cache,
                         int64_t n_entries, const int64_t* kv_start, const int32_t* n_visible,
                         void* km, const int64_t* km_start, int64_t n_km_rows,
                         int64_t max_blocks, int32_t* n_blocks, int last_only, void* stream);

/* Lightning-indexer score over bf16 key rows (the block-mean keys above). Identical to
 * csa2_index_score (same modes, slots, outputs, -inf rules and errors) except that
 * k_rows is [n_entries,128] bf16, 16-byte aligned, and the key values are those bf16
 * values. */
int csa2_index_score_bf16(csa2_mode_t mode, int n_q, int n_heads, int d_idx,
                          const void* q_idx, const float* w,
                          const void* k_rows, int64_t n_entries,
                          const int64_t* kv_start, const int32_t* n_visible,
                          const int32_t* pool_blocks, int n_pool, int block_size,
                          float* scores, int64_t ld_scores,
                          float* block_max, int64_t ld_block_max,
                          void* stream);

/* Cache writes ([V41F-BLOG] 2.4.4: the main KV is stored as E2M1 with one E4M3 scale per
 * 16 channels and no global scale, quantised after RoPE; the sliding-window cache keeps
 * FP8; the indexer cache is OCP MXFP4; [V41F-ARCH] 4). These produce the formats the
 * calls above read. Inputs are bf16 rows, already rotated; row r goes to cache row
 * rows[r]; a destination outside [0, n_entries) (or [0, n_rows)) is skipped, so the
 * caller may pass -1 for a row to drop. Rounding (the pages give none; readings R16 and
 * R19): nearest grid value, ties to the even code, saturating at the grid's largest
 * value, decided on float32 values:
 *   csa2_write_latent: per 16-channel group scale = E4M3(amax / 6) (float32 division)
 *       and code = E2M1 rounding of the exact quotient x / scale; zero codes when the
 *       scale is 0. Writes
 *       kv_fp4[row, 0..256) (channel 2m in the low nibble of byte m) and
 *       kv_scale[row, 0..32). x [n,512] bf16, 16-byte aligned; rows [n] int64;
 *       kv_fp4_stride >= 256 (multiple of 4), kv_scale_stride >= 32.
 *   csa2_write_e4m3: dst[row, 0..d) = E4M3(x[r, :]) (saturating at +-448; a negative
 *       value rounding to zero keeps its sign bit), d = 512 for window rows or 128 for
 *       E4M3 indexer keys; dst_stride >= d, a multiple of 8.
 *   csa2_write_mxfp4_key: per 32-channel group X = floor(log2 amax) - 2, scale byte
 *       X + 127 kept in 1..254 (127 for an all-zero group), codes E2M1(x * 2^-X); writes
 *       k_codes[row, 0..64) and k_scales[row, 0..4). x [n,128] bf16.
 * Calls only enqueue work; overlapping destination rows in one call race.
 * Errors: CSA2_ERR_INVALID_ARG (null pointer, n < 0, bad stride or alignment),
 * CSA2_ERR_UNSUPPORTED (csa2_write_e4m3 with d other than 128 or 512). */
int csa2_write_latent(int n, const void* x, const int64_t* rows, void* kv_fp4,
                      int64_t kv_fp4_stride, void* kv_scale, int64_t kv_scale_stride,
                      int64_t n_entries, void* stream);
int csa2_write_e4m3(int n, int d, const void* x, const int64_t* rows, void* dst,
                    int64_t dst_stride, int64_t n_rows, void* stream);
int csa2_write_mxfp4_key(int n, const void* x, const int64_t* rows, void* k_codes,
                         void* k_scales, int64_t n_entries, void* stream);

/* HSI candidate pool ([V41F-BLOG] 2.3.4 "How does the Full Mode layer build the
 * candidate pool"; [V41F-ARCH] 3). For query t with n = n_visible[t] > 0 there are
 * nb = ceil(n/8) visible blocks whose scores are block_max[t, 0..nb) (the last block's
 * missing tail counts as -inf). The block holding position n-1 is forced to +inf so it
 * always takes one of the kept slots; the min(n_keep, nb) blocks with the largest
 * values are kept, ties broken towards the lower block id; blocks whose value is -inf
 * are never kept. pool_blocks[t, 0..n_keep) receives the kept ids in ascending order,
 * then -1. n = 0 gives an all -1 row.
 *   block_max [n_q,ld_bm] f32 (as written by csa2_index_score FULL), 16-byte aligned,
 *   ld_bm a multiple of 4; n_visible [n_q] (clipped to 8*ld_bm).
 *   block_size must be 8; 1 <= n_keep <= CSA2_MAX_K; ld_pool >= n_keep.
 *   Positions of the pool are {8b .. 8b+7} of every kept block b, clipped to n. */
int csa2_block_pool(int n_q, const float* block_max, int64_t ld_bm,
                    const int32_t* n_visible, int block_size, int n_keep,
                    int32_t* pool_blocks, int64_t ld_pool,
                    void* workspace, size_t ws_bytes, void* stream);

/* How csa2_topk uses a pool of candidate blocks. */
typedef enum {
  CSA2_POOL_NONE = 0,        /* no pool: scores are indexed by cache position */
  CSA2_POOL_SLOTS = 1,       /* scores are indexed by pool slot (a Reindex layer's scores) */
  CSA2_POOL_CANDIDATES = 2   /* scores are indexed by cache position, and only positions in
                                the pool's blocks compete (a Full layer after its pool) */
} csa2_pool_use_t;

/* Top-K selection ([V41F-BLOG] 2.3.4 and 3.3.1; [V41F-ARCH] 2 "Top-K global entries").
 * For query t the candidates are slots r < n_cols (and r < n_valid[t] when n_valid is
 * not NULL) whose score is finite or +inf (-inf and NaN are never selected); with
 * CSA2_POOL_CANDIDATES only slots r with r/block_size among pool_blocks[t, ..] compete.
 * The min(k, #candidates) slots with the largest scores are chosen, ties broken towards
 * the lower slot. Each chosen slot is mapped to a cache position: identity, or with
 * CSA2_POOL_SLOTS pool_blocks[t*n_pool + r/block_size]*block_size + r%block_size.
 * topk_idx[t, 0..k) receives the positions in ascending order of slot, then -1.
 * CSA2_POOL_CANDIDATES with the pool csa2_block_pool wrote from these scores' block
 * maxima (n_keep > k) gives exactly the unrestricted Top-K: a block outside the pool
 * has n_keep - 1 blocks ranked above it, each holding an entry that outranks all of its
 * entries, so none of them can be among the k best; the kernel then examines only the
 * pool's slots. The pool must be ascending with -1 padding (as csa2_block_pool writes).
 *   scores [n_q,ld_scores] f32, 16-byte aligned, ld_scores a multiple of 4;
 *       n_cols <= ld_scores.
 *   block_max [n_q,ld_block_max] f32, may be NULL: when given it must hold the maxima
 *       of 8-slot blocks of these scores (as csa2_index_score writes them), 16-byte
 *       aligned with ld_block_max a multiple of 4; it lets the kernel examine only blocks
 *       that can hold a winner. The result is identical.
 *   1 <= k <= CSA2_MAX_K; ld_idx >= k; block_size must be 8. */
int csa2_topk(int n_q, const float* scores, int64_t ld_scores, int64_t n_cols,
              const int32_t* n_valid,
              const float* block_max, int64_t ld_block_max,
              int k, csa2_pool_use_t pool_use, const int32_t* pool_blocks, int n_pool,
              int block_size, int32_t* topk_idx, int64_t ld_idx,
              void* workspace, size_t ws_bytes, void* stream);

/* The Full layer's pool and its Top-K in one call ([V41F-BLOG] 2.3.4; [V41F-ARCH] 3):
 * the same results as csa2_block_pool(n_q, block_max, ld_bm, n_visible, block_size,
 * n_keep, pool_blocks, ld_pool, ...) followed by csa2_topk(n_q, scores, ld_scores, n_cols,
 * n_visible, NULL, 0, k, CSA2_POOL_CANDIDATES, pool_blocks, n_keep, block_size, topk_idx,
 * ld_idx, ...), in one kernel that keeps the pool in on-chip memory between the two
 * selections. Both outputs are written. Arguments and limits are those of the two calls
 * (block_max and scores as csa2_index_score FULL writes them). */
int csa2_pool_topk(int n_q, const float* block_max, int64_t ld_bm,
                   const int32_t* n_visible, int block_size, int n_keep,
                   int32_t* pool_blocks, int64_t ld_pool,
                   const float* scores, int64_t ld_scores, int64_t n_cols, int k,
                   int32_t* topk_idx, int64_t ld_idx, void* stream);

/* The HSI pool and the Full layer's candidate blocks in one call ([V41F-BLOG] 2.3.2 and
 * 2.3.4, "How does the Full Mode layer build the candidate pool"; [V41F-ARCH] 3).
 * pool_blocks receives exactly what csa2_block_pool writes for the same arguments.
 * cand_blocks receives a subset of the pool, ascending and -1 padded to n_keep, that holds
 * every block containing one of the k best entries of the scores whose 8-slot maxima
 * block_max holds: a block holding such an entry has fewer than k blocks ranked above it
 * by (maximum desc, id asc), each holding a better entry of its own, so it is among the k
 * best blocks; the candidates are the pool blocks whose maximum reaches a threshold that
 * the (k+1)-th best block (the forced latest block counted first) reaches. Rescoring the
 * candidates' slots (csa2_index_score REINDEX with cand_blocks as the pool) and taking the
 * Top-K among them (csa2_topk, CSA2_POOL_SLOTS) therefore gives exactly the Full layer's
 * Top-K over its whole score row, from a quarter of the pool's rows. The threshold comes
 * from the pool selection's first histogram pass; when that pass cannot give one, every
 * pool block is a candidate (the result is the same, only slower).
 *   block_max, ld_bm, n_visible, block_size, n_keep, pool_blocks, ld_pool: as
 *       csa2_block_pool; 1 <= k < n_keep; cand_blocks [n_q,ld_cand] int32, ld_cand >= n_keep.
 * Caller-owned device buffers, no scratch; errors as csa2_block_pool. */
int csa2_pool_candidates(int n_q, const float* block_max, int64_t ld_bm,
                         const int32_t* n_visible, int block_size, int n_keep,
                         int32_t* pool_blocks, int64_t ld_pool, int k, int32_t* cand_blocks,
                         int64_t ld_cand, void* stream);

/* The decoder Full layer's whole selection in one call, for E4M3 indexer keys and a bf16
 * indexer query ([V41F-BLOG] 2.3.1, 2.3.2 and 2.3.4; [V41F-ARCH] 2 and 3): the HSI pool
 * (exactly what csa2_block_pool writes into pool_blocks) and the Full layer's Top-K
 * (exactly what csa2_topk returns over the whole score row of csa2_index_score (FULL) for
 * the same query: the k best visible positions, ties to the lower position, ascending, -1
 * padded), from the Full pass's block maxima and block statistics. The Top-K lies in the
 * pool's candidate blocks (as csa2_pool_candidates defines them, with threshold t2); in
 * each, a winner is the argmax (score = the block maximum) or another slot scoring at most
 * the block's second score, while the k-th best score reaches t2; so only the candidate
 * blocks whose second key reaches t2 are rescored (with q_idx and w against k_cache,
 * repeating the Full pass's arithmetic step for step) and every other candidate enters
 * with its argmax alone. It replaces csa2_pool_candidates + csa2_index_score (REINDEX over
 * the candidates) + csa2_topk.
 *   block_max, ld_bm, n_visible, block_size, n_keep, pool_blocks, ld_pool: as
 *       csa2_block_pool; block_max and block_aux [n_q, ld_bm] (uint32) are those written
 *       by one csa2_index_score (FULL) pass of this q_idx and w;
 *   n_heads, d_idx, q_idx, w, k_cache, n_entries, kv_start: as csa2_index_score (E4M3 keys);
 *   1 <= k < n_keep; topk_idx [n_q, ld_idx] int32, ld_idx >= k.
 * Caller-owned device buffers, no scratch; errors as csa2_block_pool and csa2_index_score. */
int csa2_full_select(int n_q, const float* block_max, int64_t ld_bm, const int32_t* n_visible,
                     int block_size, int n_keep, int32_t* pool_blocks, int64_t ld_pool,
                     int n_heads, int d_idx, const void* q_idx, const float* w,
                     const void* k_cache, int64_t n_entries, const int64_t* kv_start,
                     const uint32_t* block_aux, int k, int32_t* topk_idx, int64_t ld_idx,
                     void* stream);

/* csa2_full_select for MXFP4 indexer keys ([V41F-BLOG] 2.4.4 and 3.1): the same pool and
 * Top-K, from the block maxima and block statistics of one csa2_index_score_mxfp4 (FULL)
 * pass of this q_idx and w, with the rescored candidate slots computed from k_codes and
 * k_scales exactly as that pass computes them. k_codes, k_scales as csa2_index_score_mxfp4;
 * other arguments and errors as csa2_full_select, plus CSA2_ERR_INVALID_ARG for a NULL or
 * misaligned k_scales. It replaces csa2_pool_candidates + csa2_index_score_mxfp4 (REINDEX
 * over the candidates) + csa2_topk. */
int csa2_full_select_mxfp4(int n_q, const float* block_max, int64_t ld_bm,
                           const int32_t* n_visible, int block_size, int n_keep,
                           int32_t* pool_blocks, int64_t ld_pool, int n_heads, int d_idx,
                           const void* q_idx, const float* w, const void* k_codes,
                           const void* k_scales, int64_t n_entries, const int64_t* kv_start,
                           const uint32_t* block_aux, int k, int32_t* topk_idx, int64_t ld_idx,
                           void* stream);

/* Joint sparse attention over the selected entries and the sliding window
 * ([V41F-BLOG] 2.2.2, 3.3.1 and 3.3.2 "the readout"; [V41F-ARCH] 2 and 4).
 * For query t let S be {valid positions in topk_idx[t, 0..k)} plus the SWA rows
 * swa_start[t] .. swa_start[t]+n_swa[t]-1. Each entry c_j is a 512-vector used both
 * as key and as value:
 *   main entry at position p, row R = kv_start[t]+p:
 *       c[i] = E2M1(code i of kv_fp4 row R) * E4M3(kv_scale[R, i/16]); code 2m sits in
 *       the low nibble of byte m, code 2m+1 in the high nibble;
 *   SWA row:  c[i] = E4M3(window_kv[row, i]).
 * For head h: l_j = softmax_scale * q[t,h,:] . c_j,  p = softmax over S (one softmax
 * for main and window entries), out[t,h,:] = sum_j p_j c_j (bf16, round to nearest
 * even), lse[t,h] = log sum_j exp(l_j) (f32). An empty S gives out = 0, lse = -inf.
 * Entries of topk_idx that are negative or whose row is outside [0, n_entries) are
 * skipped, as are SWA rows outside [0, n_window_rows). Duplicated positions are
 * attended as many times as they occur. Reuse layers call this with the indices
 * published by the latest Full or Reindex layer.
 *   n_heads, head_dim must be 64 and 512.
 *   q [n_q,64,512] bf16 (16-byte aligned);
 *   kv_fp4 rows of 256 bytes at kv_fp4_stride bytes (>= 256, multiple of 16);
 *   kv_scale rows of 32 bytes at kv_scale_stride bytes (>= 32, multiple of 16);
 *   topk_idx [n_q,ld_idx] int32 with 0 <= k <= CSA2_MAX_K;
 *   window_kv [n_window_rows,512] E4M3; swa_start [n_q] int64; n_swa [n_q] int32 (values
 *   above 128 are clamped to 128);
 *   out [n_q,64,512] bf16; lse [n_q,64] f32 or NULL.
 * Workspace: none (csa2_workspace_bytes returns 0; the arguments are ignored). Each
 * (query, 16-head group) is computed by two workgroups, one per 256-channel half of the
 * output, which repeat the same logits and softmax, so nothing is combined across
 * workgroups and results do not depend on timing.
 * Limits: kv_fp4_stride and kv_scale_stride at most 16,368 bytes. */
int csa2_sparse_attn(int n_q, int n_heads, int head_dim, const void* q,
                     const void* kv_fp4, int64_t kv_fp4_stride,
                     const void* kv_scale, int64_t kv_scale_stride, int64_t n_entries,
                     const int64_t* kv_start, const int32_t* topk_idx, int64_t ld_idx, int k,
                     const void* window_kv, int64_t n_window_rows,
                     const int64_t* swa_start, const int32_t* n_swa,
                     float softmax_scale, void* out, float* lse,
                     void* workspace, size_t ws_bytes, void* stream);

/* Library version string (static storage). */
const char* csa2_version(void);

/* Message of the last failed call on this thread ("" when none). */
const char* csa2_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
