// C ABI of the CSA2 read path (declared in include/csa2.h): host-side argument checks,
// then kernel launches on the caller's stream. Every check runs before any HIP call, so
// a rejected call launches nothing and writes nothing.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "csa2.h"
#include "csa2_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return CSA2_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CSA2_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

#define REQUIRE(cond, code, ...)      \
  do {                                \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

}  // namespace

extern "C" {

const char* csa2_version(void) { return "csa2-gfx950 0.1.0"; }

const char* csa2_last_error(void) { return g_err; }

size_t csa2_workspace_bytes(int op, int n_q, int64_t max_cols, int k) {
  // No call of this library needs scratch memory: the selections keep their state in LDS
  // and the attention's workgroups write disjoint output channels.
  (void)op;
  (void)n_q;
  (void)max_cols;
  (void)k;
  return 0;
}

// Every indexer-key format: key_format 0 (E4M3 rows, k_scales NULL), 1 (MXFP4 codes in
// k_cache, E8M0 scale rows in k_scales) or 2 (bf16 rows, k_scales NULL). `fn` names the
// entry point in messages.
static int index_score_common(const char* fn, int key_format, csa2_mode_t mode, int n_q,
                              int n_heads, int d_idx,
                              const void* q_idx, const float* w, const void* k_cache,
                              const void* k_scales, int64_t n_entries, const int64_t* kv_start,
                              const int32_t* n_visible, const int32_t* pool_blocks, int n_pool,
                              int block_size, float* scores, int64_t ld_scores, float* block_max,
                              int64_t ld_block_max, uint32_t* block_aux, void* stream) {
  REQUIRE(mode == CSA2_FULL || mode == CSA2_REINDEX, CSA2_ERR_INVALID_ARG,
          "%s: mode %d does no scoring (Reuse layers attend with published indices)", fn,
          (int)mode);
  REQUIRE(n_heads == CSA2_IDX_HEADS && d_idx == CSA2_IDX_DIM, CSA2_ERR_UNSUPPORTED,
          "%s: indexer shape %dx%d, only %dx%d is built", fn, n_heads, d_idx,
          CSA2_IDX_HEADS, CSA2_IDX_DIM);
  REQUIRE(block_size == CSA2_CANDIDATE_BLOCK_SIZE, CSA2_ERR_UNSUPPORTED,
          "%s: block_size %d, only %d is built", fn, block_size, CSA2_CANDIDATE_BLOCK_SIZE);
  REQUIRE(n_q >= 0 && n_q <= 65535, CSA2_ERR_INVALID_ARG, "%s: n_q %d out of range", fn, n_q);
  if (n_q == 0) return ok();
  REQUIRE(q_idx && w && k_cache && kv_start && n_visible, CSA2_ERR_INVALID_ARG,
          "%s: null pointer argument", fn);
  REQUIRE(scores != nullptr || (mode == CSA2_FULL && block_max != nullptr), CSA2_ERR_INVALID_ARG,
          "%s: scores may be NULL only in FULL mode with block_max", fn);
  REQUIRE(n_entries >= 0, CSA2_ERR_INVALID_ARG, "%s: n_entries < 0", fn);
  REQUIRE(ld_scores >= 1 && ld_scores <= ((int64_t)1 << 31), CSA2_ERR_INVALID_ARG,
          "%s: ld_scores %lld out of range", fn, (long long)ld_scores);
  REQUIRE(k_scales == nullptr || aligned(k_scales, 4), CSA2_ERR_INVALID_ARG,
          "%s: k_scales must be 4-byte aligned", fn);
  REQUIRE(aligned(q_idx, 16) && aligned(k_cache, 16), CSA2_ERR_INVALID_ARG,
          "%s: q_idx and k_cache must be 16-byte aligned", fn);
  REQUIRE(aligned(w, 4) && aligned(scores, 4) && aligned(kv_start, 8) && aligned(n_visible, 4),
          CSA2_ERR_INVALID_ARG, "%s: misaligned argument", fn);
  if (mode == CSA2_REINDEX) {
    REQUIRE(pool_blocks != nullptr, CSA2_ERR_INVALID_ARG, "%s: REINDEX needs pool_blocks", fn);
    REQUIRE(n_pool >= 1 && n_pool <= CSA2_MAX_K, CSA2_ERR_INVALID_ARG,
            "%s: n_pool %d out of range", fn, n_pool);
    REQUIRE(ld_scores >= (int64_t)n_pool * block_size, CSA2_ERR_INVALID_ARG,
            "%s: ld_scores %lld < n_pool*block_size", fn, (long long)ld_scores);
  } else {
    REQUIRE(pool_blocks == nullptr, CSA2_ERR_INVALID_ARG, "%s: FULL takes no pool_blocks", fn);
  }
  if (block_max != nullptr) {
    REQUIRE(ld_block_max >= (ld_scores + 7) / 8, CSA2_ERR_INVALID_ARG,
            "%s: ld_block_max %lld < ceil(ld_scores/8)", fn, (long long)ld_block_max);
    REQUIRE(aligned(block_max, 4), CSA2_ERR_INVALID_ARG, "%s: misaligned block_max", fn);
  }
  if (block_aux != nullptr) {
    REQUIRE(key_format != 2 && mode == CSA2_FULL && block_max != nullptr, CSA2_ERR_INVALID_ARG,
            "%s: block_aux is written by a FULL pass over E4M3 or MXFP4 keys beside block_max",
            fn);
    REQUIRE(aligned(block_aux, 4), CSA2_ERR_INVALID_ARG, "%s: misaligned block_aux", fn);
  }
  return hip_status(csa2::launch_index_score(
                        mode == CSA2_REINDEX, key_format, n_q,
                        static_cast<const uint16_t*>(q_idx), w,
                        static_cast<const uint8_t*>(k_cache),
                        static_cast<const uint8_t*>(k_scales), n_entries, kv_start, n_visible,
                        pool_blocks, mode == CSA2_REINDEX ? n_pool : 0, scores, ld_scores, block_max,
                        ld_block_max, block_aux, static_cast<hipStream_t>(stream)),
                    fn);
}

int csa2_index_score(csa2_mode_t mode, int n_q, int n_heads, int d_idx, const void* q_idx,
                     const float* w, const void* k_cache, int64_t n_entries,
                     const int64_t* kv_start, const int32_t* n_visible, const int32_t* pool_blocks,
                     int n_pool, int block_size, float* scores, int64_t ld_scores,
                     float* block_max, int64_t ld_block_max, uint32_t* block_aux,
                     void* stream) {
  return index_score_common("csa2_index_score", 0, mode, n_q, n_heads, d_idx, q_idx, w, k_cache,
                            nullptr, n_entries, kv_start, n_visible, pool_blocks, n_pool,
                            block_size, scores, ld_scores, block_max, ld_block_max, block_aux,
                            stream);
}

int csa2_index_score_shared(int n_q, int n_heads, int d_idx, const void* q_idx, const float* w,
                            const void* k_cache, int64_t n_entries, int64_t kv_start,
                            const int32_t* n_visible, float* scores, int64_t ld_scores,
                            float* block_max, int64_t ld_block_max, void* stream) {
  const char* fn = "csa2_index_score_shared";
  REQUIRE(n_heads == CSA2_IDX_HEADS && d_idx == CSA2_IDX_DIM, CSA2_ERR_UNSUPPORTED,
          "%s: indexer shape %dx%d, only %dx%d is built", fn, n_heads, d_idx, CSA2_IDX_HEADS,
          CSA2_IDX_DIM);
  REQUIRE(n_q >= 0 && n_q <= (1 << 22), CSA2_ERR_INVALID_ARG, "%s: n_q %d out of range", fn, n_q);
  if (n_q == 0) return ok();
  REQUIRE(q_idx && w && k_cache && n_visible && scores, CSA2_ERR_INVALID_ARG,
          "%s: null pointer argument", fn);
  REQUIRE(n_entries >= 0, CSA2_ERR_INVALID_ARG, "%s: n_entries < 0", fn);
  REQUIRE(ld_scores >= 1 && ld_scores <= ((int64_t)1 << 31), CSA2_ERR_INVALID_ARG,
          "%s: ld_scores %lld out of range", fn, (long long)ld_scores);
  REQUIRE(aligned(q_idx, 16) && aligned(k_cache, 16), CSA2_ERR_INVALID_ARG,
          "%s: q_idx and k_cache must be 16-byte aligned", fn);
  REQUIRE(aligned(w, 4) && aligned(scores, 4) && aligned(n_visible, 4), CSA2_ERR_INVALID_ARG,
          "%s: misaligned argument", fn);
  if (block_max != nullptr) {
    REQUIRE(ld_block_max >= (ld_scores + 7) / 8, CSA2_ERR_INVALID_ARG,
            "%s: ld_block_max %lld < ceil(ld_scores/8)", fn, (long long)ld_block_max);
    REQUIRE(aligned(block_max, 4), CSA2_ERR_INVALID_ARG, "%s: misaligned block_max", fn);
  }
  return hip_status(csa2::launch_index_score_shared(
                        n_q, static_cast<const uint16_t*>(q_idx), w,
                        static_cast<const uint8_t*>(k_cache), n_entries, kv_start, n_visible,
                        scores, ld_scores, block_max, ld_block_max,
                        static_cast<hipStream_t>(stream)),
                    fn);
}

int csa2_index_score_mxfp4(csa2_mode_t mode, int n_q, int n_heads, int d_idx, const void* q_idx,
                           const float* w, const void* k_codes, const void* k_scales,
                           int64_t n_entries, const int64_t* kv_start, const int32_t* n_visible,
                           const int32_t* pool_blocks, int n_pool, int block_size, float* scores,
                           int64_t ld_scores, float* block_max, int64_t ld_block_max,
                           uint32_t* block_aux, void* stream) {
  REQUIRE(n_q == 0 || k_scales != nullptr, CSA2_ERR_INVALID_ARG,
          "csa2_index_score_mxfp4: null k_scales");
  return index_score_common("csa2_index_score_mxfp4", 1, mode, n_q, n_heads, d_idx, q_idx, w,
                            k_codes, k_scales, n_entries, kv_start, n_visible, pool_blocks,
                            n_pool, block_size, scores, ld_scores, block_max, ld_block_max,
                            block_aux, stream);
}

int csa2_index_score_bf16(csa2_mode_t mode, int n_q, int n_heads, int d_idx, const void* q_idx,
                          const float* w, const void* k_rows, int64_t n_entries,
                          const int64_t* kv_start, const int32_t* n_visible,
                          const int32_t* pool_blocks, int n_pool, int block_size, float* scores,
                          int64_t ld_scores, float* block_max, int64_t ld_block_max,
                          void* stream) {
  return index_score_common("csa2_index_score_bf16", 2, mode, n_q, n_heads, d_idx, q_idx, w,
                            k_rows, nullptr, n_entries, kv_start, n_visible, pool_blocks, n_pool,
                            block_size, scores, ld_scores, block_max, ld_block_max, nullptr, stream);
}

int csa2_block_mean_keys(int n_q, int d_idx, int block_size, const void* k_cache,
                         int64_t n_entries, const int64_t* kv_start, const int32_t* n_visible,
                         void* km, const int64_t* km_start, int64_t n_km_rows, int64_t max_blocks,
                         int32_t* n_blocks, int last_only, void* stream) {
  const char* fn = "csa2_block_mean_keys";
  REQUIRE(d_idx == CSA2_IDX_DIM, CSA2_ERR_UNSUPPORTED, "%s: d_idx %d, only %d is built", fn,
          d_idx, CSA2_IDX_DIM);
  REQUIRE(block_size == CSA2_CANDIDATE_BLOCK_SIZE, CSA2_ERR_UNSUPPORTED,
          "%s: block_size %d, only %d is built", fn, block_size, CSA2_CANDIDATE_BLOCK_SIZE);
  REQUIRE(n_q >= 0 && n_q <= 65535, CSA2_ERR_INVALID_ARG, "%s: n_q %d out of range", fn, n_q);
  if (n_q == 0) return ok();
  REQUIRE(k_cache && kv_start && n_visible && km && km_start && n_blocks, CSA2_ERR_INVALID_ARG,
          "%s: null pointer argument", fn);
  REQUIRE(n_entries >= 0 && n_km_rows >= 0, CSA2_ERR_INVALID_ARG,
          "%s: n_entries and n_km_rows must be >= 0", fn);
  REQUIRE(max_blocks >= 1 && max_blocks <= ((int64_t)1 << 28), CSA2_ERR_INVALID_ARG,
          "%s: max_blocks %lld out of range", fn, (long long)max_blocks);
  REQUIRE(aligned(k_cache, 8) && aligned(km, 16) && aligned(kv_start, 8) &&
              aligned(km_start, 8) && aligned(n_visible, 4) && aligned(n_blocks, 4),
          CSA2_ERR_INVALID_ARG, "%s: misaligned argument", fn);
  return hip_status(csa2::launch_block_mean_keys(
                        n_q, static_cast<const uint8_t*>(k_cache), n_entries, kv_start, n_visible,
                        static_cast<uint16_t*>(km), km_start, n_km_rows, max_blocks, n_blocks,
                        last_only != 0, static_cast<hipStream_t>(stream)),
                    fn);
}

int csa2_quantize_mxfp8(int n_rows, int d, const void* x, void* codes, void* scales,
                        void* stream) {
  const char* fn = "csa2_quantize_mxfp8";
  REQUIRE(d == CSA2_IDX_DIM, CSA2_ERR_UNSUPPORTED, "%s: d %d, only %d is built", fn, d,
          CSA2_IDX_DIM);
  REQUIRE(n_rows >= 0 && n_rows <= (1 << 26), CSA2_ERR_INVALID_ARG, "%s: n_rows %d out of range",
          fn, n_rows);
  if (n_rows == 0) return ok();
  REQUIRE(x && codes && scales, CSA2_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  REQUIRE(aligned(x, 16) && aligned(codes, 16) && aligned(scales, 4), CSA2_ERR_INVALID_ARG,
          "%s: x and codes must be 16-byte aligned, scales 4-byte aligned", fn);
  return hip_status(csa2::launch_mxfp8_quantize(n_rows, static_cast<const uint16_t*>(x),
                                                static_cast<uint8_t*>(codes),
                                                static_cast<uint8_t*>(scales),
                                                static_cast<hipStream_t>(stream)),
                    fn);
}

// MXFP8-query scoring over MXFP4 keys (k_scales given) or E4M3 keys (k_scales NULL).
static int index_score_q8_common(const char* fn, csa2_mode_t mode, int n_q, int n_heads,
                                 int d_idx, const void* q_codes, const void* q_scales,
                                 const float* w, const void* k_codes, const void* k_scales,
                                 int64_t n_entries, const int64_t* kv_start,
                                 const int32_t* n_visible, const int32_t* pool_blocks, int n_pool,
                                 int block_size, float* scores, int64_t ld_scores,
                                 float* block_max, int64_t ld_block_max, void* stream) {
  REQUIRE(mode == CSA2_FULL || mode == CSA2_REINDEX, CSA2_ERR_INVALID_ARG,
          "%s: mode %d does no scoring (Reuse layers attend with published indices)", fn,
          (int)mode);
  REQUIRE(block_size == CSA2_CANDIDATE_BLOCK_SIZE, CSA2_ERR_UNSUPPORTED,
          "%s: block_size %d, only %d is built", fn, block_size, CSA2_CANDIDATE_BLOCK_SIZE);
  REQUIRE(n_heads == CSA2_IDX_HEADS && d_idx == CSA2_IDX_DIM, CSA2_ERR_UNSUPPORTED,
          "%s: indexer shape %dx%d, only %dx%d is built", fn, n_heads, d_idx, CSA2_IDX_HEADS,
          CSA2_IDX_DIM);
  REQUIRE(n_q >= 0 && n_q <= 65535, CSA2_ERR_INVALID_ARG, "%s: n_q %d out of range", fn, n_q);
  if (n_q == 0) return ok();
  REQUIRE(q_codes && q_scales && w && k_codes && kv_start && n_visible,
          CSA2_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  REQUIRE(scores != nullptr || (mode == CSA2_FULL && block_max != nullptr), CSA2_ERR_INVALID_ARG,
          "%s: scores may be NULL only in FULL mode with block_max", fn);
  REQUIRE(n_entries >= 0, CSA2_ERR_INVALID_ARG, "%s: n_entries < 0", fn);
  REQUIRE(ld_scores >= 1 && ld_scores <= ((int64_t)1 << 31), CSA2_ERR_INVALID_ARG,
          "%s: ld_scores %lld out of range", fn, (long long)ld_scores);
  REQUIRE(aligned(q_codes, 16) && aligned(k_codes, 16), CSA2_ERR_INVALID_ARG,
          "%s: q_codes and k_codes must be 16-byte aligned", fn);
  if (mode == CSA2_REINDEX) {
    REQUIRE(pool_blocks != nullptr, CSA2_ERR_INVALID_ARG, "%s: REINDEX needs pool_blocks", fn);
    REQUIRE(n_pool >= 1 && n_pool <= CSA2_MAX_K, CSA2_ERR_INVALID_ARG,
            "%s: n_pool %d out of range", fn, n_pool);
    REQUIRE(ld_scores >= (int64_t)n_pool * block_size, CSA2_ERR_INVALID_ARG,
            "%s: ld_scores %lld < n_pool*block_size", fn, (long long)ld_scores);
    REQUIRE(aligned(pool_blocks, 4), CSA2_ERR_INVALID_ARG, "%s: misaligned pool_blocks", fn);
  } else {
    REQUIRE(pool_blocks == nullptr, CSA2_ERR_INVALID_ARG, "%s: FULL takes no pool_blocks", fn);
  }
  REQUIRE(aligned(q_scales, 4) && aligned(k_scales, 4) && aligned(w, 4) && aligned(scores, 4) &&
              aligned(kv_start, 8) && aligned(n_visible, 4),
          CSA2_ERR_INVALID_ARG, "%s: misaligned argument", fn);
  if (block_max != nullptr) {
    REQUIRE(ld_block_max >= (ld_scores + 7) / 8, CSA2_ERR_INVALID_ARG,
            "%s: ld_block_max %lld < ceil(ld_scores/8)", fn, (long long)ld_block_max);
    REQUIRE(aligned(block_max, 4), CSA2_ERR_INVALID_ARG, "%s: misaligned block_max", fn);
  }
  return hip_status(csa2::launch_index_score_q8(
                        mode == CSA2_REINDEX, k_scales != nullptr, n_q,
                        static_cast<const uint8_t*>(q_codes),
                        static_cast<const uint8_t*>(q_scales), w,
                        static_cast<const uint8_t*>(k_codes), static_cast<const uint8_t*>(k_scales),
                        n_entries, kv_start, n_visible, pool_blocks,
                        mode == CSA2_REINDEX ? n_pool : 0, scores, ld_scores, block_max,
                        ld_block_max, static_cast<hipStream_t>(stream)),
                    fn);
}

int csa2_index_score_mxfp4_q8(csa2_mode_t mode, int n_q, int n_heads, int d_idx,
                              const void* q_codes, const void* q_scales, const float* w,
                              const void* k_codes, const void* k_scales, int64_t n_entries,
                              const int64_t* kv_start, const int32_t* n_visible,
                              const int32_t* pool_blocks, int n_pool, int block_size,
                              float* scores, int64_t ld_scores, float* block_max,
                              int64_t ld_block_max, void* stream) {
  REQUIRE(n_q == 0 || k_scales != nullptr, CSA2_ERR_INVALID_ARG,
          "csa2_index_score_mxfp4_q8: null k_scales");
  return index_score_q8_common("csa2_index_score_mxfp4_q8", mode, n_q, n_heads, d_idx, q_codes,
                               q_scales, w, k_codes, k_scales, n_entries, kv_start, n_visible,
                               pool_blocks, n_pool, block_size, scores, ld_scores, block_max,
                               ld_block_max, stream);
}

int csa2_index_score_q8(csa2_mode_t mode, int n_q, int n_heads, int d_idx, const void* q_codes,
                        const void* q_scales, const float* w, const void* k_cache,
                        int64_t n_entries, const int64_t* kv_start, const int32_t* n_visible,
                        const int32_t* pool_blocks, int n_pool, int block_size, float* scores,
                        int64_t ld_scores, float* block_max, int64_t ld_block_max, void* stream) {
  return index_score_q8_common("csa2_index_score_q8", mode, n_q, n_heads, d_idx, q_codes,
                               q_scales, w, k_cache, nullptr, n_entries, kv_start, n_visible,
                               pool_blocks, n_pool, block_size, scores, ld_scores, block_max,
                               ld_block_max, stream);
}

int csa2_index_score_shared_q8(int n_q, int n_heads, int d_idx, const void* q_codes,
                               const void* q_scales, const float* w, const void* k_cache,
                               int64_t n_entries, int64_t kv_start, const int32_t* n_visible,
                               float* scores, int64_t ld_scores, float* block_max,
                               int64_t ld_block_max, void* stream) {
  const char* fn = "csa2_index_score_shared_q8";
  REQUIRE(n_heads == CSA2_IDX_HEADS && d_idx == CSA2_IDX_DIM, CSA2_ERR_UNSUPPORTED,
          "%s: indexer shape %dx%d, only %dx%d is built", fn, n_heads, d_idx, CSA2_IDX_HEADS,
          CSA2_IDX_DIM);
  REQUIRE(n_q >= 0 && n_q <= (1 << 22), CSA2_ERR_INVALID_ARG, "%s: n_q %d out of range", fn, n_q);
  if (n_q == 0) return ok();
  REQUIRE(q_codes && q_scales && w && k_cache && n_visible && scores, CSA2_ERR_INVALID_ARG,
          "%s: null pointer argument", fn);
  REQUIRE(n_entries >= 0, CSA2_ERR_INVALID_ARG, "%s: n_entries < 0", fn);
  REQUIRE(ld_scores >= 1 && ld_scores <= ((int64_t)1 << 31), CSA2_ERR_INVALID_ARG,
          "%s: ld_scores %lld out of range", fn, (long long)ld_scores);
  REQUIRE(aligned(q_codes, 16) && aligned(k_cache, 16), CSA2_ERR_INVALID_ARG,
          "%s: q_codes and k_cache must be 16-byte aligned", fn);
  REQUIRE(aligned(q_scales, 4) && aligned(w, 4) && aligned(scores, 4) && aligned(n_visible, 4),
          CSA2_ERR_INVALID_ARG, "%s: misaligned argument", fn);
  if (block_max != nullptr) {
    REQUIRE(ld_block_max >= (ld_scores + 7) / 8, CSA2_ERR_INVALID_ARG,
            "%s: ld_block_max %lld < ceil(ld_scores/8)", fn, (long long)ld_block_max);
    REQUIRE(aligned(block_max, 4), CSA2_ERR_INVALID_ARG, "%s: misaligned block_max", fn);
  }
  return hip_status(csa2::launch_index_score_shared_q8(
                        n_q, static_cast<const uint8_t*>(q_codes),
                        static_cast<const uint8_t*>(q_scales), w,
                        static_cast<const uint8_t*>(k_cache), n_entries, kv_start, n_visible,
                        scores, ld_scores, block_max, ld_block_max,
                        static_cast<hipStream_t>(stream)),
                    fn);
}

int csa2_compress_kv(int m, int n_tokens, int d, const void* c, const void* z, int64_t ld_in,
                     void* out, int64_t ld_out, void* stream) {
  const char* fn = "csa2_compress_kv";
  REQUIRE(d == CSA2_HEAD_DIM, CSA2_ERR_UNSUPPORTED, "%s: d %d, only %d is built", fn, d,
          CSA2_HEAD_DIM);
  REQUIRE(m >= 1 && m <= 8, CSA2_ERR_UNSUPPORTED, "%s: m %d, only 1..8 is built", fn, m);
  REQUIRE(n_tokens >= 0 && n_tokens <= (1 << 28), CSA2_ERR_INVALID_ARG,
          "%s: n_tokens %d out of range", fn, n_tokens);
  const int n_out = n_tokens / m;
  if (n_out == 0) return ok();
  REQUIRE(c && z && out, CSA2_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  REQUIRE(ld_in >= d && ld_in % 8 == 0 && ld_out >= d && ld_out % 8 == 0, CSA2_ERR_INVALID_ARG,
          "%s: ld_in and ld_out must be >= d and multiples of 8", fn);
  REQUIRE(aligned(c, 16) && aligned(z, 16) && aligned(out, 16), CSA2_ERR_INVALID_ARG,
          "%s: c, z and out must be 16-byte aligned", fn);
  return hip_status(csa2::launch_compress(m, n_out, static_cast<const uint16_t*>(c),
                                          static_cast<const uint16_t*>(z), ld_in,
                                          static_cast<uint16_t*>(out), ld_out,
                                          static_cast<hipStream_t>(stream)),
                    fn);
}

int csa2_project_index_key(int n, int d_in, int d_out, const void* entries, int64_t ld_entries,
                           const void* w_ik, void* out, int64_t ld_out, void* stream) {
  const char* fn = "csa2_project_index_key";
  REQUIRE(d_in == CSA2_HEAD_DIM && d_out == CSA2_IDX_DIM, CSA2_ERR_UNSUPPORTED,
          "%s: %d -> %d, only %d -> %d is built", fn, d_in, d_out, CSA2_HEAD_DIM, CSA2_IDX_DIM);
  REQUIRE(n >= 0 && n <= (1 << 28), CSA2_ERR_INVALID_ARG, "%s: n %d out of range", fn, n);
  if (n == 0) return ok();
  REQUIRE(entries && w_ik && out, CSA2_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  REQUIRE(ld_entries >= d_in && ld_entries % 8 == 0 && ld_out >= d_out, CSA2_ERR_INVALID_ARG,
          "%s: ld_entries must be >= %d (a multiple of 8) and ld_out >= %d", fn, d_in, d_out);
  REQUIRE(aligned(entries, 16) && aligned(w_ik, 16) && aligned(out, 2), CSA2_ERR_INVALID_ARG,
          "%s: entries and w_ik must be 16-byte aligned", fn);
  return hip_status(csa2::launch_project_index_key(n, static_cast<const uint16_t*>(entries),
                                                   ld_entries, static_cast<const uint16_t*>(w_ik),
                                                   static_cast<uint16_t*>(out), ld_out,
                                                   static_cast<hipStream_t>(stream)),
                    fn);
}

int csa2_write_latent(int n, const void* x, const int64_t* rows, void* kv_fp4,
                      int64_t kv_fp4_stride, void* kv_scale, int64_t kv_scale_stride,
                      int64_t n_entries, void* stream) {
  REQUIRE(n >= 0 && n <= (1 << 26), CSA2_ERR_INVALID_ARG, "csa2_write_latent: n %d out of range", n);
  if (n == 0) return ok();
  REQUIRE(x && rows && kv_fp4 && kv_scale, CSA2_ERR_INVALID_ARG, "csa2_write_latent: null pointer argument");
  REQUIRE(n_entries >= 0, CSA2_ERR_INVALID_ARG, "csa2_write_latent: n_entries < 0");
  REQUIRE(kv_fp4_stride >= 256 && kv_fp4_stride % 4 == 0 && kv_scale_stride >= 32,
          CSA2_ERR_INVALID_ARG, "csa2_write_latent: strides must be >= 256 (a multiple of 4) and >= 32");
  REQUIRE(aligned(x, 16) && aligned(kv_fp4, 4) && aligned(rows, 8), CSA2_ERR_INVALID_ARG,
          "csa2_write_latent: x must be 16-byte, kv_fp4 4-byte and rows 8-byte aligned");
  return hip_status(csa2::launch_latent_write(n, static_cast<const uint16_t*>(x), rows,
                                              static_cast<uint8_t*>(kv_fp4), kv_fp4_stride,
                                              static_cast<uint8_t*>(kv_scale), kv_scale_stride,
                                              n_entries, static_cast<hipStream_t>(stream)),
                    "csa2_write_latent");
}

int csa2_write_e4m3(int n, int d, const void* x, const int64_t* rows, void* dst,
                    int64_t dst_stride, int64_t n_rows, void* stream) {
  REQUIRE(d == CSA2_IDX_DIM || d == CSA2_HEAD_DIM, CSA2_ERR_UNSUPPORTED,
          "csa2_write_e4m3: d %d, only %d (indexer keys) and %d (window rows) are built", d,
          CSA2_IDX_DIM, CSA2_HEAD_DIM);
  REQUIRE(n >= 0 && n <= (1 << 26), CSA2_ERR_INVALID_ARG, "csa2_write_e4m3: n %d out of range", n);
  if (n == 0) return ok();
  REQUIRE(x && rows && dst, CSA2_ERR_INVALID_ARG, "csa2_write_e4m3: null pointer argument");
  REQUIRE(n_rows >= 0 && dst_stride >= d && dst_stride % 8 == 0, CSA2_ERR_INVALID_ARG,
          "csa2_write_e4m3: need n_rows >= 0 and dst_stride >= d, a multiple of 8");
  REQUIRE(aligned(x, 16) && aligned(dst, 8) && aligned(rows, 8), CSA2_ERR_INVALID_ARG,
          "csa2_write_e4m3: x must be 16-byte, dst and rows 8-byte aligned");
  return hip_status(csa2::launch_e4m3_write(n, d, static_cast<const uint16_t*>(x), rows,
                                            static_cast<uint8_t*>(dst), dst_stride, n_rows,
                                            static_cast<hipStream_t>(stream)),
                    "csa2_write_e4m3");
}

int csa2_write_mxfp4_key(int n, const void* x, const int64_t* rows, void* k_codes,
                         void* k_scales, int64_t n_entries, void* stream) {
  REQUIRE(n >= 0 && n <= (1 << 26), CSA2_ERR_INVALID_ARG, "csa2_write_mxfp4_key: n %d out of range", n);
  if (n == 0) return ok();
  REQUIRE(x && rows && k_codes && k_scales, CSA2_ERR_INVALID_ARG,
          "csa2_write_mxfp4_key: null pointer argument");
  REQUIRE(n_entries >= 0, CSA2_ERR_INVALID_ARG, "csa2_write_mxfp4_key: n_entries < 0");
  REQUIRE(aligned(x, 16) && aligned(k_codes, 4) && aligned(rows, 8), CSA2_ERR_INVALID_ARG,
          "csa2_write_mxfp4_key: x must be 16-byte, k_codes 4-byte and rows 8-byte aligned");
  return hip_status(csa2::launch_mxfp4_key_write(n, static_cast<const uint16_t*>(x), rows,
                                                 static_cast<uint8_t*>(k_codes),
                                                 static_cast<uint8_t*>(k_scales), n_entries,
                                                 static_cast<hipStream_t>(stream)),
                    "csa2_write_mxfp4_key");
}

int csa2_block_pool(int n_q, const float* block_max, int64_t ld_bm, const int32_t* n_visible,
                    int block_size, int n_keep, int32_t* pool_blocks, int64_t ld_pool,
                    void* workspace, size_t ws_bytes, void* stream) {
  (void)workspace;
  (void)ws_bytes;
  REQUIRE(block_size == CSA2_CANDIDATE_BLOCK_SIZE, CSA2_ERR_UNSUPPORTED,
          "csa2_block_pool: block_size %d, only %d is built", block_size, CSA2_CANDIDATE_BLOCK_SIZE);
  REQUIRE(n_q >= 0 && n_q <= 65535, CSA2_ERR_INVALID_ARG, "csa2_block_pool: n_q %d out of range", n_q);
  REQUIRE(n_keep >= 1 && n_keep <= CSA2_MAX_K, CSA2_ERR_INVALID_ARG,
          "csa2_block_pool: n_keep %d out of range [1, %d]", n_keep, CSA2_MAX_K);
  if (n_q == 0) return ok();
  REQUIRE(block_max && n_visible && pool_blocks, CSA2_ERR_INVALID_ARG, "csa2_block_pool: null pointer argument");
  REQUIRE(ld_bm >= 1 && ld_pool >= n_keep, CSA2_ERR_INVALID_ARG,
          "csa2_block_pool: bad leading dimension (ld_bm %lld, ld_pool %lld)", (long long)ld_bm,
          (long long)ld_pool);
  REQUIRE(aligned(block_max, 16) && ld_bm % 4 == 0, CSA2_ERR_INVALID_ARG,
          "csa2_block_pool: block_max must be 16-byte aligned with ld_bm a multiple of 4");
  REQUIRE(aligned(n_visible, 4) && aligned(pool_blocks, 4), CSA2_ERR_INVALID_ARG,
          "csa2_block_pool: misaligned argument");
  return hip_status(csa2::launch_block_pool(n_q, block_max, ld_bm, n_visible, n_keep, pool_blocks,
                                            ld_pool, static_cast<hipStream_t>(stream)),
                    "csa2_block_pool");
}

int csa2_topk(int n_q, const float* scores, int64_t ld_scores, int64_t n_cols,
              const int32_t* n_valid, const float* block_max, int64_t ld_block_max, int k,
              csa2_pool_use_t pool_use, const int32_t* pool_blocks, int n_pool, int block_size,
              int32_t* topk_idx, int64_t ld_idx, void* workspace, size_t ws_bytes,
              void* stream) {
  (void)workspace;
  (void)ws_bytes;
  REQUIRE(block_size == CSA2_CANDIDATE_BLOCK_SIZE, CSA2_ERR_UNSUPPORTED,
          "csa2_topk: block_size %d, only %d is built", block_size, CSA2_CANDIDATE_BLOCK_SIZE);
  REQUIRE(n_q >= 0 && n_q <= 65535, CSA2_ERR_INVALID_ARG, "csa2_topk: n_q %d out of range", n_q);
  REQUIRE(k >= 1 && k <= CSA2_MAX_K, CSA2_ERR_INVALID_ARG, "csa2_topk: k %d out of range [1, %d]", k,
          CSA2_MAX_K);
  if (n_q == 0) return ok();
  REQUIRE(scores && topk_idx, CSA2_ERR_INVALID_ARG, "csa2_topk: null pointer argument");
  REQUIRE(n_cols >= 0 && n_cols <= ld_scores && ld_scores <= ((int64_t)1 << 31), CSA2_ERR_INVALID_ARG,
          "csa2_topk: need 0 <= n_cols <= ld_scores <= 2^31 (n_cols %lld, ld %lld)",
          (long long)n_cols, (long long)ld_scores);
  REQUIRE(ld_idx >= k, CSA2_ERR_INVALID_ARG, "csa2_topk: ld_idx %lld < k", (long long)ld_idx);
  REQUIRE(aligned(scores, 16) && ld_scores % 4 == 0, CSA2_ERR_INVALID_ARG,
          "csa2_topk: scores must be 16-byte aligned with ld_scores a multiple of 4");
  REQUIRE(aligned(topk_idx, 4) && aligned(n_valid, 4), CSA2_ERR_INVALID_ARG,
          "csa2_topk: misaligned argument");
  if (block_max != nullptr)
    REQUIRE(ld_block_max >= (n_cols + 7) / 8 && ld_block_max % 4 == 0 && aligned(block_max, 16),
            CSA2_ERR_INVALID_ARG,
            "csa2_topk: block_max must be 16-byte aligned with ld_block_max >= ceil(n_cols/8) "
            "and a multiple of 4 (got %lld)", (long long)ld_block_max);
  REQUIRE(pool_use == CSA2_POOL_NONE || pool_use == CSA2_POOL_SLOTS ||
              pool_use == CSA2_POOL_CANDIDATES,
          CSA2_ERR_INVALID_ARG, "csa2_topk: pool_use %d unknown", (int)pool_use);
  REQUIRE((pool_use == CSA2_POOL_NONE) == (pool_blocks == nullptr), CSA2_ERR_INVALID_ARG,
          "csa2_topk: pool_blocks must be given exactly when a pool is used");
  if (pool_use != CSA2_POOL_NONE)
    REQUIRE(n_pool >= 1 && n_pool <= CSA2_MAX_K && aligned(pool_blocks, 4), CSA2_ERR_INVALID_ARG,
            "csa2_topk: n_pool %d out of range [1, %d]", n_pool, CSA2_MAX_K);
  if (pool_use == CSA2_POOL_SLOTS)
    REQUIRE(n_cols <= (int64_t)n_pool * block_size, CSA2_ERR_INVALID_ARG,
            "csa2_topk: pool of %d blocks cannot cover %lld slots", n_pool, (long long)n_cols);
  return hip_status(csa2::launch_topk(n_q, scores, ld_scores, n_cols, n_valid,
                                      pool_use == CSA2_POOL_CANDIDATES ? nullptr : block_max,
                                      ld_block_max, k, (int)pool_use, pool_blocks,
                                      pool_use != CSA2_POOL_NONE ? n_pool : 0, topk_idx, ld_idx,
                                      static_cast<hipStream_t>(stream)),
                    "csa2_topk");
}

int csa2_pool_topk(int n_q, const float* block_max, int64_t ld_bm, const int32_t* n_visible,
                   int block_size, int n_keep, int32_t* pool_blocks, int64_t ld_pool,
                   const float* scores, int64_t ld_scores, int64_t n_cols, int k,
                   int32_t* topk_idx, int64_t ld_idx, void* stream) {
  REQUIRE(block_size == CSA2_CANDIDATE_BLOCK_SIZE, CSA2_ERR_UNSUPPORTED,
          "csa2_pool_topk: block_size %d, only %d is built", block_size, CSA2_CANDIDATE_BLOCK_SIZE);
  REQUIRE(n_q >= 0 && n_q <= 65535, CSA2_ERR_INVALID_ARG, "csa2_pool_topk: n_q %d out of range", n_q);
  REQUIRE(n_keep >= 1 && n_keep <= CSA2_MAX_K, CSA2_ERR_INVALID_ARG,
          "csa2_pool_topk: n_keep %d out of range [1, %d]", n_keep, CSA2_MAX_K);
  REQUIRE(k >= 1 && k <= CSA2_MAX_K, CSA2_ERR_INVALID_ARG, "csa2_pool_topk: k %d out of range [1, %d]",
          k, CSA2_MAX_K);
  if (n_q == 0) return ok();
  REQUIRE(block_max && n_visible && pool_blocks && scores && topk_idx, CSA2_ERR_INVALID_ARG,
          "csa2_pool_topk: null pointer argument");
  REQUIRE(ld_bm >= 1 && ld_pool >= n_keep, CSA2_ERR_INVALID_ARG,
          "csa2_pool_topk: bad leading dimension (ld_bm %lld, ld_pool %lld)", (long long)ld_bm,
          (long long)ld_pool);
  REQUIRE(aligned(block_max, 16) && ld_bm % 4 == 0, CSA2_ERR_INVALID_ARG,
          "csa2_pool_topk: block_max must be 16-byte aligned with ld_bm a multiple of 4");
  REQUIRE(n_cols >= 0 && n_cols <= ld_scores && ld_scores <= ((int64_t)1 << 31), CSA2_ERR_INVALID_ARG,
          "csa2_pool_topk: need 0 <= n_cols <= ld_scores <= 2^31 (n_cols %lld, ld %lld)",
          (long long)n_cols, (long long)ld_scores);
  REQUIRE(ld_idx >= k, CSA2_ERR_INVALID_ARG, "csa2_pool_topk: ld_idx %lld < k", (long long)ld_idx);
  REQUIRE(aligned(scores, 16) && ld_scores % 4 == 0, CSA2_ERR_INVALID_ARG,
          "csa2_pool_topk: scores must be 16-byte aligned with ld_scores a multiple of 4");
  REQUIRE(aligned(n_visible, 4) && aligned(pool_blocks, 4) && aligned(topk_idx, 4),
          CSA2_ERR_INVALID_ARG, "csa2_pool_topk: misaligned argument");
  return hip_status(csa2::launch_pool_topk(n_q, block_max, ld_bm, n_visible, n_keep, pool_blocks,
                                           ld_pool, scores, ld_scores, n_cols, k, topk_idx,
                                           ld_idx, static_cast<hipStream_t>(stream)),
                    "csa2_pool_topk");
}

int csa2_pool_candidates(int n_q, const float* block_max, int64_t ld_bm,
                         const int32_t* n_visible, int block_size, int n_keep,
                         int32_t* pool_blocks, int64_t ld_pool, int k, int32_t* cand_blocks,
                         int64_t ld_cand, void* stream) {
  const char* fn = "csa2_pool_candidates";
  REQUIRE(block_size == CSA2_CANDIDATE_BLOCK_SIZE, CSA2_ERR_UNSUPPORTED,
          "%s: block_size %d, only %d is built", fn, block_size, CSA2_CANDIDATE_BLOCK_SIZE);
  REQUIRE(n_q >= 0 && n_q <= 65535, CSA2_ERR_INVALID_ARG, "%s: n_q %d out of range", fn, n_q);
  REQUIRE(n_keep >= 1 && n_keep <= CSA2_MAX_K, CSA2_ERR_INVALID_ARG,
          "%s: n_keep %d out of range [1, %d]", fn, n_keep, CSA2_MAX_K);
  REQUIRE(k >= 1 && k < n_keep, CSA2_ERR_INVALID_ARG, "%s: k %d must lie in [1, n_keep)", fn, k);
  if (n_q == 0) return ok();
  REQUIRE(block_max && n_visible && pool_blocks && cand_blocks, CSA2_ERR_INVALID_ARG,
          "%s: null pointer argument", fn);
  REQUIRE(ld_bm >= 1 && ld_pool >= n_keep && ld_cand >= n_keep, CSA2_ERR_INVALID_ARG,
          "%s: bad leading dimension (ld_bm %lld, ld_pool %lld, ld_cand %lld)", fn,
          (long long)ld_bm, (long long)ld_pool, (long long)ld_cand);
  REQUIRE(aligned(block_max, 16) && ld_bm % 4 == 0, CSA2_ERR_INVALID_ARG,
          "%s: block_max must be 16-byte aligned with ld_bm a multiple of 4", fn);
  REQUIRE(aligned(n_visible, 4) && aligned(pool_blocks, 4) && aligned(cand_blocks, 4),
          CSA2_ERR_INVALID_ARG, "%s: misaligned argument", fn);
  return hip_status(csa2::launch_block_pool_cand(n_q, block_max, ld_bm, n_visible, n_keep,
                                                 pool_blocks, ld_pool, k, cand_blocks, ld_cand,
                                                 static_cast<hipStream_t>(stream)),
                    fn);
}

static int full_select_common(const char* fn, int n_q, const float* block_max, int64_t ld_bm,
                              const int32_t* n_visible, int block_size, int n_keep,
                              int32_t* pool_blocks, int64_t ld_pool, int n_heads, int d_idx,
                              const void* q_idx, const float* w, const void* k_cache,
                              const void* k_scales, int64_t n_entries, const int64_t* kv_start,
                              const uint32_t* block_aux, int k, int32_t* topk_idx, int64_t ld_idx,
                              void* stream) {
  REQUIRE(block_size == CSA2_CANDIDATE_BLOCK_SIZE, CSA2_ERR_UNSUPPORTED,
          "%s: block_size %d, only %d is built", fn, block_size, CSA2_CANDIDATE_BLOCK_SIZE);
  REQUIRE(n_heads == CSA2_IDX_HEADS && d_idx == CSA2_IDX_DIM, CSA2_ERR_UNSUPPORTED,
          "%s: indexer shape %dx%d, only %dx%d is built", fn, n_heads, d_idx,
          CSA2_IDX_HEADS, CSA2_IDX_DIM);
  REQUIRE(n_q >= 0 && n_q <= 65535, CSA2_ERR_INVALID_ARG, "%s: n_q %d out of range", fn, n_q);
  REQUIRE(n_keep >= 1 && n_keep <= CSA2_MAX_K, CSA2_ERR_INVALID_ARG,
          "%s: n_keep %d out of range [1, %d]", fn, n_keep, CSA2_MAX_K);
  REQUIRE(k >= 1 && k < n_keep, CSA2_ERR_INVALID_ARG, "%s: k %d must lie in [1, n_keep)", fn, k);
  if (n_q == 0) return ok();
  REQUIRE(block_max && n_visible && pool_blocks && q_idx && w && k_cache && kv_start && topk_idx &&
              block_aux,
          CSA2_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  REQUIRE(n_entries >= 0, CSA2_ERR_INVALID_ARG, "%s: n_entries < 0", fn);
  REQUIRE(ld_bm >= 1 && ld_pool >= n_keep && ld_idx >= k, CSA2_ERR_INVALID_ARG,
          "%s: bad leading dimension (ld_bm %lld, ld_pool %lld, ld_idx %lld)", fn,
          (long long)ld_bm, (long long)ld_pool, (long long)ld_idx);
  REQUIRE(aligned(block_max, 16) && ld_bm % 4 == 0, CSA2_ERR_INVALID_ARG,
          "%s: block_max must be 16-byte aligned with ld_bm a multiple of 4", fn);
  REQUIRE(aligned(q_idx, 16) && aligned(k_cache, 16), CSA2_ERR_INVALID_ARG,
          "%s: q_idx and the key rows must be 16-byte aligned", fn);
  REQUIRE(k_scales == nullptr || aligned(k_scales, 4), CSA2_ERR_INVALID_ARG,
          "%s: misaligned k_scales", fn);
  REQUIRE(aligned(w, 4) && aligned(kv_start, 8) && aligned(n_visible, 4) &&
              aligned(pool_blocks, 4) && aligned(topk_idx, 4) && aligned(block_aux, 4),
          CSA2_ERR_INVALID_ARG, "%s: misaligned argument", fn);
  return hip_status(csa2::launch_full_select(n_q, block_max, ld_bm, n_visible, n_keep, pool_blocks,
                                             ld_pool, static_cast<const uint16_t*>(q_idx), w,
                                             static_cast<const uint8_t*>(k_cache),
                                             static_cast<const uint8_t*>(k_scales), n_entries,
                                             kv_start, block_aux, k, topk_idx, ld_idx,
                                             static_cast<hipStream_t>(stream)),
                    fn);
}

int csa2_full_select(int n_q, const float* block_max, int64_t ld_bm, const int32_t* n_visible,
                     int block_size, int n_keep, int32_t* pool_blocks, int64_t ld_pool,
                     int n_heads, int d_idx, const void* q_idx, const float* w,
                     const void* k_cache, int64_t n_entries, const int64_t* kv_start,
                     const uint32_t* block_aux, int k, int32_t* topk_idx, int64_t ld_idx,
                     void* stream) {
  return full_select_common("csa2_full_select", n_q, block_max, ld_bm, n_visible, block_size,
                            n_keep, pool_blocks, ld_pool, n_heads, d_idx, q_idx, w, k_cache,
                            nullptr, n_entries, kv_start, block_aux, k, topk_idx, ld_idx, stream);
}

int csa2_full_select_mxfp4(int n_q, const float* block_max, int64_t ld_bm,
                           const int32_t* n_visible, int block_size, int n_keep,
                           int32_t* pool_blocks, int64_t ld_pool, int n_heads, int d_idx,
                           const void* q_idx, const float* w, const void* k_codes,
                           const void* k_scales, int64_t n_entries, const int64_t* kv_start,
                           const uint32_t* block_aux, int k, int32_t* topk_idx, int64_t ld_idx,
                           void* stream) {
  REQUIRE(n_q == 0 || k_scales != nullptr, CSA2_ERR_INVALID_ARG,
          "csa2_full_select_mxfp4: null k_scales");
  return full_select_common("csa2_full_select_mxfp4", n_q, block_max, ld_bm, n_visible,
                            block_size, n_keep, pool_blocks, ld_pool, n_heads, d_idx, q_idx, w,
                            k_codes, k_scales, n_entries, kv_start, block_aux, k, topk_idx,
                            ld_idx, stream);
}

int csa2_sparse_attn(int n_q, int n_heads, int head_dim, const void* q, const void* kv_fp4,
                     int64_t kv_fp4_stride, const void* kv_scale, int64_t kv_scale_stride,
                     int64_t n_entries, const int64_t* kv_start, const int32_t* topk_idx,
                     int64_t ld_idx, int k, const void* window_kv, int64_t n_window_rows,
                     const int64_t* swa_start, const int32_t* n_swa, float softmax_scale,
                     void* out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  REQUIRE(n_heads == CSA2_N_HEADS && head_dim == CSA2_HEAD_DIM, CSA2_ERR_UNSUPPORTED,
          "csa2_sparse_attn: %d heads x %d, only %dx%d is built", n_heads, head_dim, CSA2_N_HEADS,
          CSA2_HEAD_DIM);
  REQUIRE(n_q >= 0 && n_q <= 65535, CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: n_q %d out of range", n_q);
  REQUIRE(k >= 0 && k <= CSA2_MAX_K, CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: k %d out of range [0, %d]",
          k, CSA2_MAX_K);
  if (n_q == 0) return ok();
  REQUIRE(q && kv_fp4 && kv_scale && kv_start && window_kv && swa_start && n_swa && out,
          CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: null pointer argument");
  REQUIRE(k == 0 || topk_idx != nullptr, CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: null topk_idx");
  REQUIRE(k == 0 || ld_idx >= k, CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: ld_idx %lld < k", (long long)ld_idx);
  // The gathers use buffer descriptors whose record stride field holds at most 16,383.
  REQUIRE(kv_fp4_stride >= CSA2_FP4_ROW_BYTES && kv_fp4_stride <= 16368 && kv_fp4_stride % 16 == 0,
          CSA2_ERR_INVALID_ARG,
          "csa2_sparse_attn: kv_fp4_stride %lld must be in [256, 16368] and a multiple of 16",
          (long long)kv_fp4_stride);
  REQUIRE(kv_scale_stride >= CSA2_SCALE_ROW_BYTES && kv_scale_stride <= 16368 &&
              kv_scale_stride % 16 == 0,
          CSA2_ERR_INVALID_ARG,
          "csa2_sparse_attn: kv_scale_stride %lld must be in [32, 16368] and a multiple of 16",
          (long long)kv_scale_stride);
  REQUIRE(n_entries >= 0 && n_window_rows >= 0, CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: negative row count");
  REQUIRE(aligned(q, 16) && aligned(kv_fp4, 16) && aligned(kv_scale, 16) && aligned(window_kv, 16) &&
              aligned(out, 16) && aligned(kv_start, 8) && aligned(swa_start, 8) && aligned(n_swa, 4) &&
              aligned(topk_idx, 4) && aligned(lse, 4),
          CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: misaligned argument");
  (void)workspace;   // no scratch memory is needed (csa2_workspace_bytes returns 0)
  (void)ws_bytes;
  return hip_status(csa2::launch_sparse_attn(
                        n_q, static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(kv_fp4),
                        kv_fp4_stride, static_cast<const uint8_t*>(kv_scale), kv_scale_stride,
                        n_entries, kv_start, topk_idx, ld_idx, k,
                        static_cast<const uint8_t*>(window_kv), n_window_rows, swa_start, n_swa,
                        softmax_scale, static_cast<uint16_t*>(out), lse,
                        static_cast<hipStream_t>(stream)),
                    "csa2_sparse_attn");
}

}  // extern "C"
