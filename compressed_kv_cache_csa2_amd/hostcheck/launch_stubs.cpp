// Host-check build of the C ABI: every kernel launcher replaced by a stub that launches
// nothing and reports hipErrorNotSupported, so the argument checks of csa2_api.hip can run
// under AddressSanitizer and UndefinedBehaviorSanitizer on a machine without a GPU. A call
// that passes every check therefore fails with CSA2_ERR_HIP instead of computing anything;
// this library is a test artefact and is never the product's libcsa2.so.
#include "csa2_launch.h"

namespace csa2 {

namespace {
hipError_t stub() { return hipErrorNotSupported; }
}  // namespace

hipError_t launch_index_score(bool, int, int, const uint16_t*, const float*, const uint8_t*,
                              const uint8_t*, int64_t, const int64_t*, const int32_t*,
                              const int32_t*, int, float*, int64_t, float*, int64_t, uint32_t*,
                              hipStream_t) { return stub(); }
hipError_t launch_block_mean_keys(int, const uint8_t*, int64_t, const int64_t*, const int32_t*,
                                  uint16_t*, const int64_t*, int64_t, int64_t, int32_t*, bool,
                                  hipStream_t) { return stub(); }
hipError_t launch_index_score_shared(int, const uint16_t*, const float*, const uint8_t*, int64_t,
                                     int64_t, const int32_t*, float*, int64_t, float*, int64_t,
                                     hipStream_t) { return stub(); }
hipError_t launch_block_pool(int, const float*, int64_t, const int32_t*, int, int32_t*, int64_t,
                             hipStream_t) { return stub(); }
hipError_t launch_topk(int, const float*, int64_t, int64_t, const int32_t*, const float*, int64_t,
                       int, int, const int32_t*, int, int32_t*, int64_t, hipStream_t) {
  return stub();
}
hipError_t launch_pool_topk(int, const float*, int64_t, const int32_t*, int, int32_t*, int64_t,
                            const float*, int64_t, int64_t, int, int32_t*, int64_t,
                            hipStream_t) { return stub(); }
hipError_t launch_block_pool_cand(int, const float*, int64_t, const int32_t*, int, int32_t*,
                                  int64_t, int, int32_t*, int64_t, hipStream_t) { return stub(); }
hipError_t launch_full_select(int, const float*, int64_t, const int32_t*, int, int32_t*, int64_t,
                              const uint16_t*, const float*, const uint8_t*, const uint8_t*,
                              int64_t, const int64_t*, const uint32_t*, int, int32_t*, int64_t,
                              hipStream_t) {
  return stub();
}
hipError_t launch_sparse_attn(int, const uint16_t*, const uint8_t*, int64_t, const uint8_t*,
                              int64_t, int64_t, const int64_t*, const int32_t*, int64_t, int,
                              const uint8_t*, int64_t, const int64_t*, const int32_t*, float,
                              uint16_t*, float*, hipStream_t) { return stub(); }
hipError_t launch_index_score_q8(bool, bool, int, const uint8_t*, const uint8_t*, const float*,
                                 const uint8_t*, const uint8_t*, int64_t, const int64_t*,
                                 const int32_t*, const int32_t*, int, float*, int64_t, float*,
                                 int64_t, hipStream_t) { return stub(); }
hipError_t launch_index_score_shared_q8(int, const uint8_t*, const uint8_t*, const float*,
                                        const uint8_t*, int64_t, int64_t, const int32_t*, float*,
                                        int64_t, float*, int64_t, hipStream_t) { return stub(); }
hipError_t launch_mxfp8_quantize(int, const uint16_t*, uint8_t*, uint8_t*, hipStream_t) {
  return stub();
}
hipError_t launch_compress(int, int, const uint16_t*, const uint16_t*, int64_t, uint16_t*, int64_t,
                           hipStream_t) { return stub(); }
hipError_t launch_project_index_key(int, const uint16_t*, int64_t, const uint16_t*, uint16_t*,
                                    int64_t, hipStream_t) { return stub(); }
hipError_t launch_latent_write(int, const uint16_t*, const int64_t*, uint8_t*, int64_t, uint8_t*,
                               int64_t, int64_t, hipStream_t) { return stub(); }
hipError_t launch_e4m3_write(int, int, const uint16_t*, const int64_t*, uint8_t*, int64_t, int64_t,
                             hipStream_t) { return stub(); }
hipError_t launch_mxfp4_key_write(int, const uint16_t*, const int64_t*, uint8_t*, uint8_t*,
                                  int64_t, hipStream_t) { return stub(); }

}  // namespace csa2
