// Launchers of libvelox for the host-sanitizer build of its host code: the
// argument checks and entry points are the product's own sources, built with
// -fsanitize=address,undefined; no kernel exists here, so a call that passes
// its checks returns VELOX_ERR_HIP (hipErrorNoDevice) instead of launching.
#include "velox_launch.h"

namespace velox {

hipError_t launch_pool_queries(const velox_problem&, const void*, float*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_block_score(const velox_problem&, const void*, const float*, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_pool_keys(const velox_problem&, const void*, float*, int, int, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_cached_score(const velox_problem&, const float*, int, const float*, float*, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_frustum_overlap(const velox_problem&, const float*, const float*, const float*, float, float*,
                                  uint8_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_modulate_select(const velox_problem&, const float*, const float*, const uint8_t*, int32_t*,
                                  int32_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t device_scratch(void** ptr) {
  *ptr = nullptr;
  return hipErrorNoDevice;
}
hipError_t launch_sparse_attn(const velox_problem&, const void*, const void*, const void*, const int32_t*,
                              const int32_t*, void*, float*, int, float*, float*, hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace velox
