// Kernel launchers of libvelox, callable from host-only translation units:
// they need HIP's runtime-API types, not the kernel language.  Not part of
// the public ABI (include/velox.h).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "velox.h"

namespace velox {

// Launchers.  Arguments are validated by the caller (velox_api.cpp).
hipError_t launch_pool_queries(const velox_problem& p, const void* q, float* qbar, hipStream_t s);
hipError_t launch_block_score(const velox_problem& p, const void* k, const float* qbar, float* scores,
                              hipStream_t s);
hipError_t launch_pool_keys(const velox_problem& p, const void* k, float* kbar, int cache_blocks, int first,
                            int num, hipStream_t s);
hipError_t launch_cached_score(const velox_problem& p, const float* kbar, int cache_blocks, const float* qbar,
                               float* scores, int nscore, hipStream_t s);
hipError_t launch_frustum_overlap(const velox_problem& p, const float* yaw, const float* past_depth,
                                  const float* query_depth, float fov, float* overlap, uint8_t* covered,
                                  hipStream_t s);
hipError_t launch_modulate_select(const velox_problem& p, const float* scores, const float* overlap,
                                  const uint8_t* covered, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t s);
// This device's scratch array of VELOX_NOALLOC_SCRATCH_BYTES (a static
// __device__ array): its address on the current device, looked up there on
// the first call and kept per device.  Allocates nothing.
hipError_t device_scratch(void** ptr);
// splits == 0: one workgroup per row, direct output.  splits > 0: split-KV with
// float32 partials part_o [rows*splits, blk, d] and part_lse [rows*splits, blk].
hipError_t launch_sparse_attn(const velox_problem& p, const void* q, const void* k, const void* v,
                              const int32_t* kv_idx, const int32_t* kv_cnt, void* out, float* lse, int splits,
                              float* part_o, float* part_lse, hipStream_t s);

}  // namespace velox
