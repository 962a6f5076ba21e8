// Internal declarations shared by the HIP translation units of libvelox.
// Not part of the public ABI (include/velox.h).
#pragma once

#include <hip/hip_runtime.h>
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
hipError_t launch_mfma_probe(int grid, int iters, int64_t* clocks, float* sink, hipStream_t s);
hipError_t launch_hbm_read_probe(const void* buf, size_t bytes, int grid, float* sink, hipStream_t s);
hipError_t launch_modulate_select(const velox_problem& p, const float* scores, const float* overlap,
                                  const uint8_t* covered, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t s);
// splits == 0: one workgroup per row, direct output.  splits > 0: split-KV with
// float32 partials part_o [rows*splits, blk, d] and part_lse [rows*splits, blk].
hipError_t launch_sparse_attn(const velox_problem& p, const void* q, const void* k, const void* v,
                              const int32_t* kv_idx, const int32_t* kv_cnt, void* out, float* lse, int splits,
                              float* part_o, float* part_lse, hipStream_t s);

// Derived sizes of a validated problem.
struct Dims {
  int B, H, d, T, C, blk, nq, nk, ncur, top_k, k_eff;
  int64_t N;
};

inline Dims dims(const velox_problem& p) {
  Dims x;
  x.B = p.batch;
  x.H = p.heads;
  x.d = p.head_dim;
  x.T = p.chunk_tokens;
  x.C = p.past_chunks;
  x.blk = p.block;
  x.nq = p.chunk_tokens / p.block;
  x.N = (int64_t)(p.past_chunks + 1) * p.chunk_tokens;
  x.nk = (int)(x.N / p.block);
  x.ncur = x.nq;
  x.top_k = p.top_k;
  x.k_eff = p.top_k < x.nk ? p.top_k : x.nk;
  return x;
}

// Number of XCDs of an MI355X; workgroups are dispatched round-robin over them.
constexpr int kNumXcd = 8;

// Map a dispatch-order workgroup id to a work item so that consecutive work
// items run on the same XCD (and share its L2): XCD x receives the items
// [x*per, (x+1)*per).  Identity when the grid does not divide evenly.
__device__ __forceinline__ int xcd_grouped(int wg, int nwg) {
  if (nwg % kNumXcd) return wg;
  const int per = nwg / kNumXcd;
  return (wg % kNumXcd) * per + wg / kNumXcd;
}

}  // namespace velox
