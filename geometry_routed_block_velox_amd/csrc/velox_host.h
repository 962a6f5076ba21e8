// Host-only helpers of libvelox: derived sizes and the argument checks of
// every entry point (velox_check.cpp).  Plain C++, no HIP headers, so the
// checks build and run anywhere, sanitizers included.  Not part of the public
// ABI (include/velox.h).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "velox.h"

namespace velox {

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

inline bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }
inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Checks shared by every entry point.  Routing needs top_k >= ncur (the
// current chunk is always kept); attention only needs a list stride >= 1.
velox_status check_problem(const velox_problem* p, bool routing);

// Argument checks of each entry point, everything short of launching: the
// status the entry point returns before any device work (VELOX_OK: launch).
velox_status check_route(const velox_problem* p, const void* q, const void* k, const float* overlap,
                         const uint8_t* covered, const int32_t* kv_idx, const int32_t* kv_cnt, const void* workspace,
                         size_t workspace_bytes);
// velox_route_noalloc: velox_route's checks without the workspace, and the
// scratch it needs (pooled queries, plus the scores when `scores` is NULL)
// within VELOX_NOALLOC_SCRATCH_BYTES.
velox_status check_route_noalloc(const velox_problem* p, const void* q, const void* k, const float* overlap,
                                 const uint8_t* covered, const int32_t* kv_idx, const int32_t* kv_cnt,
                                 const float* scores);
// Bytes of the pooled queries, the first part of a routing workspace.
size_t route_qbar_bytes(const velox_problem& p);
velox_status check_score(const velox_problem* p, const void* q, const void* k, const float* scores,
                         const void* workspace, size_t workspace_bytes);
velox_status check_frustum_overlap(const velox_problem* p, const float* yaw, const float* past_depth,
                                   const float* query_depth, float fov_deg, const float* overlap,
                                   const uint8_t* covered);
velox_status check_pool_keys(const velox_problem* p, const void* k, const float* kbar, int32_t cache_blocks,
                             int32_t first_block, int32_t num_blocks);
velox_status check_route_cached(const velox_problem* p, const void* q, const float* kbar, int32_t cache_blocks,
                                const float* overlap, const uint8_t* covered, const int32_t* kv_idx,
                                const int32_t* kv_cnt, const float* scores, const void* workspace,
                                size_t workspace_bytes);
velox_status check_select(const velox_problem* p, const float* scores, const float* overlap, const uint8_t* covered,
                          const int32_t* kv_idx, const int32_t* kv_cnt);
velox_status check_sparse_attn(const velox_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* kv_idx, const int32_t* kv_cnt, const void* out);
velox_status check_sparse_attn_split(const velox_problem* p, const void* q, const void* k, const void* v,
                                     const int32_t* kv_idx, const int32_t* kv_cnt, int32_t num_splits,
                                     const void* out, const void* workspace, size_t workspace_bytes);

}  // namespace velox
