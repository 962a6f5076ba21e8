// Launching entry points of the C ABI declared in include/velox.h: each runs
// its host-side argument check (velox_check.cpp) and then enqueues its
// kernels, asynchronously, on the caller's stream.  Host-only C++: it needs
// HIP's runtime-API types, not the kernel language.
#include <stdint.h>

#include "velox_host.h"
#include "velox_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

velox_status hip_status(hipError_t e) {
  if (e == hipSuccess) return VELOX_OK;
  g_last_hip_error = (int)e;
  return VELOX_ERR_HIP;
}

hipStream_t hip_stream(velox_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// Scores buffer of the routing calls: the caller's, or the workspace past the pooled queries.
float* scores_buffer(const velox_problem* p, float* scores, void* workspace) {
  if (scores) return scores;
  return reinterpret_cast<float*>(static_cast<char*>(workspace) + velox::route_qbar_bytes(*p));
}

}  // namespace

extern "C" {

velox_status velox_route(const velox_problem* p, const void* q, const void* k, const float* overlap,
                         const uint8_t* covered, int32_t* kv_idx, int32_t* kv_cnt, float* scores, void* workspace,
                         size_t workspace_bytes, velox_stream_t stream) {
  const velox_status st = velox::check_route(p, q, k, overlap, covered, kv_idx, kv_cnt, workspace, workspace_bytes);
  if (st != VELOX_OK) return st;
  float* qbar = static_cast<float*>(workspace);
  float* s = scores_buffer(p, scores, workspace);
  hipStream_t hs = hip_stream(stream);
  hipError_t e = velox::launch_pool_queries(*p, q, qbar, hs);
  if (e == hipSuccess) e = velox::launch_block_score(*p, k, qbar, s, hs);
  if (e == hipSuccess) e = velox::launch_modulate_select(*p, s, overlap, covered, kv_idx, kv_cnt, hs);
  return hip_status(e);
}

velox_status velox_route_noalloc(const velox_problem* p, const void* q, const void* k, const float* overlap,
                                 const uint8_t* covered, int32_t* kv_idx, int32_t* kv_cnt, float* scores,
                                 velox_stream_t stream) {
  const velox_status st = velox::check_route_noalloc(p, q, k, overlap, covered, kv_idx, kv_cnt, scores);
  if (st != VELOX_OK) return st;
  void* scratch = nullptr;
  hipError_t e = velox::device_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e);
  // the same layout as velox_route's workspace: pooled queries, then the scores
  float* qbar = static_cast<float*>(scratch);
  float* s = scores_buffer(p, scores, scratch);
  hipStream_t hs = hip_stream(stream);
  e = velox::launch_pool_queries(*p, q, qbar, hs);
  if (e == hipSuccess) e = velox::launch_block_score(*p, k, qbar, s, hs);
  if (e == hipSuccess) e = velox::launch_modulate_select(*p, s, overlap, covered, kv_idx, kv_cnt, hs);
  return hip_status(e);
}

velox_status velox_score(const velox_problem* p, const void* q, const void* k, float* scores, void* workspace,
                         size_t workspace_bytes, velox_stream_t stream) {
  const velox_status st = velox::check_score(p, q, k, scores, workspace, workspace_bytes);
  if (st != VELOX_OK) return st;
  hipStream_t hs = hip_stream(stream);
  float* qbar = static_cast<float*>(workspace);
  hipError_t e = velox::launch_pool_queries(*p, q, qbar, hs);
  if (e == hipSuccess) e = velox::launch_block_score(*p, k, qbar, scores, hs);
  return hip_status(e);
}

velox_status velox_frustum_overlap(const velox_problem* p, const float* yaw, const float* past_depth,
                                   const float* query_depth, float fov_deg, float* overlap, uint8_t* covered,
                                   velox_stream_t stream) {
  const velox_status st = velox::check_frustum_overlap(p, yaw, past_depth, query_depth, fov_deg, overlap, covered);
  if (st != VELOX_OK) return st;
  return hip_status(
      velox::launch_frustum_overlap(*p, yaw, past_depth, query_depth, fov_deg, overlap, covered, hip_stream(stream)));
}

velox_status velox_pool_keys(const velox_problem* p, const void* k, float* kbar, int32_t cache_blocks,
                             int32_t first_block, int32_t num_blocks, velox_stream_t stream) {
  const velox_status st = velox::check_pool_keys(p, k, kbar, cache_blocks, first_block, num_blocks);
  if (st != VELOX_OK) return st;
  if (num_blocks == 0) return VELOX_OK;
  return hip_status(
      velox::launch_pool_keys(*p, k, kbar, cache_blocks, first_block, num_blocks, hip_stream(stream)));
}

velox_status velox_route_cached(const velox_problem* p, const void* q, const float* kbar, int32_t cache_blocks,
                                const float* overlap, const uint8_t* covered, int32_t* kv_idx, int32_t* kv_cnt,
                                float* scores, void* workspace, size_t workspace_bytes, velox_stream_t stream) {
  const velox_status st = velox::check_route_cached(p, q, kbar, cache_blocks, overlap, covered, kv_idx, kv_cnt,
                                                    scores, workspace, workspace_bytes);
  if (st != VELOX_OK) return st;
  const velox::Dims x = velox::dims(*p);
  // Blocks whose pooled keys are read: the past ones, plus the current chunk's
  // when raw scores are returned (their selection does not depend on them).
  const int nscore = scores ? x.nk : x.C * x.nq;
  float* qbar = static_cast<float*>(workspace);
  float* s = scores_buffer(p, scores, workspace);
  hipStream_t hs = hip_stream(stream);
  hipError_t e = velox::launch_pool_queries(*p, q, qbar, hs);
  if (e == hipSuccess && nscore > 0) e = velox::launch_cached_score(*p, kbar, cache_blocks, qbar, s, nscore, hs);
  if (e == hipSuccess) e = velox::launch_modulate_select(*p, s, overlap, covered, kv_idx, kv_cnt, hs);
  return hip_status(e);
}

velox_status velox_select(const velox_problem* p, const float* scores, const float* overlap,
                          const uint8_t* covered, int32_t* kv_idx, int32_t* kv_cnt, velox_stream_t stream) {
  const velox_status st = velox::check_select(p, scores, overlap, covered, kv_idx, kv_cnt);
  if (st != VELOX_OK) return st;
  return hip_status(velox::launch_modulate_select(*p, scores, overlap, covered, kv_idx, kv_cnt, hip_stream(stream)));
}

velox_status velox_sparse_attn(const velox_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* kv_idx, const int32_t* kv_cnt, void* out, float* lse,
                               velox_stream_t stream) {
  const velox_status st = velox::check_sparse_attn(p, q, k, v, kv_idx, kv_cnt, out);
  if (st != VELOX_OK) return st;
  return hip_status(velox::launch_sparse_attn(*p, q, k, v, kv_idx, kv_cnt, out, lse, 0, nullptr, nullptr,
                                              hip_stream(stream)));
}

velox_status velox_sparse_attn_split(const velox_problem* p, const void* q, const void* k, const void* v,
                                     const int32_t* kv_idx, const int32_t* kv_cnt, int32_t num_splits, void* out,
                                     float* lse, void* workspace, size_t workspace_bytes, velox_stream_t stream) {
  const velox_status st =
      velox::check_sparse_attn_split(p, q, k, v, kv_idx, kv_cnt, num_splits, out, workspace, workspace_bytes);
  if (st != VELOX_OK) return st;
  const velox::Dims x = velox::dims(*p);
  const size_t parts = (size_t)x.B * x.H * x.nq * num_splits;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             velox::align256(parts * x.blk * x.d * sizeof(float)));
  return hip_status(velox::launch_sparse_attn(*p, q, k, v, kv_idx, kv_cnt, out, lse, num_splits, part_o, part_lse,
                                              hip_stream(stream)));
}

int velox_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
