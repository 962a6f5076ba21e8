// Host side of the C ABI declared in include/velox.h: argument validation,
// workspace layout and kernel launches.  Validation is pure host code and
// works without a GPU; launches are asynchronous on the caller's stream.
#include <math.h>
#include <stdint.h>

#include "velox_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

velox_status hip_status(hipError_t e) {
  if (e == hipSuccess) return VELOX_OK;
  g_last_hip_error = (int)e;
  return VELOX_ERR_HIP;
}

// Checks shared by every entry point.  Routing needs top_k >= ncur (the
// current chunk is always kept); attention only needs a list stride >= 1.
velox_status check_problem(const velox_problem* p, bool routing) {
  if (!p) return VELOX_ERR_NULL_POINTER;
  if (p->batch < 1 || p->heads < 1 || p->head_dim < 1 || p->block < 1 || p->chunk_tokens < p->block ||
      p->past_chunks < 0)
    return VELOX_ERR_BAD_SHAPE;
  if (p->chunk_tokens % p->block) return VELOX_ERR_BAD_SHAPE;
  if (!isfinite(p->alpha) || p->alpha < 0.f) return VELOX_ERR_BAD_SHAPE;
  if (p->modulation != VELOX_MOD_SCALE && p->modulation != VELOX_MOD_LOG_PROB) return VELOX_ERR_BAD_SHAPE;
  if (p->dtype != VELOX_F32 && p->dtype != VELOX_BF16) return VELOX_ERR_UNSUPPORTED;
  if ((p->head_dim != 64 && p->head_dim != 128) || (p->block != 64 && p->block != 128))
    return VELOX_ERR_UNSUPPORTED;
  const int64_t nq = p->chunk_tokens / p->block;
  const int64_t nk = ((int64_t)p->past_chunks + 1) * nq;
  if (p->top_k < (routing ? nq : 1)) return VELOX_ERR_BAD_SHAPE;
  if (nq > VELOX_MAX_QUERY_BLOCKS || nk > VELOX_MAX_KV_BLOCKS) return VELOX_ERR_UNSUPPORTED;
  if ((int64_t)p->batch * p->heads > VELOX_MAX_HEADS_TOTAL) return VELOX_ERR_UNSUPPORTED;
  // Grid sizes: one workgroup per row must fit the 32-bit grid.
  if ((int64_t)p->batch * p->heads * nq > INT32_MAX / 2) return VELOX_ERR_UNSUPPORTED;
  return VELOX_OK;
}

}  // namespace

extern "C" {

velox_status velox_check(const velox_problem* p) { return check_problem(p, true); }

size_t velox_route_workspace_bytes(const velox_problem* p) {
  if (velox_check(p) != VELOX_OK) return 0;
  const velox::Dims x = velox::dims(*p);
  const size_t rows = (size_t)x.B * x.H * x.nq;
  return align256(rows * x.d * sizeof(float)) + align256(rows * x.nk * sizeof(float));
}

velox_status velox_route(const velox_problem* p, const void* q, const void* k, const float* overlap,
                         const uint8_t* covered, int32_t* kv_idx, int32_t* kv_cnt, float* scores, void* workspace,
                         size_t workspace_bytes, velox_stream_t stream) {
  const velox_status st = velox_check(p);
  if (st != VELOX_OK) return st;
  if (!q || !k || !covered || !kv_idx || !kv_cnt || !workspace || (p->past_chunks > 0 && !overlap))
    return VELOX_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k)) return VELOX_ERR_MISALIGNED;
  if (workspace_bytes < velox_route_workspace_bytes(p) || ((uintptr_t)workspace & 255u))
    return VELOX_ERR_WORKSPACE;
  const velox::Dims x = velox::dims(*p);
  const size_t rows = (size_t)x.B * x.H * x.nq;
  float* qbar = static_cast<float*>(workspace);
  float* s = scores ? scores : reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                        align256(rows * x.d * sizeof(float)));
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = velox::launch_pool_queries(*p, q, qbar, hs);
  if (e == hipSuccess) e = velox::launch_block_score(*p, k, qbar, s, hs);
  if (e == hipSuccess) e = velox::launch_modulate_select(*p, s, overlap, covered, kv_idx, kv_cnt, hs);
  return hip_status(e);
}

velox_status velox_score(const velox_problem* p, const void* q, const void* k, float* scores, void* workspace,
                         size_t workspace_bytes, velox_stream_t stream) {
  const velox_status st = velox_check(p);
  if (st != VELOX_OK) return st;
  if (!q || !k || !scores || !workspace) return VELOX_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k)) return VELOX_ERR_MISALIGNED;
  if (workspace_bytes < velox_route_workspace_bytes(p) || ((uintptr_t)workspace & 255u))
    return VELOX_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  float* qbar = static_cast<float*>(workspace);
  hipError_t e = velox::launch_pool_queries(*p, q, qbar, hs);
  if (e == hipSuccess) e = velox::launch_block_score(*p, k, qbar, scores, hs);
  return hip_status(e);
}

velox_status velox_frustum_overlap(const velox_problem* p, const float* yaw, const float* past_depth,
                                   const float* query_depth, float fov_deg, float* overlap, uint8_t* covered,
                                   velox_stream_t stream) {
  const velox_status st = check_problem(p, false);
  if (st != VELOX_OK) return st;
  if (!yaw || !query_depth || !covered || (p->past_chunks > 0 && (!past_depth || !overlap)))
    return VELOX_ERR_NULL_POINTER;
  if (!(fov_deg > 0.f && fov_deg <= 180.f)) return VELOX_ERR_BAD_SHAPE;
  return hip_status(velox::launch_frustum_overlap(*p, yaw, past_depth, query_depth, fov_deg, overlap, covered,
                                                  reinterpret_cast<hipStream_t>(stream)));
}

velox_status velox_pool_keys(const velox_problem* p, const void* k, float* kbar, int32_t cache_blocks,
                             int32_t first_block, int32_t num_blocks, velox_stream_t stream) {
  const velox_status st = check_problem(p, false);
  if (st != VELOX_OK) return st;
  if (!k || !kbar) return VELOX_ERR_NULL_POINTER;
  if (!aligned16(k) || !aligned16(kbar)) return VELOX_ERR_MISALIGNED;
  const velox::Dims x = velox::dims(*p);
  if (first_block < 0 || num_blocks < 0 || (int64_t)first_block + num_blocks > x.nk ||
      (int64_t)first_block + num_blocks > cache_blocks)
    return VELOX_ERR_BAD_SHAPE;
  if ((int64_t)x.B * x.H * num_blocks > INT32_MAX - 3) return VELOX_ERR_UNSUPPORTED;
  if (num_blocks == 0) return VELOX_OK;
  return hip_status(velox::launch_pool_keys(*p, k, kbar, cache_blocks, first_block, num_blocks,
                                            reinterpret_cast<hipStream_t>(stream)));
}

velox_status velox_route_cached(const velox_problem* p, const void* q, const float* kbar, int32_t cache_blocks,
                                const float* overlap, const uint8_t* covered, int32_t* kv_idx, int32_t* kv_cnt,
                                float* scores, void* workspace, size_t workspace_bytes, velox_stream_t stream) {
  const velox_status st = velox_check(p);
  if (st != VELOX_OK) return st;
  if (!q || !kbar || !covered || !kv_idx || !kv_cnt || !workspace || (p->past_chunks > 0 && !overlap))
    return VELOX_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(kbar)) return VELOX_ERR_MISALIGNED;
  const velox::Dims x = velox::dims(*p);
  // Blocks whose pooled keys are read: the past ones, plus the current chunk's
  // when raw scores are returned (their selection does not depend on them).
  const int nscore = scores ? x.nk : x.C * x.nq;
  if (cache_blocks < 0 || cache_blocks < nscore) return VELOX_ERR_BAD_SHAPE;
  if (workspace_bytes < velox_route_workspace_bytes(p) || ((uintptr_t)workspace & 255u))
    return VELOX_ERR_WORKSPACE;
  const size_t rows = (size_t)x.B * x.H * x.nq;
  float* qbar = static_cast<float*>(workspace);
  float* s = scores ? scores : reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                        align256(rows * x.d * sizeof(float)));
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = velox::launch_pool_queries(*p, q, qbar, hs);
  if (e == hipSuccess && nscore > 0) e = velox::launch_cached_score(*p, kbar, cache_blocks, qbar, s, nscore, hs);
  if (e == hipSuccess) e = velox::launch_modulate_select(*p, s, overlap, covered, kv_idx, kv_cnt, hs);
  return hip_status(e);
}

velox_status velox_select(const velox_problem* p, const float* scores, const float* overlap,
                          const uint8_t* covered, int32_t* kv_idx, int32_t* kv_cnt, velox_stream_t stream) {
  const velox_status st = velox_check(p);
  if (st != VELOX_OK) return st;
  if (!scores || !covered || !kv_idx || !kv_cnt || (p->past_chunks > 0 && !overlap)) return VELOX_ERR_NULL_POINTER;
  return hip_status(velox::launch_modulate_select(*p, scores, overlap, covered, kv_idx, kv_cnt,
                                                  reinterpret_cast<hipStream_t>(stream)));
}

velox_status velox_sparse_attn(const velox_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* kv_idx, const int32_t* kv_cnt, void* out, float* lse,
                               velox_stream_t stream) {
  const velox_status st = check_problem(p, false);
  if (st != VELOX_OK) return st;
  if (!q || !k || !v || !kv_idx || !kv_cnt || !out) return VELOX_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return VELOX_ERR_MISALIGNED;
  return hip_status(velox::launch_sparse_attn(*p, q, k, v, kv_idx, kv_cnt, out, lse, 0, nullptr, nullptr,
                                              reinterpret_cast<hipStream_t>(stream)));
}

size_t velox_sparse_attn_split_workspace_bytes(const velox_problem* p, int32_t num_splits) {
  if (check_problem(p, false) != VELOX_OK || num_splits < 1 || num_splits > VELOX_MAX_SPLITS) return 0;
  const velox::Dims x = velox::dims(*p);
  const size_t parts = (size_t)x.B * x.H * x.nq * num_splits;
  return align256(parts * x.blk * x.d * sizeof(float)) + align256(parts * x.blk * sizeof(float));
}

int32_t velox_sparse_attn_auto_splits(const velox_problem* p, int32_t num_cus) {
  if (check_problem(p, false) != VELOX_OK || num_cus < 1) return 1;
  const velox::Dims x = velox::dims(*p);
  const int64_t rows = (int64_t)x.B * x.H * x.nq;
  if (rows >= num_cus) return 1;
  // About two workgroups per CU, each segment keeping at least 4 listed blocks.
  int64_t s = (2 * (int64_t)num_cus + rows - 1) / rows;
  const int64_t by_len = x.top_k / 4 > 1 ? x.top_k / 4 : 1;
  if (s > by_len) s = by_len;
  if (s > VELOX_MAX_SPLITS) s = VELOX_MAX_SPLITS;
  return (int32_t)(s < 1 ? 1 : s);
}

velox_status velox_sparse_attn_split(const velox_problem* p, const void* q, const void* k, const void* v,
                                     const int32_t* kv_idx, const int32_t* kv_cnt, int32_t num_splits, void* out,
                                     float* lse, void* workspace, size_t workspace_bytes, velox_stream_t stream) {
  const velox_status st = check_problem(p, false);
  if (st != VELOX_OK) return st;
  if (num_splits < 1 || num_splits > VELOX_MAX_SPLITS) return VELOX_ERR_BAD_SHAPE;
  if (!q || !k || !v || !kv_idx || !kv_cnt || !out || !workspace) return VELOX_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return VELOX_ERR_MISALIGNED;
  const velox::Dims x = velox::dims(*p);
  const int64_t parts = (int64_t)x.B * x.H * x.nq * num_splits;
  if (parts > INT32_MAX / 2) return VELOX_ERR_UNSUPPORTED;
  if (workspace_bytes < velox_sparse_attn_split_workspace_bytes(p, num_splits) || ((uintptr_t)workspace & 255u))
    return VELOX_ERR_WORKSPACE;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             align256((size_t)parts * x.blk * x.d * sizeof(float)));
  return hip_status(velox::launch_sparse_attn(*p, q, k, v, kv_idx, kv_cnt, out, lse, num_splits, part_o, part_lse,
                                              reinterpret_cast<hipStream_t>(stream)));
}

velox_status velox_mfma_probe(int32_t grid, int32_t iters, int64_t* clocks, float* sink, velox_stream_t stream) {
  if (!clocks || !sink) return VELOX_ERR_NULL_POINTER;
  if (grid < 1 || grid > 65536 || iters < 1) return VELOX_ERR_BAD_SHAPE;
  return hip_status(velox::launch_mfma_probe(grid, iters, clocks, sink, reinterpret_cast<hipStream_t>(stream)));
}

velox_status velox_hbm_read_probe(const void* buf, size_t bytes, int32_t grid, float* sink,
                                  velox_stream_t stream) {
  if (!buf || !sink) return VELOX_ERR_NULL_POINTER;
  if (grid < 1 || grid > 65536 || bytes == 0 || bytes % 16) return VELOX_ERR_BAD_SHAPE;
  if (!aligned16(buf) || ((uintptr_t)sink & 3u)) return VELOX_ERR_MISALIGNED;
  return hip_status(velox::launch_hbm_read_probe(buf, bytes, grid, sink, reinterpret_cast<hipStream_t>(stream)));
}

const char* velox_status_string(velox_status s) {
  switch (s) {
    case VELOX_OK: return "ok";
    case VELOX_ERR_NULL_POINTER: return "a required pointer is NULL";
    case VELOX_ERR_BAD_SHAPE: return "invalid problem shape or parameter";
    case VELOX_ERR_UNSUPPORTED: return "configuration not supported by this build";
    case VELOX_ERR_MISALIGNED: return "tensor pointer not 16-byte aligned";
    case VELOX_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case VELOX_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int velox_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
