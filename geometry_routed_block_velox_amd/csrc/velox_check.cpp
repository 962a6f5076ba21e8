// Host-only part of the C ABI declared in include/velox.h: problem and
// argument checks, workspace sizes, the split heuristic and status strings.
// Plain C++ with no HIP headers: it builds and runs without a GPU toolchain,
// also under the host sanitizers.  The launching entry points
// (velox_api.cpp) call these checks before any device work.
#include <math.h>
#include <stdint.h>

#include "velox_host.h"

namespace velox {

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

namespace {

velox_status check_workspace(const void* workspace, size_t workspace_bytes, size_t needed) {
  if (workspace_bytes < needed || ((uintptr_t)workspace & 255u)) return VELOX_ERR_WORKSPACE;
  return VELOX_OK;
}

}  // namespace

velox_status check_route(const velox_problem* p, const void* q, const void* k, const float* overlap,
                         const uint8_t* covered, const int32_t* kv_idx, const int32_t* kv_cnt, const void* workspace,
                         size_t workspace_bytes) {
  const velox_status st = check_problem(p, true);
  if (st != VELOX_OK) return st;
  if (!q || !k || !covered || !kv_idx || !kv_cnt || !workspace || (p->past_chunks > 0 && !overlap))
    return VELOX_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k)) return VELOX_ERR_MISALIGNED;
  return check_workspace(workspace, workspace_bytes, velox_route_workspace_bytes(p));
}

size_t route_qbar_bytes(const velox_problem& p) {
  const Dims x = dims(p);
  return align256((size_t)x.B * x.H * x.nq * x.d * sizeof(float));
}

velox_status check_route_noalloc(const velox_problem* p, const void* q, const void* k, const float* overlap,
                                 const uint8_t* covered, const int32_t* kv_idx, const int32_t* kv_cnt,
                                 const float* scores) {
  const velox_status st = check_problem(p, true);
  if (st != VELOX_OK) return st;
  if (!q || !k || !covered || !kv_idx || !kv_cnt || (p->past_chunks > 0 && !overlap)) return VELOX_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k)) return VELOX_ERR_MISALIGNED;
  const size_t need = scores ? route_qbar_bytes(*p) : velox_route_workspace_bytes(p);
  if (need > VELOX_NOALLOC_SCRATCH_BYTES) return VELOX_ERR_WORKSPACE;
  return VELOX_OK;
}

velox_status check_score(const velox_problem* p, const void* q, const void* k, const float* scores,
                         const void* workspace, size_t workspace_bytes) {
  const velox_status st = check_problem(p, true);
  if (st != VELOX_OK) return st;
  if (!q || !k || !scores || !workspace) return VELOX_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k)) return VELOX_ERR_MISALIGNED;
  return check_workspace(workspace, workspace_bytes, velox_route_workspace_bytes(p));
}

velox_status check_frustum_overlap(const velox_problem* p, const float* yaw, const float* past_depth,
                                   const float* query_depth, float fov_deg, const float* overlap,
                                   const uint8_t* covered) {
  const velox_status st = check_problem(p, false);
  if (st != VELOX_OK) return st;
  if (!yaw || !query_depth || !covered || (p->past_chunks > 0 && (!past_depth || !overlap)))
    return VELOX_ERR_NULL_POINTER;
  if (!(fov_deg > 0.f && fov_deg <= 180.f)) return VELOX_ERR_BAD_SHAPE;
  return VELOX_OK;
}

velox_status check_pool_keys(const velox_problem* p, const void* k, const float* kbar, int32_t cache_blocks,
                             int32_t first_block, int32_t num_blocks) {
  const velox_status st = check_problem(p, false);
  if (st != VELOX_OK) return st;
  if (!k || !kbar) return VELOX_ERR_NULL_POINTER;
  if (!aligned16(k) || !aligned16(kbar)) return VELOX_ERR_MISALIGNED;
  const Dims x = dims(*p);
  if (first_block < 0 || num_blocks < 0 || (int64_t)first_block + num_blocks > x.nk ||
      (int64_t)first_block + num_blocks > cache_blocks)
    return VELOX_ERR_BAD_SHAPE;
  if ((int64_t)x.B * x.H * num_blocks > INT32_MAX - 3) return VELOX_ERR_UNSUPPORTED;
  return VELOX_OK;
}

velox_status check_route_cached(const velox_problem* p, const void* q, const float* kbar, int32_t cache_blocks,
                                const float* overlap, const uint8_t* covered, const int32_t* kv_idx,
                                const int32_t* kv_cnt, const float* scores, const void* workspace,
                                size_t workspace_bytes) {
  const velox_status st = check_problem(p, true);
  if (st != VELOX_OK) return st;
  if (!q || !kbar || !covered || !kv_idx || !kv_cnt || !workspace || (p->past_chunks > 0 && !overlap))
    return VELOX_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(kbar)) return VELOX_ERR_MISALIGNED;
  const Dims x = dims(*p);
  // Blocks whose pooled keys are read: the past ones, plus the current chunk's
  // when raw scores are returned (their selection does not depend on them).
  const int nscore = scores ? x.nk : x.C * x.nq;
  if (cache_blocks < 0 || cache_blocks < nscore) return VELOX_ERR_BAD_SHAPE;
  return check_workspace(workspace, workspace_bytes, velox_route_workspace_bytes(p));
}

velox_status check_select(const velox_problem* p, const float* scores, const float* overlap, const uint8_t* covered,
                          const int32_t* kv_idx, const int32_t* kv_cnt) {
  const velox_status st = check_problem(p, true);
  if (st != VELOX_OK) return st;
  if (!scores || !covered || !kv_idx || !kv_cnt || (p->past_chunks > 0 && !overlap)) return VELOX_ERR_NULL_POINTER;
  return VELOX_OK;
}

velox_status check_sparse_attn(const velox_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* kv_idx, const int32_t* kv_cnt, const void* out) {
  const velox_status st = check_problem(p, false);
  if (st != VELOX_OK) return st;
  if (!q || !k || !v || !kv_idx || !kv_cnt || !out) return VELOX_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return VELOX_ERR_MISALIGNED;
  return VELOX_OK;
}

velox_status check_sparse_attn_split(const velox_problem* p, const void* q, const void* k, const void* v,
                                     const int32_t* kv_idx, const int32_t* kv_cnt, int32_t num_splits,
                                     const void* out, const void* workspace, size_t workspace_bytes) {
  const velox_status st = check_problem(p, false);
  if (st != VELOX_OK) return st;
  if (num_splits < 1 || num_splits > VELOX_MAX_SPLITS) return VELOX_ERR_BAD_SHAPE;
  if (!q || !k || !v || !kv_idx || !kv_cnt || !out || !workspace) return VELOX_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return VELOX_ERR_MISALIGNED;
  const Dims x = dims(*p);
  const int64_t parts = (int64_t)x.B * x.H * x.nq * num_splits;
  if (parts > INT32_MAX / 2) return VELOX_ERR_UNSUPPORTED;
  return check_workspace(workspace, workspace_bytes, velox_sparse_attn_split_workspace_bytes(p, num_splits));
}

}  // namespace velox

extern "C" {

velox_status velox_check(const velox_problem* p) { return velox::check_problem(p, true); }

size_t velox_route_workspace_bytes(const velox_problem* p) {
  if (velox_check(p) != VELOX_OK) return 0;
  const velox::Dims x = velox::dims(*p);
  const size_t rows = (size_t)x.B * x.H * x.nq;
  return velox::align256(rows * x.d * sizeof(float)) + velox::align256(rows * x.nk * sizeof(float));
}

size_t velox_sparse_attn_split_workspace_bytes(const velox_problem* p, int32_t num_splits) {
  if (velox::check_problem(p, false) != VELOX_OK || num_splits < 1 || num_splits > VELOX_MAX_SPLITS) return 0;
  const velox::Dims x = velox::dims(*p);
  const size_t parts = (size_t)x.B * x.H * x.nq * num_splits;
  return velox::align256(parts * x.blk * x.d * sizeof(float)) + velox::align256(parts * x.blk * sizeof(float));
}

int32_t velox_sparse_attn_auto_splits(const velox_problem* p, int32_t num_cus) {
  if (velox::check_problem(p, false) != VELOX_OK || num_cus < 1) return 1;
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

const char* velox_status_string(int32_t status) {
  switch (status) {
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

}  // extern "C"
