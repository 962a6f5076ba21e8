// velox_modulate_select: overlap modulation + per-row top-k from a score
// matrix in memory (velox_select, and callers that bring their own scores).
// The modulation and the selection are row_select.h's; one workgroup of
// kSelThreads threads per row, dynamic LDS = nk keys.
#include "row_select.h"

namespace velox {
namespace {

__global__ __launch_bounds__(kSelThreads) void modulate_select_kernel(
    const float* __restrict__ scores, const float* __restrict__ overlap, const uint8_t* __restrict__ covered,
    int32_t* __restrict__ kv_idx, int32_t* __restrict__ kv_cnt, int H, int nq, int nk, int blk, int T, int C,
    float alpha, int top_k, int keff, int log_prob) {
  extern __shared__ uint32_t keys[];
  __shared__ SelectShared sh;
  const int row = blockIdx.x;
  const int b = row / (H * nq);
  const int i = row % nq;
  const bool cov = covered[b * nq + i] != 0;
  const float* srow = scores + (size_t)row * nk;
  const float* orow = overlap + ((size_t)b * nq + i) * C;
  for (int j = threadIdx.x; j < nk; j += kSelThreads)
    keys[j] = order_key(modulated_importance(srow[j], j, blk, T, C, cov, orow, alpha, log_prob));
  __syncthreads();
  select_row(keys, nk, keff, top_k, sh, kv_idx + (size_t)row * top_k, kv_cnt + row);
}

}  // namespace

hipError_t launch_modulate_select(const velox_problem& p, const float* scores, const float* overlap,
                                  const uint8_t* covered, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t s) {
  const Dims x = dims(p);
  const int rows = x.B * x.H * x.nq;
  hipLaunchKernelGGL(modulate_select_kernel, dim3(rows), dim3(kSelThreads), (size_t)x.nk * sizeof(uint32_t), s,
                     scores, overlap, covered, kv_idx, kv_cnt, x.H, x.nq, x.nk, x.blk, x.T, x.C, p.alpha, x.top_k,
                     x.k_eff, p.modulation == VELOX_MOD_LOG_PROB ? 1 : 0);
  return hipGetLastError();
}

}  // namespace velox
