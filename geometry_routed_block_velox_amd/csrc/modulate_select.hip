// velox_modulate_select: overlap modulation + per-row top-k from a score
// matrix in memory (velox_select, and callers that bring their own scores).
// The modulation and the selection are row_select.h's; one workgroup of
// kSelThreads threads per row, each holding KPT of the row's keys.
#include "row_select.h"

namespace velox {
namespace {

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void modulate_select_kernel(
    const float* __restrict__ scores, const float* __restrict__ overlap, const uint8_t* __restrict__ covered,
    int32_t* __restrict__ kv_idx, int32_t* __restrict__ kv_cnt, int H, int nq, int nk, int blk, int T, int C,
    float alpha, int top_k, int keff, int log_prob) {
  __shared__ SelectShared sh;
  const int row = blockIdx.x;
  const int b = row / (H * nq);
  const int i = row % nq;
  int cov_raw = covered[b * nq + i];  // waited for together with the scores
  const float* srow = scores + (size_t)row * nk;
  const float* orow = overlap + ((size_t)b * nq + i) * C;
  // Every load is issued before the first is used: one memory latency per
  // row.  Lanes past the row's end re-read its last block; with no past chunk
  // the overlap row is absent and the (unused) overlap value is read from the
  // scores instead.
  const float* obase = C > 0 ? orow : srow;
  const int cmax = C > 0 ? C - 1 : 0;
  // chunk of block j = floor(j / nq), nq = T / blk blocks per chunk: (j + 1/2) / nq
  // is at least 1/(2 nq) >= 1/128 from an integer, far more than float32's
  // error at j < 2^13, so the float product floors exactly.
  const float inv_nq = (float)blk / (float)T;
  float s[KPT], o[KPT];
  int c[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int j = min(u * kSelThreads + (int)threadIdx.x, nk - 1);
    c[u] = (int)(((float)j + 0.5f) * inv_nq);
    s[u] = srow[j];
    o[u] = obase[min(c[u], cmax)];
  }
  // keep the compiler from moving loads behind a use
#pragma unroll
  for (int u = 0; u < KPT; ++u) asm volatile("" ::"v"(s[u]), "v"(o[u]));
  asm volatile("" : "+v"(cov_raw));
  const bool cov = cov_raw != 0;
  uint32_t key[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) key[u] = order_key(modulated_importance(s[u], c[u], C, cov, o[u], alpha, log_prob));
  select_row<KPT>(key, nk, keff, top_k, sh, kv_idx + (size_t)row * top_k, kv_cnt + row);
}

template <int KPT>
void launch_kpt(const Dims& x, const velox_problem& p, const float* scores, const float* overlap,
                const uint8_t* covered, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t s) {
  hipLaunchKernelGGL(modulate_select_kernel<KPT>, dim3(x.B * x.H * x.nq), dim3(kSelThreads), 0, s, scores, overlap,
                     covered, kv_idx, kv_cnt, x.H, x.nq, x.nk, x.blk, x.T, x.C, p.alpha, x.top_k, x.k_eff,
                     p.modulation == VELOX_MOD_LOG_PROB ? 1 : 0);
}

}  // namespace

hipError_t launch_modulate_select(const velox_problem& p, const float* scores, const float* overlap,
                                  const uint8_t* covered, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t s) {
  const Dims x = dims(p);
  if (x.nk <= 4 * kSelThreads)
    launch_kpt<4>(x, p, scores, overlap, covered, kv_idx, kv_cnt, s);
  else if (x.nk <= 8 * kSelThreads)
    launch_kpt<8>(x, p, scores, overlap, covered, kv_idx, kv_cnt, s);
  else if (x.nk <= 16 * kSelThreads)
    launch_kpt<16>(x, p, scores, overlap, covered, kv_idx, kv_cnt, s);
  else if (x.nk <= kMaxKpt * kSelThreads)
    launch_kpt<kMaxKpt>(x, p, scores, overlap, covered, kv_idx, kv_cnt, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace velox
