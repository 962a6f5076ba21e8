// velox_frustum_overlap: on-device overlap of past chunks' frustum slices
// with the current view's query strips.
//
// The article (sns.style "Velox", Deep analysis, first and third steps)
// represents every past chunk as a camera frustum slice with a depth
// interval, and builds these slices asynchronously next to denoising
// (same section, paragraph on the H200 timing).  With no geometry in the
// article, the slices here are horizontal angle ranges yaw_c +- fov/2 with a
// depth interval; query block i is the i-th of nq equal angular strips of
// the current view with its own depth interval, and
//   O[b,i,c] = (covered fraction of strip i's angle by chunk c's range)
//            * (covered fraction of strip i's depth interval by chunk c's)
// with angle differences wrapped to (-180, 180]; covered[b,i] = any O > 0.
//
// One wave per (b, i); lanes stride over the past chunks.  float32 arithmetic;
// the work is tiny (B*nq*C values) and latency-bound.
#include "velox_internal.h"

namespace velox {
namespace {

__device__ __forceinline__ float wrap_deg(float x) {
  float r = fmodf(x + 180.0f, 360.0f);
  if (r < 0.f) r += 360.0f;
  r -= 180.0f;
  return r == -180.0f ? 180.0f : r;
}

__global__ __launch_bounds__(64) void frustum_overlap_kernel(const float* __restrict__ yaw,
                                                             const float* __restrict__ past_depth,
                                                             const float* __restrict__ query_depth, float fov,
                                                             int nq, int C, float* __restrict__ overlap,
                                                             uint8_t* __restrict__ covered) {
  const int bi = blockIdx.x, lane = threadIdx.x;
  const int b = bi / nq, i = bi % nq;
  const float half = 0.5f * fov;
  const float s0 = -half + fov * (float)i / (float)nq;
  const float s1 = -half + fov * (float)(i + 1) / (float)nq;
  const float q0 = query_depth[2 * bi], q1 = query_depth[2 * bi + 1];
  const float qlen = fmaxf(q1 - q0, 1e-12f);
  const float ycur = yaw[(size_t)b * (C + 1) + C];
  bool any = false;
  for (int c = lane; c < C; c += 64) {
    const float rel = wrap_deg(yaw[(size_t)b * (C + 1) + c] - ycur);
    const float ang = fmaxf(0.f, fminf(s1, rel + half) - fmaxf(s0, rel - half)) / (s1 - s0);
    const float n0 = past_depth[((size_t)b * C + c) * 2], n1 = past_depth[((size_t)b * C + c) * 2 + 1];
    const float dep = fmaxf(0.f, fminf(q1, n1) - fmaxf(q0, n0)) / qlen;
    const float o = ang * dep;
    overlap[(size_t)bi * C + c] = o;
    any |= o > 0.f;
  }
  any = __any(any);
  if (lane == 0) covered[bi] = any ? 1 : 0;
}

}  // namespace

hipError_t launch_frustum_overlap(const velox_problem& p, const float* yaw, const float* past_depth,
                                  const float* query_depth, float fov, float* overlap, uint8_t* covered,
                                  hipStream_t s) {
  const Dims x = dims(p);
  hipLaunchKernelGGL(frustum_overlap_kernel, dim3(x.B * x.nq), dim3(64), 0, s, yaw, past_depth, query_depth, fov,
                     x.nq, x.C, overlap, covered);
  return hipGetLastError();
}

}  // namespace velox
