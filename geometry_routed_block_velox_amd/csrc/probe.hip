// Measurement aids beside the published peaks.
//
// velox_mfma_probe: an MFMA-only kernel that measures the bf16 matrix-core
// rate and the shader clock the chip sustains under that load.
//
// Every wave runs `iters` rounds of 16 independent v_mfma_f32_32x32x16_bf16
// (four accumulator chains, operands in registers, no memory traffic), and
// the first wave of each workgroup records the elapsed shader clocks
// (s_memtime) and the elapsed 100 MHz reference clock (s_memrealtime).  The
// caller times the launch with events; FLOPs = grid * 4 waves * iters * 16 *
// 32768.
//
// velox_hbm_read_probe: a read-only streaming kernel (each workgroup reads a
// contiguous slice with 16-byte loads, sixteen in flight per thread) that
// measures the HBM read bandwidth a kernel can reach, the reference for
// read-dominated kernels such as the block scoring (a device copy mixes reads
// and writes).
#include "velox_internal.h"

namespace velox {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, int64_t* __restrict__ clocks,
                                                         float* __restrict__ sink) {
  const int tid = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(tid + i));
    b[i] = (__bf16)(0.002f * (float)(tid - i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const int64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  }
  const int64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[blockIdx.x * 256 + tid] = s;  // keeps the MFMAs alive
  if (tid == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

template <int U>
__global__ __launch_bounds__(256) void hbm_read_probe_kernel(const float4* __restrict__ p, long long n4,
                                                             float* __restrict__ sink) {
  // Workgroup g reads the contiguous slice [g*per, (g+1)*per) of the buffer,
  // U 16-byte loads per thread in flight, consecutive threads on consecutive words.
  const long long per = (n4 + gridDim.x - 1) / gridDim.x;
  const long long begin = (long long)blockIdx.x * per;
  const long long end = begin + per < n4 ? begin + per : n4;
  long long i = begin + threadIdx.x;
  float acc = 0.f;
  for (; i + (U - 1) * 256 < end; i += U * 256) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
  }
  for (; i < end; i += 256) {
    const float4 a = p[i];
    acc += (a.x + a.y) + (a.z + a.w);
  }
  sink[(long long)blockIdx.x * 256 + threadIdx.x] = acc;  // keeps the loads alive
}

}  // namespace

hipError_t launch_hbm_read_probe(const void* buf, size_t bytes, int grid, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(hbm_read_probe_kernel<16>, dim3(grid), dim3(256), 0, s, static_cast<const float4*>(buf),
                     (long long)(bytes / 16), sink);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int grid, int iters, int64_t* clocks, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(grid), dim3(256), 0, s, iters, clocks, sink);
  return hipGetLastError();
}

}  // namespace velox
