// velox_block_score: mean-pooled block importance.
//
// The article (sns.style "Velox", Deep analysis) modulates the block
// importance the model already computes in every layer; here that
// importance is the dot product of the mean-pooled query block and the
// mean-pooled key block, scaled by 1/sqrt(d):
//   qbar_i = mean of Q over query block i, kbar_j = mean of K over KV block j,
//   s[b,h,i,j] = <qbar_i, kbar_j> / sqrt(d).
//
// Two launches:
//   pool_queries_kernel  Q [B,H,T,d] -> qbar [B,H,nq,d] (float32 workspace).
//   block_score_kernel   streams K once: each workgroup pools JB consecutive
//                        KV blocks of one (b,h) and scores them against the
//                        head's qbar kept in LDS.
// Cached variant (the article's Outlook section asks how the method behaves
// for rollouts far longer than 48 chunks; past chunks' keys do not change,
// so their pooled keys can be kept per layer):
//   pool_keys_kernel     K blocks [first, first+num) -> float32 cache kbar.
//   cached_score_kernel  scores from cached kbar rows instead of K.
// Both pool with the same wave_pool() and score with the same score_rows(),
// so cached and direct routing give bit-identical scores.
// All are HBM-bound streaming reads (about 0.25 FLOP per byte).  Each wave
// pools a whole block with 16-byte loads: a wave-wide load covers 64*16 B of
// consecutive rows, the per-lane partial sums are folded with lane
// exchanges, so a block needs no barrier.  Sums are float32.
#include "velox_internal.h"

namespace velox {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Bf16In {
  using T = uint16_t;
  static constexpr int VEC = 8;  // elements per 16-byte load
  static __device__ __forceinline__ void add(const u32x4& r, float* acc) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(w[i] << 16);
      acc[2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

struct F32In {
  using T = float;
  static constexpr int VEC = 4;
  static __device__ __forceinline__ void add(const u32x4& r, float* acc) {
    acc[0] += __uint_as_float(r.x);
    acc[1] += __uint_as_float(r.y);
    acc[2] += __uint_as_float(r.z);
    acc[3] += __uint_as_float(r.w);
  }
};

// One wave pools a [BLK, D] block at `src` into D floats at `dst`
// (written by the first CPR lanes).  Lane l reads 16-byte chunk l % CPR of
// rows l / CPR + RPI * it, so every wave-wide load is one contiguous 1 KiB
// span of the block.
template <class E, int D, int BLK>
__device__ __forceinline__ void wave_pool(const typename E::T* __restrict__ src, float* __restrict__ dst,
                                          int lane) {
  constexpr int VEC = E::VEC;
  constexpr int CPR = D / VEC;   // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;  // rows per wave-wide load
  constexpr int NIT = BLK / RPI;
  static_assert(CPR <= 64 && 64 % CPR == 0 && BLK % RPI == 0, "bad pooling shape");
  const int c = lane % CPR;
  const u32x4* p = reinterpret_cast<const u32x4*>(src) + (lane / CPR) * CPR + c;
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
  // Loads are issued in batches of up to 16 (64 VGPRs) before they are consumed.
  constexpr int NB = NIT < 16 ? NIT : 16;
  static_assert(NIT % NB == 0, "bad batch");
#pragma unroll
  for (int b0 = 0; b0 < NIT; b0 += NB) {
    u32x4 r[NB];
#pragma unroll
    for (int it = 0; it < NB; ++it) r[it] = __builtin_nontemporal_load(p + (b0 + it) * RPI * CPR);
#pragma unroll
    for (int it = 0; it < NB; ++it) E::add(r[it], acc);
  }
#pragma unroll
  for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] += __shfl_xor(acc[v], off);
  if (lane < CPR) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) dst[c * VEC + v] = acc[v] * (1.0f / BLK);
  }
}

// One wave per query block: grid = ceil(B*H*nq / 4) workgroups of 256.
template <class E, int D, int BLK>
__global__ __launch_bounds__(256) void pool_queries_kernel(const typename E::T* __restrict__ q,
                                                           float* __restrict__ qbar, int nblocks) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + wave;
  if (g >= nblocks) return;
  wave_pool<E, D, BLK>(q + (size_t)g * BLK * D, qbar + (size_t)g * D, lane);
}

constexpr int kJB = 32;  // KV blocks per scoring workgroup (measured best of 8, 16, 32, 48, 64)

// One wave per cached block: grid = ceil(B*H*num / 4) workgroups of 256.
template <class E, int D, int BLK>
__global__ __launch_bounds__(256) void pool_keys_kernel(const typename E::T* __restrict__ k, float* __restrict__ kbar,
                                                        int nk, int cache_blocks, int first, int num, int nitems) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + wave;
  if (g >= nitems) return;
  const int bh = g / num, j = first + g % num;
  wave_pool<E, D, BLK>(k + ((size_t)bh * nk + j) * BLK * D, kbar + ((size_t)bh * cache_blocks + j) * D, lane);
}

// Row pitch (floats) of the pooled rows staged in LDS: 16-byte aligned rows whose
// starting banks differ by 4, so the 16-byte reads of up to 16 rows at once are
// conflict-free.
template <int D>
constexpr int kLD = D + 4;

// s[i, j0+jj] = <qs_i, ks_jj> / sqrt(d) for the jn blocks staged in LDS.  Each
// thread computes a 2 x 2 patch (query rows i, i + ceil(nq/2); blocks jj,
// jj + JB/2) from 16-byte LDS reads, so every operand read feeds two FMAs;
// each dot product is one FMA chain over e = 0..D-1 in order.
template <int D>
__device__ __forceinline__ void score_rows(const float* qs, const float* ks, int nq, int jn, int j0, int nk,
                                           float* __restrict__ sh) {
  constexpr int LD = kLD<D>;
  static_assert(kJB % 2 == 0 && D % 4 == 0, "bad scoring patch");
  const float rs = 1.0f / sqrtf((float)D);
  constexpr int JP = kJB / 2;  // block pairs per workgroup
  const int ip_n = (nq + 1) / 2;
  for (int pt = threadIdx.x; pt < ip_n * JP; pt += 256) {
    // patch (i0, i0 + ip_n) x (jj0, jj0 + JP): the 16 blocks read together are consecutive rows
    const int i0 = pt / JP, jj0 = pt % JP;
    if (jj0 >= jn) continue;
    const int i1 = i0 + ip_n < nq ? i0 + ip_n : i0, jj1 = jj0 + JP < jn ? jj0 + JP : jj0;
    const float4* a0 = reinterpret_cast<const float4*>(qs + i0 * LD);
    const float4* a1 = reinterpret_cast<const float4*>(qs + i1 * LD);
    const float4* b0 = reinterpret_cast<const float4*>(ks + jj0 * LD);
    const float4* b1 = reinterpret_cast<const float4*>(ks + jj1 * LD);
    float d00 = 0.f, d01 = 0.f, d10 = 0.f, d11 = 0.f;
#pragma unroll 8
    for (int e = 0; e < D / 4; ++e) {
      const float4 x0 = a0[e], x1 = a1[e], y0 = b0[e], y1 = b1[e];
      d00 = __builtin_fmaf(x0.x, y0.x, d00);
      d01 = __builtin_fmaf(x0.x, y1.x, d01);
      d10 = __builtin_fmaf(x1.x, y0.x, d10);
      d11 = __builtin_fmaf(x1.x, y1.x, d11);
      d00 = __builtin_fmaf(x0.y, y0.y, d00);
      d01 = __builtin_fmaf(x0.y, y1.y, d01);
      d10 = __builtin_fmaf(x1.y, y0.y, d10);
      d11 = __builtin_fmaf(x1.y, y1.y, d11);
      d00 = __builtin_fmaf(x0.z, y0.z, d00);
      d01 = __builtin_fmaf(x0.z, y1.z, d01);
      d10 = __builtin_fmaf(x1.z, y0.z, d10);
      d11 = __builtin_fmaf(x1.z, y1.z, d11);
      d00 = __builtin_fmaf(x0.w, y0.w, d00);
      d01 = __builtin_fmaf(x0.w, y1.w, d01);
      d10 = __builtin_fmaf(x1.w, y0.w, d10);
      d11 = __builtin_fmaf(x1.w, y1.w, d11);
    }
    float* r0 = sh + (size_t)i0 * nk + j0;
    r0[jj0] = d00 * rs;
    if (jj1 != jj0) r0[jj1] = d01 * rs;
    if (i1 != i0) {
      float* r1 = sh + (size_t)i1 * nk + j0;
      r1[jj0] = d10 * rs;
      if (jj1 != jj0) r1[jj1] = d11 * rs;
    }
  }
}

// Copy n pooled rows (D floats each, contiguous in global memory) into LDS rows of pitch kLD<D>, 16 bytes
// per load.
template <int D>
__device__ __forceinline__ void stage_rows(const float* __restrict__ src, float* dst, int n) {
  constexpr int LD = kLD<D>, C4 = D / 4;
  const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll 4
  for (int x = threadIdx.x; x < n * C4; x += 256)
    *reinterpret_cast<float4*>(dst + (x / C4) * LD + (x % C4) * 4) = s4[x];
}

// grid = (ceil(nk / JB), B*H); 256 threads; dynamic LDS (nq + JB) * kLD<D> floats.
template <class E, int D, int BLK>
__global__ __launch_bounds__(256) void block_score_kernel(const typename E::T* __restrict__ k,
                                                          const float* __restrict__ qbar,
                                                          float* __restrict__ scores, int nq, int nk) {
  extern __shared__ float lds[];
  constexpr int LD = kLD<D>;
  float* qs = lds;
  float* ks = lds + nq * LD;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bh = blockIdx.y;
  const int j0 = blockIdx.x * kJB;
  const int jn = min(kJB, nk - j0);

  stage_rows<D>(qbar + (size_t)bh * nq * D, qs, nq);
  const typename E::T* kh = k + (size_t)bh * nk * BLK * D;
  for (int jj = wave; jj < jn; jj += 4) wave_pool<E, D, BLK>(kh + (size_t)(j0 + jj) * BLK * D, ks + jj * LD, lane);
  __syncthreads();
  score_rows<D>(qs, ks, nq, jn, j0, nk, scores + (size_t)bh * nq * nk);
}

// Scores of KV blocks [0, nscore) from cached pooled keys kbar [B*H, cache_blocks, D].
// grid = (ceil(nscore / JB), B*H); 256 threads; dynamic LDS as block_score_kernel.
template <int D>
__global__ __launch_bounds__(256) void cached_score_kernel(const float* __restrict__ kbar,
                                                           const float* __restrict__ qbar,
                                                           float* __restrict__ scores, int nq, int nk,
                                                           int cache_blocks, int nscore) {
  extern __shared__ float lds[];
  constexpr int LD = kLD<D>;
  float* qs = lds;
  float* ks = lds + nq * LD;
  const int bh = blockIdx.y;
  const int j0 = blockIdx.x * kJB;
  const int jn = min(kJB, nscore - j0);
  stage_rows<D>(qbar + (size_t)bh * nq * D, qs, nq);
  stage_rows<D>(kbar + ((size_t)bh * cache_blocks + j0) * D, ks, jn);
  __syncthreads();
  score_rows<D>(qs, ks, nq, jn, j0, nk, scores + (size_t)bh * nq * nk);
}

template <class E, int D, int BLK>
hipError_t pool_q(const Dims& x, const void* q, float* qbar, hipStream_t s) {
  const int nblocks = x.B * x.H * x.nq;
  hipLaunchKernelGGL((pool_queries_kernel<E, D, BLK>), dim3((nblocks + 3) / 4), dim3(256), 0, s,
                     static_cast<const typename E::T*>(q), qbar, nblocks);
  return hipGetLastError();
}

template <class E, int D, int BLK>
hipError_t score(const Dims& x, const void* k, const float* qbar, float* scores, hipStream_t s) {
  const size_t lds = (size_t)(x.nq + kJB) * kLD<D> * sizeof(float);
  hipLaunchKernelGGL((block_score_kernel<E, D, BLK>), dim3((x.nk + kJB - 1) / kJB, x.B * x.H), dim3(256), lds, s,
                     static_cast<const typename E::T*>(k), qbar, scores, x.nq, x.nk);
  return hipGetLastError();
}

template <class E, int D, int BLK>
hipError_t pool_k(const Dims& x, const void* k, float* kbar, int cache_blocks, int first, int num, hipStream_t s) {
  const int nitems = x.B * x.H * num;
  hipLaunchKernelGGL((pool_keys_kernel<E, D, BLK>), dim3((nitems + 3) / 4), dim3(256), 0, s,
                     static_cast<const typename E::T*>(k), kbar, x.nk, cache_blocks, first, num, nitems);
  return hipGetLastError();
}

}  // namespace

#define VELOX_DISPATCH(FN, ...)                                                         \
  do {                                                                                  \
    const bool bf = p.dtype == VELOX_BF16;                                              \
    if (p.head_dim == 128 && p.block == 128)                                            \
      return bf ? FN<Bf16In, 128, 128>(__VA_ARGS__) : FN<F32In, 128, 128>(__VA_ARGS__); \
    if (p.head_dim == 128 && p.block == 64)                                             \
      return bf ? FN<Bf16In, 128, 64>(__VA_ARGS__) : FN<F32In, 128, 64>(__VA_ARGS__);   \
    if (p.head_dim == 64 && p.block == 128)                                             \
      return bf ? FN<Bf16In, 64, 128>(__VA_ARGS__) : FN<F32In, 64, 128>(__VA_ARGS__);   \
    if (p.head_dim == 64 && p.block == 64)                                              \
      return bf ? FN<Bf16In, 64, 64>(__VA_ARGS__) : FN<F32In, 64, 64>(__VA_ARGS__);     \
    return hipErrorInvalidValue;                                                        \
  } while (0)

hipError_t launch_pool_queries(const velox_problem& p, const void* q, float* qbar, hipStream_t s) {
  const Dims x = dims(p);
  VELOX_DISPATCH(pool_q, x, q, qbar, s);
}

hipError_t launch_block_score(const velox_problem& p, const void* k, const float* qbar, float* scores,
                              hipStream_t s) {
  const Dims x = dims(p);
  VELOX_DISPATCH(score, x, k, qbar, scores, s);
}

hipError_t launch_pool_keys(const velox_problem& p, const void* k, float* kbar, int cache_blocks, int first,
                            int num, hipStream_t s) {
  const Dims x = dims(p);
  VELOX_DISPATCH(pool_k, x, k, kbar, cache_blocks, first, num, s);
}

hipError_t launch_cached_score(const velox_problem& p, const float* kbar, int cache_blocks, const float* qbar,
                               float* scores, int nscore, hipStream_t s) {
  const Dims x = dims(p);
  const size_t lds = (size_t)(x.nq + kJB) * (x.d + 4) * sizeof(float);
  const dim3 grid((nscore + kJB - 1) / kJB, x.B * x.H);
  if (x.d == 128)
    hipLaunchKernelGGL(cached_score_kernel<128>, grid, dim3(256), lds, s, kbar, qbar, scores, x.nq, x.nk,
                       cache_blocks, nscore);
  else if (x.d == 64)
    hipLaunchKernelGGL(cached_score_kernel<64>, grid, dim3(256), lds, s, kbar, qbar, scores, x.nq, x.nk,
                       cache_blocks, nscore);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace velox
