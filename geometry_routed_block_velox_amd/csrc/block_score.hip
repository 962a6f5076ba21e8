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
// Both pool keys with the same wave_pool() and score with the same 16 x 16
// fp32 matrix-core tiles (mfma_scores(), same fragments, same steps), so
// cached and direct routing give bit-identical scores.
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

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Scores of one 16 x 16 tile on the fp32 matrix cores (v_mfma_f32_16x16x4_f32):
// s[m][n] = <qbar_m, kbar_n> / sqrt(D).  Lane l feeds query row and key row
// l % 16, and of each the D/4 consecutive elements starting at D/4 * (l / 16):
// in step t the four lane groups supply elements t, D/4 + t, D/2 + t and
// 3D/4 + t, so the D/4 steps take every element once.  a, b: the lane's D/4
// values.  Returns acc[r] = s[4 * (l / 16) + r][l % 16].
template <int D>
__device__ __forceinline__ f32x4 mfma_scores(const float (&a)[D / 4], const float (&b)[D / 4]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < D / 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], b[t], acc, 0, 0, 0);
  const float rs = 1.0f / sqrtf((float)D);
  return acc * rs;
}

// The lane's D/4 values of row `row` (rows of pitch P floats at `rows`) for mfma_scores.
template <int D, int P>
__device__ __forceinline__ void load_frag(const float* rows, int row, int lane, float (&f)[D / 4]) {
  const float4* src = reinterpret_cast<const float4*>(rows + (size_t)row * P + (D / 4) * (lane >> 4));
#pragma unroll
  for (int x = 0; x < D / 16; ++x) {
    const float4 v = src[x];
    f[4 * x] = v.x;
    f[4 * x + 1] = v.y;
    f[4 * x + 2] = v.z;
    f[4 * x + 3] = v.w;
  }
}

// Make every loaded value an output of an (empty) asm statement, so that all
// loads issued before it are in flight together instead of being interleaved
// with the products one latency at a time.
template <int N>
__device__ __forceinline__ void hold(float (&f)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(f[i]));
}

// Write a tile's scores: query blocks m0 + 4*(l/16) + r (< nq), blocks n0 + l%16 (< nlim) of the
// row-major [nq, nk] score rows at `sh`.
__device__ __forceinline__ void store_tile(const f32x4& acc, float* __restrict__ sh, int m0, int n0, int nq,
                                           int nlim, int nk, int lane) {
  const int n = n0 + (lane & 15);
  if (n >= nlim) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + 4 * (lane >> 4) + r;
    if (m < nq) sh[(size_t)m * nk + n] = acc[r];
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
  // 16 x 16 tiles of (query blocks) x (the jn pooled blocks), spread over the 4 waves
  constexpr int NT = kJB / 16;
  const int mtiles = (nq + 15) / 16;
  float* sh = scores + (size_t)bh * nq * nk;
  for (int tile = wave; tile < mtiles * NT; tile += 4) {
    const int mt = tile / NT, nt = tile % NT;
    if (nt * 16 >= jn) continue;
    float a[D / 4], b[D / 4];
    load_frag<D, LD>(qs, min(mt * 16 + (lane & 15), nq - 1), lane, a);
    load_frag<D, LD>(ks, min(nt * 16 + (lane & 15), jn - 1), lane, b);
    hold(a);
    hold(b);
    store_tile(mfma_scores<D>(a, b), sh, mt * 16, j0 + nt * 16, nq, j0 + jn, nk, lane);
  }
}

constexpr int kCJB = 64;  // cached blocks per scoring workgroup: one 16-block tile per wave

// Scores of KV blocks [0, nscore) from cached pooled keys kbar [B*H, cache_blocks, D],
// with the same tiles and fragments as block_score_kernel.  The workgroup stages the
// head's nq pooled queries in LDS (one barrier); each wave loads its own 16 cached rows
// (coalesced, issued before the queries' loads are waited for), moves them into its own
// LDS rows and scores them against the MT*16 (>= nq) query blocks as soon as they have
// arrived, so one wave's products overlap other waves' loads.
// grid = (ceil(nscore / kCJB), B*H); 256 threads; dynamic LDS (nq + kCJB) * kLD<D> floats.
template <int D, int MT>
__global__ __launch_bounds__(256) void cached_score_kernel(const float* __restrict__ kbar,
                                                           const float* __restrict__ qbar,
                                                           float* __restrict__ scores, int nq, int nk,
                                                           int cache_blocks, int nscore) {
  extern __shared__ float lds[];
  constexpr int LD = kLD<D>, C4 = D / 4;
  constexpr int KR = 16 * C4 / 64;    // 16-byte pieces of the wave's 16 rows per lane
  constexpr int QR = MT * 16 * C4 / 256;  // 16-byte query pieces per thread (covers MT*16 >= nq rows)
  float* qs = lds;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* ks = lds + nq * LD + wave * 16 * LD;
  const int bh = blockIdx.y;
  const int n0 = blockIdx.x * kCJB + wave * 16;
  const int jn = min(16, nscore - n0);  // rows of this wave (<= 0: none)
  const float4* q4 = reinterpret_cast<const float4*>(qbar + (size_t)bh * nq * D);
  // a wave past the end (jn <= 0) re-reads row nscore-1 and discards it
  const int jc = max(jn, 1);
  const float4* k4 = reinterpret_cast<const float4*>(kbar + ((size_t)bh * cache_blocks + min(n0, nscore - 1)) * D);
  float4 qr[QR], kr[KR];
#pragma unroll
  for (int u = 0; u < QR; ++u) qr[u] = q4[min(u * 256 + (int)threadIdx.x, nq * C4 - 1)];
#pragma unroll
  for (int u = 0; u < KR; ++u) kr[u] = k4[min(u * 64 + lane, jc * C4 - 1)];
  // the queries are written to LDS first; only their loads (issued first) are waited for
#pragma unroll
  for (int u = 0; u < QR; ++u) asm volatile("" : "+v"(qr[u].x), "+v"(qr[u].y), "+v"(qr[u].z), "+v"(qr[u].w));
#pragma unroll
  for (int u = 0; u < QR; ++u) {
    const int x = u * 256 + (int)threadIdx.x;
    if (x < nq * C4) *reinterpret_cast<float4*>(qs + (x / C4) * LD + (x % C4) * 4) = qr[u];
  }
  // wait for the LDS writes only: the cached rows' loads stay in flight across the barrier
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (jn <= 0) return;
#pragma unroll
  for (int u = 0; u < KR; ++u) asm volatile("" : "+v"(kr[u].x), "+v"(kr[u].y), "+v"(kr[u].z), "+v"(kr[u].w));
#pragma unroll
  for (int u = 0; u < KR; ++u) {
    const int x = u * 64 + lane;
    if (x < jn * C4) *reinterpret_cast<float4*>(ks + (x / C4) * LD + (x % C4) * 4) = kr[u];
  }
  float a[MT][D / 4], b[D / 4];
  load_frag<D, LD>(ks, min(lane & 15, jn - 1), lane, b);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) load_frag<D, LD>(qs, min(mt * 16 + (lane & 15), nq - 1), lane, a[mt]);
  hold(b);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) hold(a[mt]);
  float* sh = scores + (size_t)bh * nq * nk;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) store_tile(mfma_scores<D>(a[mt], b), sh, mt * 16, n0, nq, nscore, nk, lane);
}

template <int D, int MT>
void cached_score_mt(const Dims& x, const float* kbar, int cache_blocks, const float* qbar, float* scores,
                     int nscore, hipStream_t s) {
  const size_t lds = (size_t)(x.nq + kCJB) * kLD<D> * sizeof(float);
  hipLaunchKernelGGL((cached_score_kernel<D, MT>), dim3((nscore + kCJB - 1) / kCJB, x.B * x.H), dim3(256), lds, s,
                     kbar, qbar, scores, x.nq, x.nk, cache_blocks, nscore);
}

template <int D>
hipError_t cached_score_d(const Dims& x, const float* kbar, int cache_blocks, const float* qbar, float* scores,
                          int nscore, hipStream_t s) {
  if (x.nq <= 16)
    cached_score_mt<D, 1>(x, kbar, cache_blocks, qbar, scores, nscore, s);
  else if (x.nq <= 32)
    cached_score_mt<D, 2>(x, kbar, cache_blocks, qbar, scores, nscore, s);
  else if (x.nq <= 64)
    cached_score_mt<D, 4>(x, kbar, cache_blocks, qbar, scores, nscore, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
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
  if (x.d == 128) return cached_score_d<128>(x, kbar, cache_blocks, qbar, scores, nscore, s);
  if (x.d == 64) return cached_score_d<64>(x, kbar, cache_blocks, qbar, scores, nscore, s);
  return hipErrorInvalidValue;
}

}  // namespace velox
