// velox_modulate_select: overlap modulation + per-row top-k.
//
// The article (sns.style "Velox", Deep analysis, third and fourth steps):
// frustum-slice overlap softly modulates the model's block importance in
// regions the history covers, uncovered regions keep the native routing, and
// per region only the needed context is kept.  Per row (b,h,i):
//   m_j = +inf                                  if block j is in the current chunk
//       = s_j * (1 + alpha * overlap[b,i,c(j)]) if the row is covered
//       = s_j                                   otherwise
// (each operation a separately rounded float32 operation), or, in the
// sign-safe mode that reads the importance as the softmax probability of
// s_j, m_j = s_j + log1p(alpha * overlap) for covered past blocks; then keep the
// k_eff largest m_j with ties to the lower index, written in ascending order.
//
// One workgroup (256 threads) per row.  The m_j become order-preserving
// 32-bit keys in LDS (larger key = larger m; -0 is folded onto +0), a
// four-pass 8-bit radix select finds the exact k_eff-th largest key K* and
// how many keys equal to K* are kept; then two workgroup prefix scans in
// block-index order decide the kept ties (lowest index first) and compact
// the kept ids, so the output comes out sorted without a sort.
#include "velox_internal.h"

namespace velox {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float modulated(float s, float alpha, float o) {
#pragma clang fp contract(off)
  const float a = alpha * o;
  const float f = 1.0f + a;
  return s * f;
}

// Sign-safe mode: p_j * (1 + alpha*o) with p_j = softmax(s)_j ranks like this.
// log1p runs in float64 and is rounded once, so the term does not depend on
// the float32 log1p's last-bit behaviour.
__device__ __forceinline__ float modulated_log_prob(float s, float alpha, float o) {
#pragma clang fp contract(off)
  const float a = alpha * o;
  const float lt = (float)log1p((double)a);
  return s + lt;
}

__device__ __forceinline__ uint32_t order_key(float m) {
  uint32_t u = __float_as_uint(m);
  if (m == 0.0f) u = 0u;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Exclusive prefix sum over the workgroup (4 waves); `tmp` holds 4 ints.
__device__ __forceinline__ int block_excl_scan(int x, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(x, lane);
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) base += (w < wave) ? tmp[w] : 0;
  __syncthreads();
  return base + incl - x;
}

// grid = B*H*nq; dynamic LDS = nk * 4 bytes.
__global__ __launch_bounds__(kThreads) void modulate_select_kernel(
    const float* __restrict__ scores, const float* __restrict__ overlap, const uint8_t* __restrict__ covered,
    int32_t* __restrict__ kv_idx, int32_t* __restrict__ kv_cnt, int H, int nq, int nk, int blk, int T, int C,
    float alpha, int top_k, int keff, int log_prob) {
  extern __shared__ uint32_t keys[];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel_digit, sel_above;
  __shared__ int scan_tmp[4];

  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int b = row / (H * nq);
  const int i = row % nq;
  const bool cov = covered[b * nq + i] != 0;
  const float* srow = scores + (size_t)row * nk;
  const float* orow = overlap + ((size_t)b * nq + i) * C;
  int32_t* out = kv_idx + (size_t)row * top_k;

  for (int j = tid; j < nk; j += kThreads) {
    const int c = (j * blk) / T;
    float m;
    if (c >= C)
      m = __builtin_inff();
    else if (cov)
      m = log_prob ? modulated_log_prob(srow[j], alpha, orow[c]) : modulated(srow[j], alpha, orow[c]);
    else
      m = srow[j];
    keys[j] = order_key(m);
  }
  __syncthreads();

  // Radix select of the keff-th largest key: `prefix` holds the digits fixed
  // so far, `kr` the rank still to find among keys matching it.
  uint32_t prefix = 0u, mask = 0u;
  int kr = keff;
  if (keff < nk) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0u;
      __syncthreads();
      for (int j = tid; j < nk; j += kThreads) {
        const uint32_t key = keys[j];
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l owns bins 255-4l .. 252-4l (descending digit order)
        int cnt[4], sum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          cnt[q] = (int)hist[255 - (4 * tid + q)];
          sum += cnt[q];
        }
        int run = wave_incl_scan(sum, tid) - sum;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (run < kr && run + cnt[q] >= kr) {
            sel_digit = 255u - (uint32_t)(4 * tid + q);
            sel_above = (uint32_t)run;
          }
          run += cnt[q];
        }
      }
      __syncthreads();
      prefix |= sel_digit << shift;
      mask |= 255u << shift;
      kr -= (int)sel_above;
      __syncthreads();  // sel_* and hist are rewritten next pass
    }
  } else {
    prefix = 0u;  // keep everything: every key is >= 0 and none is "equal" beyond kr
    kr = nk;
  }
  const uint32_t kstar = prefix;

  // Contiguous ranges per thread keep the scans in block-index order.
  const int per = (nk + kThreads - 1) / kThreads;
  const int j0 = min(nk, tid * per), j1 = min(nk, j0 + per);
  int my_eq = 0;
  for (int j = j0; j < j1; ++j) my_eq += (keys[j] == kstar);
  const int eq_before = block_excl_scan(my_eq, scan_tmp);
  int my_keep = 0, eqr = eq_before;
  for (int j = j0; j < j1; ++j) {
    const uint32_t key = keys[j];
    const bool eq = key == kstar;
    my_keep += (key > kstar) || (eq && eqr < kr);
    eqr += eq;
  }
  int pos = block_excl_scan(my_keep, scan_tmp);
  eqr = eq_before;
  for (int j = j0; j < j1; ++j) {
    const uint32_t key = keys[j];
    const bool eq = key == kstar;
    if ((key > kstar) || (eq && eqr < kr)) out[pos++] = j;
    eqr += eq;
  }
  for (int x = keff + tid; x < top_k; x += kThreads) out[x] = -1;
  if (tid == 0) kv_cnt[row] = keff;
}

}  // namespace

hipError_t launch_modulate_select(const velox_problem& p, const float* scores, const float* overlap,
                                  const uint8_t* covered, int32_t* kv_idx, int32_t* kv_cnt, hipStream_t s) {
  const Dims x = dims(p);
  const int rows = x.B * x.H * x.nq;
  hipLaunchKernelGGL(modulate_select_kernel, dim3(rows), dim3(kThreads), (size_t)x.nk * sizeof(uint32_t), s,
                     scores, overlap, covered, kv_idx, kv_cnt, x.H, x.nq, x.nk, x.blk, x.T, x.C, p.alpha, x.top_k,
                     x.k_eff, p.modulation == VELOX_MOD_LOG_PROB ? 1 : 0);
  return hipGetLastError();
}

}  // namespace velox
