// Per-row overlap modulation and top-k selection (velox_modulate_select's
// device code, kept apart from the kernel that drives it so that another
// kernel can select a row it has scored itself).  Include from HIP sources
// only.
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
// One workgroup of kSelThreads threads per row.  The m_j become
// order-preserving 32-bit keys in LDS (larger key = larger m; -0 is folded
// onto +0), a four-pass 8-bit radix select finds the exact k_eff-th largest
// key K* and how many keys equal to K* are kept; then two workgroup prefix
// scans in block-index order decide the kept ties (lowest index first) and
// compact the kept ids, so the output comes out sorted without a sort.
#pragma once

#include "velox_internal.h"

namespace velox {

constexpr int kSelThreads = 256;

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

// The modulated importance m_j of block j of a row (see above).
__device__ __forceinline__ float modulated_importance(float s, int j, int blk, int T, int C, bool covered,
                                                      const float* orow, float alpha, int log_prob) {
  const int c = (j * blk) / T;
  if (c >= C) return __builtin_inff();
  if (!covered) return s;
  return log_prob ? modulated_log_prob(s, alpha, orow[c]) : modulated(s, alpha, orow[c]);
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
  for (int w = 0; w < kSelThreads / 64; ++w) base += (w < wave) ? tmp[w] : 0;
  __syncthreads();
  return base + incl - x;
}

// LDS of one row selection besides the keys.
struct SelectShared {
  uint32_t hist[256];
  uint32_t sel_digit, sel_above;
  int scan_tmp[kSelThreads / 64];
};

// Keep the keff largest of the nk keys in LDS (written before a barrier):
// out[0 .. keff) = their block ids ascending, out[keff .. top_k) = -1,
// *cnt = keff.
__device__ __forceinline__ void select_row(const uint32_t* keys, int nk, int keff, int top_k, SelectShared& sh,
                                           int32_t* __restrict__ out, int32_t* __restrict__ cnt) {
  const int tid = threadIdx.x;
  // Radix select of the keff-th largest key: `prefix` holds the digits fixed
  // so far, `kr` the rank still to find among keys matching it.
  uint32_t prefix = 0u, mask = 0u;
  int kr = keff;
  if (keff < nk) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      sh.hist[tid] = 0u;
      __syncthreads();
      for (int j = tid; j < nk; j += kSelThreads) {
        const uint32_t key = keys[j];
        if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l owns bins 255-4l .. 252-4l (descending digit order)
        int c4[4], sum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c4[q] = (int)sh.hist[255 - (4 * tid + q)];
          sum += c4[q];
        }
        int run = wave_incl_scan(sum, tid) - sum;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (run < kr && run + c4[q] >= kr) {
            sh.sel_digit = 255u - (uint32_t)(4 * tid + q);
            sh.sel_above = (uint32_t)run;
          }
          run += c4[q];
        }
      }
      __syncthreads();
      prefix |= sh.sel_digit << shift;
      mask |= 255u << shift;
      kr -= (int)sh.sel_above;
      __syncthreads();  // sel_* and hist are rewritten next pass
    }
  } else {
    prefix = 0u;  // keep everything: every key is >= 0 and none is "equal" beyond kr
    kr = nk;
  }
  const uint32_t kstar = prefix;

  // Contiguous ranges per thread keep the scans in block-index order.
  const int per = (nk + kSelThreads - 1) / kSelThreads;
  const int j0 = min(nk, tid * per), j1 = min(nk, j0 + per);
  int my_eq = 0;
  for (int j = j0; j < j1; ++j) my_eq += (keys[j] == kstar);
  const int eq_before = block_excl_scan(my_eq, sh.scan_tmp);
  int my_keep = 0, eqr = eq_before;
  for (int j = j0; j < j1; ++j) {
    const uint32_t key = keys[j];
    const bool eq = key == kstar;
    my_keep += (key > kstar) || (eq && eqr < kr);
    eqr += eq;
  }
  int pos = block_excl_scan(my_keep, sh.scan_tmp);
  eqr = eq_before;
  for (int j = j0; j < j1; ++j) {
    const uint32_t key = keys[j];
    const bool eq = key == kstar;
    if ((key > kstar) || (eq && eqr < kr)) out[pos++] = j;
    eqr += eq;
  }
  for (int x = keff + tid; x < top_k; x += kSelThreads) out[x] = -1;
  if (tid == 0) *cnt = keff;
}

}  // namespace velox
