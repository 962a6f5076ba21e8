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
// One workgroup of kSelThreads threads per row; thread t holds the keys of
// blocks j = t + kSelThreads*u (u < KPT) in registers.  The m_j become
// order-preserving 32-bit keys (larger key = larger m; -0 is folded onto +0);
// an 8-bit radix select (up to four passes, from the top byte down) narrows
// the k_eff-th largest key to a prefix and the number of keys matching that
// prefix that are kept; then the kept blocks are those above the prefix and
// the first of those matching it in block order, and each one's output slot is
// the number of kept blocks before it, so the list comes out ascending
// without a sort.
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

// The modulated importance m_j of a block in chunk c of a row (see above); o
// is the row's overlap with chunk c (any value when c >= C).
__device__ __forceinline__ float modulated_importance(float s, int c, int C, bool covered, float o, float alpha,
                                                      int log_prob) {
  if (c >= C) return __builtin_inff();
  if (!covered) return s;
  return log_prob ? modulated_log_prob(s, alpha, o) : modulated(s, alpha, o);
}

__device__ __forceinline__ uint32_t order_key(float m) {
  uint32_t u = __float_as_uint(m);
  if (m == 0.0f) u = 0u;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active), in
// registers: shifts by 1, 2, 4, 8 within each row of 16 lanes (lanes without
// a source add 0), then each row's running total is carried on by the row
// broadcasts (lane 15 into rows 1 and 3, lane 31 into rows 2 and 3).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Largest keys-per-thread of a row selection (nk <= kSelThreads * kMaxKpt).
constexpr int kMaxKpt = 32;
// Copies of the first pass's histogram: lane l counts into copy l % kSelCopies,
// each copy one word further along the banks, so lanes whose keys share the top
// byte (most of a row) mostly hit different banks instead of one address.
constexpr int kSelCopies = 8;

// LDS of one row selection (the per-wave counts are an int4: four waves).
static_assert(kSelThreads == 256, "one int4 of per-wave counts");
struct SelectShared {
  uint32_t part[kSelCopies][257];  // first pass: per-copy counts
  uint32_t hist[3][256];           // first-pass totals, then the histograms of passes 2-4 (rotating)
  int4 wave_cnt[2][kMaxKpt];       // per key round: above / matching the final prefix, per wave
};

// Digit of the rank-kr key among the counts h[0..255] (ranked from digit 255
// down); *above = how many counted keys have a larger digit, *inbin = how many
// have that digit.  Every wave computes it from LDS by itself (the result is
// wave-uniform).
__device__ __forceinline__ uint32_t find_digit(const uint32_t* h, int kr, int* above, int* inbin) {
  const int lane = threadIdx.x & 63;
  // lane l owns digits 255-4l .. 252-4l, highest first
  const uint4 v = *reinterpret_cast<const uint4*>(h + 252 - 4 * lane);
  const int c4[4] = {(int)v.w, (int)v.z, (int)v.y, (int)v.x};
  const int sum = c4[0] + c4[1] + c4[2] + c4[3];
  int run = wave_incl_scan(sum) - sum;
  int dig = 0, ab = 0, nb = 0;
  bool hit = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (!hit && run < kr && run + c4[q] >= kr) {
      dig = 255 - (4 * lane + q);
      ab = run;
      nb = c4[q];
      hit = true;
    }
    run += c4[q];
  }
  const uint64_t m = __ballot(hit);  // one lane; none only if the counts miss rank kr
  const int src = m ? __builtin_ctzll(m) : 0;
  *above = __builtin_amdgcn_readlane(ab, src);
  *inbin = __builtin_amdgcn_readlane(nb, src);
  return (uint32_t)__builtin_amdgcn_readlane(dig, src);
}

// Keep the keff largest of the nk keys (thread t holds keys of blocks
// t + kSelThreads*u in key[u]; entries with j >= nk are ignored):
// out[0 .. keff) = their block ids ascending, out[keff .. top_k) = -1,
// *cnt = keff.  At most seven workgroup barriers.
template <int KPT>
__device__ __forceinline__ void select_row(const uint32_t (&key)[KPT], int nk, int keff, int top_k,
                                           SelectShared& sh, int32_t* __restrict__ out, int32_t* __restrict__ cnt) {
  static_assert(KPT >= 1 && KPT <= kMaxKpt, "bad keys per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  bool valid[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) valid[u] = tid + kSelThreads * u < nk;

  // Radix select of the keff-th largest key: `prefix` holds the digits fixed
  // so far (the bits of `mask`), `kr` the rank still to find among keys
  // matching it.  Once kr equals the number of keys matching the prefix, all of
  // them are kept and the remaining digits do not matter.
  uint32_t prefix = 0u, mask = 0u;
  int kr = keff;
  if (keff < nk) {
    for (int x = tid; x < kSelCopies * 257; x += kSelThreads) (&sh.part[0][0])[x] = 0u;
    sh.hist[1][tid] = 0u;
    sh.hist[2][tid] = 0u;
    __syncthreads();
    // pass 1: top byte of every key, into the bank-skewed copies
    uint32_t* mine = sh.part[lane % kSelCopies];
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      if (valid[u]) atomicAdd(&mine[key[u] >> 24], 1u);
    __syncthreads();
    uint32_t tot = 0u;
#pragma unroll
    for (int c = 0; c < kSelCopies; ++c) tot += sh.part[c][tid];
    sh.hist[0][tid] = tot;
    __syncthreads();
    int above, inbin;
    prefix = find_digit(sh.hist[0], kr, &above, &inbin) << 24;
    mask = 0xFF000000u;
    kr -= above;
    // passes 2-4 count the keys that still match into hist[1], hist[2], hist[0];
    // a histogram is cleared only after the barrier that follows its last read
#pragma unroll
    for (int pass = 1; pass < 4; ++pass) {
      if (inbin == kr) break;  // wave-uniform and the same in every wave
      const int shift = 24 - 8 * pass;
      uint32_t* h = sh.hist[pass % 3];
#pragma unroll
      for (int u = 0; u < KPT; ++u)
        if (valid[u] && (key[u] & mask) == prefix) atomicAdd(&h[(key[u] >> shift) & 255u], 1u);
      __syncthreads();
      if (pass == 1) sh.hist[0][tid] = 0u;  // last read: the first-pass search, before this barrier
      prefix |= find_digit(h, kr, &above, &inbin) << shift;
      mask |= 0xFFu << shift;
      kr -= above;
    }
  } else {
    kr = nk;  // keep everything: with an empty mask every key matches the prefix
  }

  // Block order is round-major (u, then wave, then lane).  Per round each wave
  // counts its keys above the prefix and matching it; the kept blocks before a
  // block are the ones above before it plus min(matching ones before it, kr).
  uint64_t bgt[KPT], beq[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    bgt[u] = __ballot(valid[u] && (key[u] & mask) > prefix);
    beq[u] = __ballot(valid[u] && (key[u] & mask) == prefix);
  }
  if (lane < 2 * KPT) {
    // lane 2u: round u above-count, lane 2u+1: equal-count of this wave
    int n = 0;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      if (lane == 2 * u) n = __builtin_popcountll(bgt[u]);
      if (lane == 2 * u + 1) n = __builtin_popcountll(beq[u]);
    }
    reinterpret_cast<int*>(&sh.wave_cnt[lane & 1][lane >> 1])[wave] = n;
  }
  __syncthreads();
  // Lane u (< KPT) reads round u's counts; a scan over the lanes gives, per
  // round, the counts before this wave's part of it.
  int gtot = 0, etot = 0, gw = 0, ew = 0;
  if (lane < KPT) {
    const int4 g = sh.wave_cnt[0][lane], e = sh.wave_cnt[1][lane];
    gtot = g.x + g.y + g.z + g.w;
    etot = e.x + e.y + e.z + e.w;
    gw = (wave > 0 ? g.x : 0) + (wave > 1 ? g.y : 0) + (wave > 2 ? g.z : 0);
    ew = (wave > 0 ? e.x : 0) + (wave > 1 ? e.y : 0) + (wave > 2 ? e.z : 0);
  }
  const int gstart = wave_incl_scan(gtot) - gtot + gw, estart = wave_incl_scan(etot) - etot + ew;
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int gt_before = __builtin_amdgcn_readlane(gstart, u) +
                          __builtin_amdgcn_mbcnt_hi((uint32_t)(bgt[u] >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bgt[u], 0u));
    const int eq_before = __builtin_amdgcn_readlane(estart, u) +
                          __builtin_amdgcn_mbcnt_hi((uint32_t)(beq[u] >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)beq[u], 0u));
    const bool gt = (bgt[u] >> lane) & 1u, eq = (beq[u] >> lane) & 1u;
    const int pos = gt_before + min(eq_before, kr);
    if ((gt || (eq && eq_before < kr)) && pos < keff) out[pos] = tid + kSelThreads * u;  // pos < keff always; a guard
  }
  for (int x = keff + tid; x < top_k; x += kSelThreads) out[x] = -1;
  if (tid == 0) *cnt = keff;
}

}  // namespace velox
