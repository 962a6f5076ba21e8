// velox_sparse_fa: block-skipping tiled attention.
//
// The article (sns.style "Velox", Deep analysis, paragraph on token-block
// granularity) routes at the tile size of a FlashAttention-style kernel so
// that the kernel really skips the blocks the router dropped.  For row
// (b,h,i) and every query token t of block i:
//   out_t = softmax(q_t K_U^T / sqrt(d)) V_U,  U = tokens of the listed blocks,
// computed with an online softmax over the list, one KV block (= one tile)
// at a time.  No causal mask.
//
// bf16 kernel (sparse_fa_bf16_kernel), one workgroup per row, BLK/32 waves,
// each wave owning 32 query tokens:
//  * Scores are formed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the accumulator then holds one query per lane
//    (lane l: query l%32; keys 8(r/4) + 4(l/32) + r%4 of each 32-key tile),
//    so softmax statistics need one cross-lane exchange (lane l <-> l^32) and
//    the output rescale is a per-lane scalar.
//  * O^T = V^T P^T takes P straight from the score registers as the B operand:
//    the contraction over keys may use any key order as long as both operands
//    agree, so the V^T tile is stored in LDS with the keys of every 16-key
//    group permuted to match the accumulator's order; each A operand is then
//    one 16-byte LDS read.  V^T is produced at staging time with an 8x8
//    bf16 register transpose per thread.
//  * K and V^T tiles are double-buffered in LDS (2 x 64 KiB at d = blk = 128):
//    the global loads of the next listed block are issued before the MFMA
//    work on the current one and written to the other buffer after it, one
//    barrier per block.  16-byte LDS chunks are XOR-swizzled by row so that
//    both the staging writes and the MFMA operand reads are conflict-free.
//  * exp2 with log2(e)/sqrt(d) folded into one FMA; the hardware v_exp_f32.
//  * Workgroups are remapped so that the rows of one head run on one XCD and
//    share its L2 while they walk their ascending block lists.
// float32 kernel (sparse_fa_f32_kernel): one thread per query token, plain
// float32 VALU arithmetic; used for float32 problems.
#include "velox_internal.h"

namespace velox {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  uint16_t ua, ub;
  __builtin_memcpy(&ua, &a, 2);
  __builtin_memcpy(&ub, &b, 2);
  return (uint32_t)ua | ((uint32_t)ub << 16);
}

// Transpose an 8x8 block of bf16: in[r] holds row r (8 elements), out[e]
// receives column e (element e of every row, in row order).
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint4& a = in[2 * p];
      const uint4& b = in[2 * p + 1];
      const uint32_t aw = (e >> 1) == 0 ? a.x : (e >> 1) == 1 ? a.y : (e >> 1) == 2 ? a.z : a.w;
      const uint32_t bw = (e >> 1) == 0 ? b.x : (e >> 1) == 1 ? b.y : (e >> 1) == 2 ? b.z : b.w;
      w[p] = (e & 1) ? ((aw >> 16) | (bw & 0xFFFF0000u)) : ((aw & 0xFFFFu) | (bw << 16));
    }
    out[e] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int D, int BLK>
struct FaShape {
  static constexpr int NW = BLK / 32;              // waves, 32 queries each
  static constexpr int NT = NW * 64;               // threads
  static constexpr int KCH = D / 8;                // 16-byte chunks per K row
  static constexpr int VCH = BLK / 8;              // 16-byte chunks per V^T row
  static constexpr int TILE_CHUNKS = BLK * D / 8;  // 16-byte chunks per K (or V) tile
  static constexpr int STAGE_CHUNKS = 2 * TILE_CHUNKS;
  static constexpr int K_LOADS = TILE_CHUNKS / NT;            // K chunks per thread
  static constexpr int V_ITEMS = (BLK / 16) * 2 * (D / 8);     // 8x8 transposes per tile
  static constexpr int V_LOADS = (V_ITEMS + NT - 1) / NT;      // per thread
  static constexpr size_t LDS_BYTES = 2 * STAGE_CHUNKS * 16;
  static_assert(TILE_CHUNKS % NT == 0, "K tile must split evenly");
  static_assert(KCH >= 8 && VCH >= 8, "swizzle needs 8 chunks per row");
};

// Global loads of one KV block into registers.
template <int D, int BLK>
struct TileRegs {
  using S = FaShape<D, BLK>;
  uint4 k[S::K_LOADS];
  uint4 v[S::V_LOADS][8];
};

template <int D, int BLK>
__device__ __forceinline__ void load_tile(TileRegs<D, BLK>& r, const uint16_t* __restrict__ kh,
                                          const uint16_t* __restrict__ vh, int j, int tid) {
  using S = FaShape<D, BLK>;
  const uint4* kb = reinterpret_cast<const uint4*>(kh + (size_t)j * BLK * D);
  const uint4* vb = reinterpret_cast<const uint4*>(vh + (size_t)j * BLK * D);
#pragma unroll
  for (int m = 0; m < S::K_LOADS; ++m) r.k[m] = kb[tid + m * S::NT];
#pragma unroll
  for (int m = 0; m < S::V_LOADS; ++m) {
    const int it = tid + m * S::NT;
    if (S::V_ITEMS % S::NT == 0 || it < S::V_ITEMS) {
      const int c = it % S::KCH, hh = (it / S::KCH) & 1, g = it / (2 * S::KCH);
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int key = 16 * g + 4 * hh + (rr & 3) + ((rr >> 2) << 3);
        r.v[m][rr] = vb[key * S::KCH + c];
      }
    }
  }
}

template <int D, int BLK>
__device__ __forceinline__ void store_tile(const TileRegs<D, BLK>& r, uint4* __restrict__ stage, int tid) {
  using S = FaShape<D, BLK>;
  uint4* ks = stage;
  uint4* vs = stage + S::TILE_CHUNKS;
#pragma unroll
  for (int m = 0; m < S::K_LOADS; ++m) {
    const int x = tid + m * S::NT;
    const int row = x / S::KCH, c = x % S::KCH;
    ks[row * S::KCH + (c ^ swz(row))] = r.k[m];
  }
#pragma unroll
  for (int m = 0; m < S::V_LOADS; ++m) {
    const int it = tid + m * S::NT;
    if (S::V_ITEMS % S::NT == 0 || it < S::V_ITEMS) {
      const int c = it % S::KCH, hh = (it / S::KCH) & 1, g = it / (2 * S::KCH);
      uint4 t[8];
      transpose8x8(r.v[m], t);
      const int vc = 2 * g + hh;  // chunk of keys at positions 16g + 8hh .. +7
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * c + e;
        vs[d * S::VCH + (vc ^ swz(d))] = t[e];
      }
    }
  }
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void sparse_fa_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ kv_cnt, uint16_t* __restrict__ out,
    float* __restrict__ lse, int nq, int nk, int top_k, float scale_log2) {
  using S = FaShape<D, BLK>;
  constexpr int DS = D / 16;    // MFMA k-steps over d (scores)
  constexpr int KT = BLK / 32;  // 32-key tiles per block
  constexpr int DT = D / 32;    // 32-row d tiles of O^T
  constexpr int PS = BLK / 16;  // MFMA k-steps over keys (PV)
  extern __shared__ uint4 smem[];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int qc = lane & 31, hh = lane >> 5;
  const int row = xcd_grouped(blockIdx.x, gridDim.x);
  const int bh = row / nq, iq = row % nq;
  const size_t N = (size_t)nk * BLK;
  const uint16_t* kh = k + (size_t)bh * N * D;
  const uint16_t* vh = v + (size_t)bh * N * D;
  const int32_t* list = kv_idx + (size_t)row * top_k;
  const int cnt = min(max(kv_cnt[row], 0), top_k);

  // Q fragments (B operand of S^T = K Q^T): query qc of this wave, d = 16s + 8hh + 0..7.
  const int tq = iq * BLK + wave * 32 + qc;
  const uint4* qrow = reinterpret_cast<const uint4*>(q + ((size_t)bh * nq * BLK + tq) * D);
  bf16x8 qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) qf[s] = as_bf16x8(qrow[2 * s + hh]);

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -__builtin_inff(), l_run = 0.f;

  auto next_valid = [&](int t) {
    while (t < cnt && (unsigned)list[t] >= (unsigned)nk) ++t;
    return t;
  };

  TileRegs<D, BLK> regs;
  int t = next_valid(0);
  if (t < cnt) {
    load_tile<D, BLK>(regs, kh, vh, list[t], tid);
    store_tile<D, BLK>(regs, smem, tid);
  }
  __syncthreads();
  int buf = 0;
  while (t < cnt) {
    const int tn = next_valid(t + 1);
    if (tn < cnt) load_tile<D, BLK>(regs, kh, vh, list[tn], tid);

    const uint4* ks = smem + buf * S::STAGE_CHUNKS;
    const uint4* vs = ks + S::TILE_CHUNKS;

    // S^T tile: rows = keys 32kt + ..., cols = this wave's 32 queries.
    f32x16 sacc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
      const int krow = 32 * kt + qc;
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const bf16x8 a = as_bf16x8(ks[krow * S::KCH + ((2 * s + hh) ^ swz(krow))]);
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kt], 0, 0, 0);
      }
    }

    // Online softmax for query qc (keys split between lanes l and l^32).
    float mx = sacc[0][0];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float resc = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
    const float mb = m_new * scale_log2;
    float lsum = 0.f;
    bf16x8 pb[PS];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][r], scale_log2, -mb));
        lsum += p;
        pb[2 * kt + (r >> 3)][r & 7] = (__bf16)p;
      }
    }
    l_run = l_run * resc + lsum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= resc;

    // O^T += V^T P^T.
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 32 * dt + qc;
#pragma unroll
      for (int s = 0; s < PS; ++s) {
        const bf16x8 a = as_bf16x8(vs[d * S::VCH + ((2 * s + hh) ^ swz(d))]);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s], oacc[dt], 0, 0, 0);
      }
    }

    if (tn < cnt) store_tile<D, BLK>(regs, smem + (buf ^ 1) * S::STAGE_CHUNKS, tid);
    __syncthreads();
    buf ^= 1;
    t = tn;
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  uint16_t* orow = out + ((size_t)bh * nq * BLK + tq) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * dt + 8 * rq + 4 * hh;
      uint2 w;
      w.x = pack_bf16x2(oacc[dt][4 * rq] * inv, oacc[dt][4 * rq + 1] * inv);
      w.y = pack_bf16x2(oacc[dt][4 * rq + 2] * inv, oacc[dt][4 * rq + 3] * inv);
      *reinterpret_cast<uint2*>(orow + d0) = w;
    }
  }
  if (lse && hh == 0) {
    lse[(size_t)bh * nq * BLK + tq] =
        l_tot > 0.f ? (m_run * scale_log2 + __builtin_log2f(l_tot)) * 0.69314718055994531f : -__builtin_inff();
  }
}

// float32 path: one thread per query token, K and V tiles staged in LDS.
template <int D, int BLK>
__global__ __launch_bounds__(BLK) void sparse_fa_f32_kernel(const float* __restrict__ q,
                                                            const float* __restrict__ k,
                                                            const float* __restrict__ v,
                                                            const int32_t* __restrict__ kv_idx,
                                                            const int32_t* __restrict__ kv_cnt,
                                                            float* __restrict__ out, float* __restrict__ lse,
                                                            int nq, int nk, int top_k, float scale_log2) {
  extern __shared__ float fs[];
  float* kt = fs;
  float* vt = fs + BLK * D;
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int bh = row / nq, iq = row % nq;
  const size_t N = (size_t)nk * BLK;
  const float* kh = k + (size_t)bh * N * D;
  const float* vh = v + (size_t)bh * N * D;
  const int32_t* list = kv_idx + (size_t)row * top_k;
  const int cnt = min(max(kv_cnt[row], 0), top_k);
  const size_t tq = (size_t)bh * nq * BLK + (size_t)iq * BLK + tid;

  float qv[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qv[e] = q[tq * D + e] * scale_log2;
    o[e] = 0.f;
  }
  float m_run = -__builtin_inff(), l_run = 0.f;
  for (int t = 0; t < cnt; ++t) {
    const int j = list[t];
    if ((unsigned)j >= (unsigned)nk) continue;
    __syncthreads();
    const float4* ksrc = reinterpret_cast<const float4*>(kh + (size_t)j * BLK * D);
    const float4* vsrc = reinterpret_cast<const float4*>(vh + (size_t)j * BLK * D);
    for (int x = tid; x < BLK * D / 4; x += BLK) {
      reinterpret_cast<float4*>(kt)[x] = ksrc[x];
      reinterpret_cast<float4*>(vt)[x] = vsrc[x];
    }
    __syncthreads();
    for (int u = 0; u < BLK; ++u) {
      float lg = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) lg += qv[e] * kt[u * D + e];
      if (lg > m_run) {
        const float resc = __builtin_amdgcn_exp2f(m_run - lg);
        l_run *= resc;
#pragma unroll
        for (int e = 0; e < D; ++e) o[e] *= resc;
        m_run = lg;
      }
      const float p = __builtin_amdgcn_exp2f(lg - m_run);
      l_run += p;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] += p * vt[u * D + e];
    }
  }
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
#pragma unroll
  for (int e = 0; e < D; ++e) out[tq * D + e] = o[e] * inv;
  if (lse) lse[tq] = l_run > 0.f ? (m_run + __builtin_log2f(l_run)) * 0.69314718055994531f : -__builtin_inff();
}

template <int D, int BLK>
hipError_t fa_bf16(const Dims& x, const void* q, const void* k, const void* v, const int32_t* kv_idx,
                   const int32_t* kv_cnt, void* out, float* lse, hipStream_t s) {
  using S = FaShape<D, BLK>;
  auto kern = sparse_fa_bf16_kernel<D, BLK>;
  // Thread-safe one-time opt-in to more than 64 KiB of dynamic LDS.
  static const hipError_t attr = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)S::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  const int rows = x.B * x.H * x.nq;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL(kern, dim3(rows), dim3(S::NT), S::LDS_BYTES, s, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), kv_idx, kv_cnt,
                     static_cast<uint16_t*>(out), lse, x.nq, x.nk, x.top_k, scale_log2);
  return hipGetLastError();
}

template <int D, int BLK>
hipError_t fa_f32(const Dims& x, const void* q, const void* k, const void* v, const int32_t* kv_idx,
                  const int32_t* kv_cnt, void* out, float* lse, hipStream_t s) {
  auto kern = sparse_fa_f32_kernel<D, BLK>;
  const size_t lds = 2 * (size_t)BLK * D * sizeof(float);
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  const int rows = x.B * x.H * x.nq;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL(kern, dim3(rows), dim3(BLK), lds, s, static_cast<const float*>(q),
                     static_cast<const float*>(k), static_cast<const float*>(v), kv_idx, kv_cnt,
                     static_cast<float*>(out), lse, x.nq, x.nk, x.top_k, scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn(const velox_problem& p, const void* q, const void* k, const void* v,
                              const int32_t* kv_idx, const int32_t* kv_cnt, void* out, float* lse,
                              hipStream_t s) {
  const Dims x = dims(p);
  const bool bf = p.dtype == VELOX_BF16;
#define VELOX_FA(Dv, Bv)                                                          \
  if (p.head_dim == Dv && p.block == Bv)                                          \
    return bf ? fa_bf16<Dv, Bv>(x, q, k, v, kv_idx, kv_cnt, out, lse, s)          \
              : fa_f32<Dv, Bv>(x, q, k, v, kv_idx, kv_cnt, out, lse, s);
  VELOX_FA(128, 128)
  VELOX_FA(128, 64)
  VELOX_FA(64, 128)
  VELOX_FA(64, 64)
#undef VELOX_FA
  return hipErrorInvalidValue;
}

}  // namespace velox
