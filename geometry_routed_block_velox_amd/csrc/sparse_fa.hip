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
// bf16 kernel (sparse_fa_bf16_kernel): one workgroup per row, 2*blk/32 waves
// (8 at blk = 128, i.e. two waves per SIMD).
//  * Work split: wave w owns 32 queries (query group w % (blk/32)) and one key
//    half (w / (blk/32)) of every tile: 32 queries x 64 keys at blk = 128.
//    Two waves per SIMD let one wave's softmax and LDS waits overlap the
//    other's MFMAs; the price is twice the LDS operand reads per MFMA of a
//    64-query split (measured: the two-wave split is faster).  The two key
//    halves keep independent online softmax states that are merged once at
//    the end of the row.
//  * Scores are formed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: lane l of an accumulator holds query l%32 and
//    keys 8(r/4) + 4(l/32) + r%4, so softmax statistics need one lane
//    exchange (l <-> l^32) and output rescaling is a per-lane scalar.
//  * O^T += V^T P^T takes P from the score registers as the B operand.  The
//    contraction may visit keys in any order as long as both operands agree;
//    the V^T operand is read from the row-major V tile with the LDS
//    transpose read ds_read_b64_tr_b16, whose 16-lane groups return lane i
//    four consecutive rows of column i -- exactly the accumulator's key order.
//  * K and V tiles go from HBM straight to LDS (global_load_lds_dwordx4, no
//    register staging), double-buffered so that the loads of the next listed
//    block overlap the MFMA work on the current one; one barrier per block.
//    16-byte chunks are XOR-swizzled per row so that the MFMA operand reads
//    of K and the transpose reads of V spread over the banks.  K operand
//    fragments are read two MFMA steps ahead of their use.  Every LDS operand
//    address is a per-lane register computed once per workgroup plus an
//    instruction immediate (stage, key tile, 16-key step): the block loop is
//    unrolled over the two stages, so it does no address arithmetic.
//  * exp2 with log2(e)/sqrt(d) folded into one FMA (hardware v_exp_f32).
//    Each wave fixes its softmax reference maximum m_ref per query from the
//    first listed block (the exact maximum over that block, so the largest
//    probability is >= 1 and nothing underflows) and never rescales O inside
//    the loop: later probabilities exp2((s - m_ref) c) may exceed 1, which
//    float32 sums and bf16 P (same exponent range as float32) hold with the
//    same relative precision, and the final normalisation uses the same
//    m_ref, so the result is the same softmax.  If any block's probability
//    sum exceeds 2^40 (logits more than 40 log2-units above the first
//    block's maximum), the workgroup reruns the row: a max-only sweep finds
//    the true maximum, then a second pass uses it (all probabilities <= 1).
//  * Workgroups are remapped so that the rows of one head run on one XCD and
//    share its L2 while they walk their ascending block lists.
// float32 kernel (sparse_fa_f32_kernel): one thread per query token, plain
// float32 VALU arithmetic; used for float32 problems.
#include "velox_internal.h"

namespace velox {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// d-steps by which the K fragment reads run ahead of their score MFMAs.
constexpr int kKAhead = 2;

// Per-block probability sum above which a row is recomputed at its true maximum.
constexpr float kOverflowGuard = 1099511627776.0f;  // 2^40

template <int D, int BLK>
struct Fa {
  static constexpr int QW = 32;                 // queries per wave
  static constexpr int NQG = BLK / QW;          // query groups
  static constexpr int NW = 2 * NQG;            // waves per workgroup: query groups x two key halves
  static constexpr int NT = NW * 64;
  static constexpr int KW = BLK / 2;            // keys per wave and tile
  static constexpr int QT = QW / 32;            // 32-query MFMA tiles per wave
  static constexpr int KTW = KW / 32;           // 32-key MFMA tiles per wave
  static constexpr int DS = D / 16;             // MFMA k-steps over d (scores)
  static constexpr int DT = D / 32;             // 32-row d tiles of O^T
  static constexpr int PS = KW / 16;            // MFMA k-steps over keys (PV)
  static constexpr int NCH = D / 8;             // 16-byte chunks per row
  static constexpr int TILE_CHUNKS = BLK * NCH; // per K (or V) tile
  static constexpr int SEGS_PER_WAVE = TILE_CHUNKS / 64 / NW;  // 1 KiB DMA segments
  static_assert(QT >= 1 && KTW >= 1 && NCH >= 8 && SEGS_PER_WAVE >= 1, "unsupported tile shape");
  static constexpr int T = BLK * D * 2;             // bytes of one K (or V) tile
  static constexpr int V0 = 2 * T, LDS_BYTES = 4 * T;  // K stages at 0 and T, V stages at 2T and 3T
  static __device__ __forceinline__ int swz_k(int row) { return row & (NCH - 1); }
  static __device__ __forceinline__ int swz_v(int row) { return (4 * row) & (NCH - 1); }
};

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

// Issue the HBM -> LDS copies of KV block j (K into st[0, TILE), V into
// st[TILE, 2*TILE)).  Lane l of DMA segment g writes 16-byte slot 64g + l,
// i.e. row (64g + l) / NCH and physical chunk (64g + l) % NCH; it fetches the
// logical chunk stored there under the row's swizzle.  Per-lane byte offsets
// within the block are precomputed once per thread in DmaOffsets.
template <int D, int BLK>
struct DmaOffsets {
  using F = Fa<D, BLK>;
  uint32_t k[F::SEGS_PER_WAVE];
  uint32_t v[F::SEGS_PER_WAVE];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < F::SEGS_PER_WAVE; ++i) {
      const int slot = (wave * F::SEGS_PER_WAVE + i) * 64 + lane;
      const int row = slot / F::NCH, pc = slot % F::NCH;
      k[i] = (uint32_t)(row * D + (pc ^ F::swz_k(row)) * 8) * 2u;
      v[i] = (uint32_t)(row * D + (pc ^ F::swz_v(row)) * 8) * 2u;
    }
  }
};

// One 16-byte-per-lane HBM -> LDS copy (global_load_lds_dwordx4): lane l
// fetches gbase + voff and the data lands at LDS byte lds + 16*l.  Written as
// inline asm so that the compiler's wait-count pass does not treat every
// later LDS read as a possible consumer of the copy; the kernel waits for
// the copies itself (s_waitcnt vmcnt(0)) before the barrier that publishes
// the tile.  The instruction writes no VGPR.
__device__ __forceinline__ void lds_dma16(uint32_t lds, const void* gbase, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds), "v"(voff), "s"(gbase)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

template <int ST, int D, int BLK>
__device__ __forceinline__ void issue_tile(uint32_t lds0, const uint16_t* __restrict__ kh,
                                           const uint16_t* __restrict__ vh, int j, int wave,
                                           const DmaOffsets<D, BLK>& off) {
  using F = Fa<D, BLK>;
  const uint16_t* kb = kh + (size_t)j * BLK * D;
  const uint16_t* vb = vh + (size_t)j * BLK * D;
#pragma unroll
  for (int i = 0; i < F::SEGS_PER_WAVE; ++i) {
    const uint32_t seg = (uint32_t)(wave * F::SEGS_PER_WAVE + i) * 1024u;
    lds_dma16(lds0 + ST * F::T + seg, kb, off.k[i]);
    lds_dma16(lds0 + F::V0 + ST * F::T + seg, vb, off.v[i]);
  }
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;

__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t addr) {
  const u32x4 x = *(const lds_u32x4_t*)(uintptr_t)addr;
  bf16x8 r;
  __builtin_memcpy(&r, &x, 16);
  return r;
}

// Per-wave state of the online softmax over this wave's key half.
template <int D, int BLK>
struct WaveState {
  using F = Fa<D, BLK>;
  bf16x8 qf[F::QT][F::DS];     // Q fragments: B operand of S^T = K Q^T
  f32x16 oacc[F::DT][F::QT];   // O^T accumulators
  float m[F::QT];              // reference maximum (raw logits) of query qc of tile qt
  float l[F::QT];              // this lane's partial sum of probabilities
  bool bad;                    // a probability sum crossed kOverflowGuard
  // Per-lane LDS byte addresses in stage 0; stage, key tile, step and half are immediate offsets.
  uint32_t ko[F::DS];          // K fragment of d-step s, key tile 0
  uint32_t vo[F::DT];          // first V^T transpose read of d tile dt
};

enum class Mode { First, Normal, MaxOnly };

// One tile from the LDS stage st: S^T = K Q^T, then
//   Mode::First   m_ref = maximum of this tile's logits, then as Normal;
//   Mode::Normal  P = exp2((S - m_ref) c), l += rowsum(P), O^T += V^T P^T;
//   Mode::MaxOnly m_ref = max(m_ref, maximum of this tile's logits) only.
template <Mode MODE, int ST, int D, int BLK>
__device__ __forceinline__ void compute_tile(WaveState<D, BLK>& w, float scale_log2) {
  using F = Fa<D, BLK>;
  f32x16 sacc[F::KTW][F::QT];
#pragma unroll
  for (int kt = 0; kt < F::KTW; ++kt)
#pragma unroll
    for (int qt = 0; qt < F::QT; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][qt][r] = 0.f;

  // K fragments are read kKAhead d-steps ahead of their MFMAs; the scheduling
  // fences (which let vector ALU work move across) keep that order, so the
  // LDS latency is covered by the MFMAs in between.
  bf16x8 kf[F::DS][F::KTW];
  auto kread = [&](int s) {
#pragma unroll
    for (int kt = 0; kt < F::KTW; ++kt) kf[s][kt] = lds_read_b128(w.ko[s] + ST * F::T + kt * 32 * F::NCH * 16);
  };
#pragma unroll
  for (int s = 0; s < kKAhead && s < F::DS; ++s) kread(s);
#pragma unroll
  for (int s = 0; s < F::DS; ++s) {
    if (s + kKAhead < F::DS) kread(s + kKAhead);
    __builtin_amdgcn_sched_barrier(0x406);
#pragma unroll
    for (int kt = 0; kt < F::KTW; ++kt)
#pragma unroll
      for (int qt = 0; qt < F::QT; ++qt)
        sacc[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s][kt], w.qf[qt][s], sacc[kt][qt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0x406);
  }

  if constexpr (MODE != Mode::Normal) {
#pragma unroll
    for (int qt = 0; qt < F::QT; ++qt) {
      float mx = sacc[0][qt][0];
#pragma unroll
      for (int kt = 0; kt < F::KTW; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][qt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      w.m[qt] = MODE == Mode::First ? mx : fmaxf(w.m[qt], mx);
    }
  }
  if constexpr (MODE == Mode::MaxOnly) return;

  float mb[F::QT];
#pragma unroll
  for (int qt = 0; qt < F::QT; ++qt) mb[qt] = w.m[qt] * scale_log2;

  // V^T operand for 16-key step ps and d tile dt: two transpose reads of keys
  // kbase + 16ps + 8half + 4hh + 0..3, columns d = 32dt + 16gd + i.  The
  // column swizzle depends only on the lane (key % 4 is fixed per lane).
  float lsum[F::QT];
#pragma unroll
  for (int qt = 0; qt < F::QT; ++qt) lsum[qt] = 0.f;
#pragma unroll
  for (int ps = 0; ps < F::PS; ++ps) {
    // P for these 16 keys: accumulator registers 8(ps%2)..+7 of key tile ps/2.
    bf16x8 pb[F::QT];
#pragma unroll
    for (int qt = 0; qt < F::QT; ++qt) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[ps >> 1][qt][8 * (ps & 1) + i], scale_log2, -mb[qt]));
        lsum[qt] += p;
        pb[qt][i] = (__bf16)p;
      }
    }
#pragma unroll
    for (int dt = 0; dt < F::DT; ++dt) {
      i16x4 part[2];
#pragma unroll
      for (int half = 0; half < 2; ++half)
        part[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(uintptr_t)(w.vo[dt] + ST * F::T + (16 * ps + 8 * half) * F::NCH * 16));
      bf16x8 a;
      __builtin_memcpy(&a, part, 16);
#pragma unroll
      for (int qt = 0; qt < F::QT; ++qt)
        w.oacc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qt], w.oacc[dt][qt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int qt = 0; qt < F::QT; ++qt) {
    w.l[qt] += lsum[qt];
    w.bad |= lsum[qt] > kOverflowGuard;
  }
}

// One pass over the row's block list with the two-stage copy pipeline: the
// copies of the next listed block go into one LDS stage while the MFMA work
// reads the other; one barrier per block.  FIRST_MODE applies to the first
// listed block, MODE to the rest.
template <Mode FIRST_MODE, Mode MODE, int D, int BLK>
__device__ __forceinline__ void run_pass(WaveState<D, BLK>& w, uint32_t lds0, const uint16_t* __restrict__ kh,
                                         const uint16_t* __restrict__ vh,
                                         const __attribute__((address_space(4))) int32_t* list, int cnt, int nk,
                                         int wave, const DmaOffsets<D, BLK>& dma, float scale_log2) {
  auto next_valid = [&](int t) {
    while (t < cnt && (unsigned)list[t] >= (unsigned)nk) ++t;
    return t;
  };
  int t = next_valid(0);
  if (t >= cnt) return;
  issue_tile<0, D, BLK>(lds0, kh, vh, list[t], wave, dma);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // peeled first block (stage 0), then two blocks per turn (stages 1, 0) so
  // that every LDS address is a loop-invariant register plus an immediate
  int tn = next_valid(t + 1);
  if (tn < cnt) issue_tile<1, D, BLK>(lds0, kh, vh, list[tn], wave, dma);
  compute_tile<FIRST_MODE, 0, D, BLK>(w, scale_log2);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  t = tn;
  while (t < cnt) {
    tn = next_valid(t + 1);
    if (tn < cnt) issue_tile<0, D, BLK>(lds0, kh, vh, list[tn], wave, dma);
    compute_tile<MODE, 1, D, BLK>(w, scale_log2);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    t = tn;
    if (t >= cnt) break;
    tn = next_valid(t + 1);
    if (tn < cnt) issue_tile<1, D, BLK>(lds0, kh, vh, list[tn], wave, dma);
    compute_tile<MODE, 0, D, BLK>(w, scale_log2);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    t = tn;
  }
}

// Split-KV: with `splits` > 0 workgroup g handles segment g % splits of row
// g / splits, the list positions [s*cnt/splits, (s+1)*cnt/splits), and
// writes a float32 partial result (normalised output and natural-log LSE of
// its segment) that merge_splits_kernel combines.  splits == 0: the whole
// row, written directly.
struct Segment {
  int row, begin, count, part;
};

__device__ __forceinline__ Segment segment_of(int g, int splits, const int32_t* __restrict__ kv_cnt, int top_k) {
  Segment sg;
  const int parts = splits > 0 ? splits : 1;
  sg.row = g / parts;
  sg.part = g;
  const int cnt = min(max(kv_cnt[sg.row], 0), top_k);
  const int s = g % parts;
  sg.begin = (int)(((long long)s * cnt) / parts);
  sg.count = (int)(((long long)(s + 1) * cnt) / parts) - sg.begin;
  return sg;
}

template <int D, int BLK>
__global__ __launch_bounds__(512) void sparse_fa_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ kv_cnt, uint16_t* __restrict__ out,
    float* __restrict__ lse, int nq, int nk, int top_k, float scale_log2, int splits, float* __restrict__ part_o,
    float* __restrict__ part_lse) {
  using F = Fa<D, BLK>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[F::LDS_BYTES];
  const uint32_t lds0 = lds_addr(lds);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = wave % F::NQG, kg = wave / F::NQG;
  const int qc = lane & 31, hh = lane >> 5;
  const int kbase = kg * F::KW;
  const Segment sg = segment_of(xcd_grouped(blockIdx.x, gridDim.x), splits, kv_cnt, top_k);
  const int row = sg.row;
  const int bh = row / nq, iq = row % nq;
  const size_t N = (size_t)nk * BLK;
  const uint16_t* kh = k + (size_t)bh * N * D;
  const uint16_t* vh = v + (size_t)bh * N * D;
  // The list is read-only here and wave-uniform: scalar loads via the constant address space.
  const __attribute__((address_space(4))) int32_t* list =
      (const __attribute__((address_space(4))) int32_t*)(kv_idx + (size_t)row * top_k + sg.begin);
  const int cnt = sg.count;

  WaveState<D, BLK> w;
  const size_t qrow0 = (size_t)bh * nq * BLK + (size_t)iq * BLK + qg * F::QW;
#pragma unroll
  for (int qt = 0; qt < F::QT; ++qt) {
    const uint4* qrow = reinterpret_cast<const uint4*>(q + (qrow0 + 32 * qt + qc) * D);
#pragma unroll
    for (int s = 0; s < F::DS; ++s) w.qf[qt][s] = as_bf16x8(qrow[2 * s + hh]);
    w.m[qt] = -__builtin_inff();
    w.l[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < F::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.oacc[dt][qt][r] = 0.f;
  }

#pragma unroll
  for (int s = 0; s < F::DS; ++s) {
    const int r = kbase + qc;
    w.ko[s] = lds0 + (uint32_t)(r * F::NCH + ((2 * s + hh) ^ F::swz_k(r))) * 16u;
  }
  {
    const int grp = lane >> 4, j = lane & 15;
    const int gd = grp & 1;
    const int key0 = kbase + 4 * hh + (j >> 2);
    const int vsw = F::swz_v(key0);
#pragma unroll
    for (int dt = 0; dt < F::DT; ++dt) {
      const int c = (4 * dt + 2 * gd + ((j & 3) >> 1)) ^ vsw;
      w.vo[dt] = lds0 + F::V0 + (uint32_t)(key0 * F::NCH * 16 + 8 * (j & 1) + c * 16);
    }
  }
  DmaOffsets<D, BLK> dma;
  dma.init(wave, lane);
  w.bad = false;
  run_pass<Mode::First, Mode::Normal, D, BLK>(w, lds0, kh, vh, list, cnt, nk, wave, dma, scale_log2);
  if (__syncthreads_or(w.bad)) {
    // Rare: some logit exceeded the first block's maximum by more than 40
    // log2-units.  Find each query's true maximum, then redo the row at it.
#pragma unroll
    for (int qt = 0; qt < F::QT; ++qt) {
      w.m[qt] = -__builtin_inff();
      w.l[qt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < F::DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) w.oacc[dt][qt][r] = 0.f;
    }
    run_pass<Mode::MaxOnly, Mode::MaxOnly, D, BLK>(w, lds0, kh, vh, list, cnt, nk, wave, dma, scale_log2);
    run_pass<Mode::Normal, Mode::Normal, D, BLK>(w, lds0, kh, vh, list, cnt, nk, wave, dma, scale_log2);
  }

  // Merge the two key halves: waves with kg = 1 hand (m, l, O) to kg = 0 through LDS.
  float* xo = reinterpret_cast<float*>(lds);           // [qg][dt][qt][r][lane]: blk*d floats = both K stages
  float* xm = reinterpret_cast<float*>(lds + F::V0);  // m: [qg][qt][lane], then l: [qg][qt][lane]
  float lw[F::QT];
#pragma unroll
  for (int qt = 0; qt < F::QT; ++qt) lw[qt] = w.l[qt] + __shfl_xor(w.l[qt], 32);
  if (kg == 1) {
#pragma unroll
    for (int qt = 0; qt < F::QT; ++qt) {
      xm[(qg * F::QT + qt) * 64 + lane] = w.m[qt];
      xm[((F::NQG + qg) * F::QT + qt) * 64 + lane] = lw[qt];
#pragma unroll
      for (int dt = 0; dt < F::DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(((qg * F::DT + dt) * F::QT + qt) * 16 + r) * 64 + lane] = w.oacc[dt][qt][r];
    }
  }
  __syncthreads();
  if (kg == 0) {
#pragma unroll
    for (int qt = 0; qt < F::QT; ++qt) {
      const float m1 = xm[(qg * F::QT + qt) * 64 + lane];
      const float l1 = xm[((F::NQG + qg) * F::QT + qt) * 64 + lane];
      const float m0 = w.m[qt];
      const float mm = fmaxf(m0, m1);
      const float a0 = m0 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((m0 - mm) * scale_log2);
      const float a1 = m1 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((m1 - mm) * scale_log2);
      const float lt = lw[qt] * a0 + l1 * a1;
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
      const size_t tq = qrow0 + 32 * qt + qc;
      // split mode: float32 partial result of this segment, token t of the block
      const size_t pt = ((size_t)sg.part * BLK + qg * F::QW + 32 * qt + qc);
      uint16_t* orow = out + tq * D;
      float* prow = part_o + pt * D;
#pragma unroll
      for (int dt = 0; dt < F::DT; ++dt) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rq + e;
            const float o1 = xo[(((qg * F::DT + dt) * F::QT + qt) * 16 + r) * 64 + lane];
            o[e] = (w.oacc[dt][qt][r] * a0 + o1 * a1) * inv;
          }
          if (splits) {
            *reinterpret_cast<float4*>(prow + 32 * dt + 8 * rq + 4 * hh) = make_float4(o[0], o[1], o[2], o[3]);
          } else {
            uint2 pk;
            pk.x = pack_bf16x2(o[0], o[1]);
            pk.y = pack_bf16x2(o[2], o[3]);
            *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * rq + 4 * hh) = pk;
          }
        }
      }
      const float row_lse =
          lt > 0.f ? (mm * scale_log2 + __builtin_log2f(lt)) * 0.69314718055994531f : -__builtin_inff();
      if (hh == 0) {
        if (splits)
          part_lse[pt] = row_lse;
        else if (lse)
          lse[tq] = row_lse;
      }
    }
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
                                                            int nq, int nk, int top_k, float scale_log2, int splits,
                                                            float* __restrict__ part_o,
                                                            float* __restrict__ part_lse) {
  extern __shared__ float fs[];
  float* kt = fs;
  float* vt = fs + BLK * D;
  const int tid = threadIdx.x;
  const Segment sg = segment_of(blockIdx.x, splits, kv_cnt, top_k);
  const int row = sg.row;
  const int bh = row / nq, iq = row % nq;
  const size_t N = (size_t)nk * BLK;
  const float* kh = k + (size_t)bh * N * D;
  const float* vh = v + (size_t)bh * N * D;
  const int32_t* list = kv_idx + (size_t)row * top_k + sg.begin;
  const int cnt = sg.count;
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
  const float row_lse = l_run > 0.f ? (m_run + __builtin_log2f(l_run)) * 0.69314718055994531f : -__builtin_inff();
  float* orow = splits ? part_o + ((size_t)sg.part * BLK + tid) * D : out + tq * D;
#pragma unroll
  for (int e = 0; e < D; ++e) orow[e] = o[e] * inv;
  if (splits)
    part_lse[(size_t)sg.part * BLK + tid] = row_lse;
  else if (lse)
    lse[tq] = row_lse;
}

// Combine the segments of every row: with L_s the segment LSEs and O_s their
// normalised outputs, LSE = log sum_s exp(L_s) and O = sum_s exp(L_s - LSE) O_s
// (segments without a valid block have L_s = -inf and weight 0).  One thread
// per output token and 4 consecutive d; grid = ceil(rows * BLK * D / 4 / 256).
template <int D, int BLK, bool OUT_BF16>
__global__ __launch_bounds__(256) void merge_splits_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_lse, int splits,
                                                           long long n_vec, void* __restrict__ out,
                                                           float* __restrict__ lse) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= n_vec) return;
  const long long tok = e / (D / 4);  // = row * BLK + t, also the output token index
  const int d = (int)(e % (D / 4)) * 4;
  const long long row = tok / BLK;
  const int t = (int)(tok % BLK);
  const float* pl = part_lse + row * splits * BLK + t;
  float mx = -__builtin_inff();
#pragma unroll 8
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, pl[(size_t)s * BLK]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  if (mx > -__builtin_inff()) {
    const float* po = part_o + (row * splits * BLK + t) * D + d;
#pragma unroll 8
    for (int s = 0; s < splits; ++s) {
      const float ls = pl[(size_t)s * BLK];
      if (ls == -__builtin_inff()) continue;
      const float w = __builtin_amdgcn_exp2f((ls - mx) * 1.4426950408889634f);
      const float4 o = *reinterpret_cast<const float4*>(po + (size_t)s * BLK * D);
      wsum += w;
      acc.x += w * o.x;
      acc.y += w * o.y;
      acc.z += w * o.z;
      acc.w += w * o.w;
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  const float4 o = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (OUT_BF16) {
    uint2 pk;
    pk.x = pack_bf16x2(o.x, o.y);
    pk.y = pack_bf16x2(o.z, o.w);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + tok * D + d) = pk;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + tok * D + d) = o;
  }
  if (lse && d == 0) lse[tok] = wsum > 0.f ? mx + __builtin_logf(wsum) : -__builtin_inff();
}

// Launchers: splits == 0 writes out/lse directly; otherwise partial results go
// to part_o/part_lse and merge_splits_kernel writes out/lse.
template <int D, int BLK>
hipError_t fa_bf16(const Dims& x, const void* q, const void* k, const void* v, const int32_t* kv_idx,
                   const int32_t* kv_cnt, void* out, float* lse, int splits, float* part_o, float* part_lse,
                   hipStream_t s) {
  const int rows = x.B * x.H * x.nq;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL((sparse_fa_bf16_kernel<D, BLK>), dim3(rows * (splits > 0 ? splits : 1)), dim3(Fa<D, BLK>::NT),
                     0, s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), kv_idx, kv_cnt, static_cast<uint16_t*>(out), lse, x.nq, x.nk,
                     x.top_k, scale_log2, splits, part_o, part_lse);
  return hipGetLastError();
}

template <int D, int BLK, bool OUT_BF16>
hipError_t merge(const Dims& x, int splits, const float* part_o, const float* part_lse, void* out, float* lse,
                 hipStream_t s) {
  const long long n = (long long)x.B * x.H * x.nq * BLK * (D / 4);
  hipLaunchKernelGGL((merge_splits_kernel<D, BLK, OUT_BF16>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     part_o, part_lse, splits, n, out, lse);
  return hipGetLastError();
}

template <int D, int BLK>
hipError_t fa_f32(const Dims& x, const void* q, const void* k, const void* v, const int32_t* kv_idx,
                  const int32_t* kv_cnt, void* out, float* lse, int splits, float* part_o, float* part_lse,
                  hipStream_t s) {
  auto kern = sparse_fa_f32_kernel<D, BLK>;
  const size_t lds = 2 * (size_t)BLK * D * sizeof(float);
  // Thread-safe one-time opt-in to more than 64 KiB of dynamic LDS.
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  const int rows = x.B * x.H * x.nq;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL(kern, dim3(rows * (splits > 0 ? splits : 1)), dim3(BLK), lds, s, static_cast<const float*>(q),
                     static_cast<const float*>(k), static_cast<const float*>(v), kv_idx, kv_cnt,
                     static_cast<float*>(out), lse, x.nq, x.nk, x.top_k, scale_log2, splits, part_o, part_lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn(const velox_problem& p, const void* q, const void* k, const void* v,
                              const int32_t* kv_idx, const int32_t* kv_cnt, void* out, float* lse, int splits,
                              float* part_o, float* part_lse, hipStream_t s) {
  const Dims x = dims(p);
  const bool bf = p.dtype == VELOX_BF16;
#define VELOX_FA(Dv, Bv)                                                                                       \
  if (p.head_dim == Dv && p.block == Bv) {                                                                     \
    hipError_t e = bf ? fa_bf16<Dv, Bv>(x, q, k, v, kv_idx, kv_cnt, out, lse, splits, part_o, part_lse, s)      \
                      : fa_f32<Dv, Bv>(x, q, k, v, kv_idx, kv_cnt, out, lse, splits, part_o, part_lse, s);      \
    if (e == hipSuccess && splits > 0)                                                                         \
      e = bf ? merge<Dv, Bv, true>(x, splits, part_o, part_lse, out, lse, s)                                   \
             : merge<Dv, Bv, false>(x, splits, part_o, part_lse, out, lse, s);                                 \
    return e;                                                                                                  \
  }
  VELOX_FA(128, 128)
  VELOX_FA(128, 64)
  VELOX_FA(64, 128)
  VELOX_FA(64, 64)
#undef VELOX_FA
  return hipErrorInvalidValue;
}

}  // namespace velox
