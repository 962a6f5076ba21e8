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
// bf16 kernel (sparse_fa_bf16_kernel): one workgroup per row, one wave per
// SIMD (4 waves at blk = 128), each wave holding up to 512 registers.
//  * Work split: wave w owns 64 queries (query group w % (blk/64), two
//    32-query MFMA tiles) and one key half (w / (blk/64)) of every tile:
//    64 queries x 64 keys at blk = 128.  Every K or V operand read from LDS
//    feeds both query tiles, so a tile costs 128 KiB of LDS operand reads
//    (K and V halves read once per query group).  The two key halves keep
//    independent online softmax states that are merged once at the end of
//    the row.
//  * Software pipeline inside each wave: iteration t computes the scores of
//    listed block t+1 on the matrix cores, S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16, while the vector ALU turns the scores of block
//    t into probabilities; then O^T += V^T P^T for block t.  The softmax of a
//    block thus overlaps the score MFMAs of the next one without a second
//    wave on the SIMD.  Lane l of a score accumulator holds query l%32 and
//    keys 8(r/4) + 4(l/32) + r%4, so softmax statistics need one lane
//    exchange (l <-> l^32) and output rescaling is a per-lane scalar.
//  * O^T += V^T P^T takes P from registers as the B operand.  The contraction
//    may visit keys in any order as long as both operands agree; the V^T
//    operand is read from the row-major V tile with the LDS transpose read
//    ds_read_b64_tr_b16, whose 16-lane groups return lane i four consecutive
//    rows of column i -- exactly the accumulator's key order.
//  * The row's Q fragments (the B operand of the score MFMAs) are loaded once
//    into AGPRs beside the O^T accumulators, so the block loop reads only K
//    and V from LDS.
//  * K and V tiles go from HBM straight to LDS (buffer_load_dwordx4 ... lds
//    through the compiler's builtin, no register staging) into two K and two
//    V slots, separate LDS arrays so that the compiler's wait counting knows
//    a copy into one slot does not feed reads of another.  Iteration t copies K of block t+2 and V of block
//    t+1 while it reads K of block t+1 and V of block t: one barrier per
//    block, and a copy has a whole iteration to land.  16-byte chunks are
//    XOR-swizzled per row so that the MFMA operand reads of K and the
//    transpose reads of V spread over the banks.
//  * Softmax without rescaling O: the probabilities of a row share one fixed
//    reference, so O and the probability sums just accumulate, and the final
//    normalisation divides by a sum taken with the same reference, which
//    gives the same softmax.  Probabilities above 1 are fine (float32 sums
//    and bf16 P have float32's exponent range and keep their relative
//    precision).  The probability sums add the bf16-rounded P that the PV
//    product uses (v_dot2_f32_bf16 against ones), so numerator and
//    denominator carry the same weights.  Two passes (attend_row):
//    - fast pass, tried first: the row's Q is multiplied by log2(e)/sqrt(d)
//      once, in bf16, so a score is already a base-2 exponent, and the
//      probability is exp2(s) itself (hardware v_exp_f32, no reference
//      subtracted, one vector operation per score less than the general
//      pass).  The pass is taken only while that cannot overflow or
//      underflow: every query's maximum over the first listed block within
//      +-40 and every block's probability sum below 2^56; otherwise the
//      workgroup drops it and runs the general pass.  Rounding the scaled Q
//      to bf16 perturbs a score by at most 2^-9 c sum_d |q_d k_d| (c the
//      scale), which moves the row's LSE by at most that much too.
//    - general pass (a function of its own, so that its registers do not
//      constrain the fast one): unscaled Q, exp2 with the scale folded into
//      one FMA, and each wave's reference maximum m_ref per query taken
//      from the first listed block (the exact maximum over that block, so
//      the largest probability is >= 1 and nothing underflows).  If any
//      block's probability sum exceeds 2^40 (logits more than 40 log2-units
//      above the first block's maximum), the workgroup reruns the row: a
//      max-only sweep finds the true maximum, then a second pass uses it
//      (all P <= 1).
//  * The block list is read through a 64-entry window in one VGPR (v_readlane
//    with a wave-uniform mask of valid entries), so no scalar memory load is
//    outstanding in the loop to force every LDS wait to drain completely.
//  * Workgroups are remapped so that the rows of one head run on one XCD and
//    share its L2 while they walk their ascending block lists.
// float32 kernel (sparse_fa_f32_kernel): one thread per query token, plain
// float32 VALU arithmetic; used for float32 problems.
#include "velox_internal.h"

namespace velox {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;

// d-steps by which the K fragment reads run ahead of their score MFMAs.
constexpr int kKAhead = 2;
// PV steps by which the V^T fragment reads run ahead of their MFMAs.
constexpr int kVAhead = 6;

// Per-block probability sum above which a row is recomputed at its true maximum.
constexpr float kOverflowGuard = 1099511627776.0f;  // 2^40
// Fast pass: every query's maximum over the first listed block must lie in
// [-kFastRange, kFastRange] (log2 units) and every block's probability sum
// below kFastGuard; otherwise the row is redone by the general pass.
constexpr float kFastRange = 40.0f;
constexpr float kFastGuard = 72057594037927936.0f;  // 2^56

template <int D, int BLK>
struct Fa {
  static constexpr int QT = 2;                  // 32-query MFMA tiles per wave
  static constexpr int QW = 32 * QT;            // queries per wave
  static constexpr int NQG = BLK / QW;          // query groups
  static constexpr int KW = BLK / 2;            // keys per wave and tile (two key halves)
  static constexpr int KTW = KW / 32;           // 32-key MFMA tiles per wave
  static constexpr int NW = 2 * NQG;            // waves per workgroup
  static constexpr int NT = NW * 64;            // = 2 * BLK
  static constexpr int DS = D / 16;             // MFMA k-steps over d (scores)
  static constexpr int DT = D / 32;             // 32-row d tiles of O^T
  static constexpr int PS = KW / 16;            // MFMA k-steps over keys (PV)
  static constexpr int NCH = D / 8;             // 16-byte chunks per row
  static constexpr int TILE_CHUNKS = BLK * NCH; // per K (or V) tile
  static constexpr int SEGS = TILE_CHUNKS / 64 / NW;  // 1 KiB copies per wave and tile (K or V)
  static constexpr int T = BLK * D * 2;         // bytes of one K (or V) tile
  static_assert(NQG >= 1 && KTW >= 1 && NCH >= 8 && SEGS >= 1, "unsupported tile shape");
  static __device__ __forceinline__ int swz_k(int row) { return row & (NCH - 1); }
  static __device__ __forceinline__ int swz_v(int row) { return (4 * row) & (NCH - 1); }
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  uint16_t ua, ub;
  __builtin_memcpy(&ua, &a, 2);
  __builtin_memcpy(&ub, &b, 2);
  return (uint32_t)ua | ((uint32_t)ub << 16);
}

// HBM -> LDS copies of KV blocks (buffer_load_dwordx4 ... lds: 16 bytes per
// lane, copy g of a tile landing at LDS tile + 1 KiB * g + 16 * lane).  Lane
// l of copy g writes LDS slot 64g + l, i.e. row slot / NCH and physical
// chunk slot % NCH, and fetches the logical chunk stored there under the
// row's swizzle: byte g * 1 KiB + sw(l, g) of the block, where sw depends on
// g only through g mod P (the swizzle repeats every NCH rows for K and every
// NCH/4 rows for V), so a lane keeps P offsets per tensor.  The buffer
// resource spans one head of K (or V); a block is addressed by its scalar
// byte offset, and offsets past the end read zeros.
template <int D, int BLK>
struct Copier {
  using F = Fa<D, BLK>;
  static constexpr int PK = F::NCH * F::NCH / 64 > 1 ? F::NCH * F::NCH / 64 : 1;
  static constexpr int PV = F::NCH * F::NCH / 256 > 1 ? F::NCH * F::NCH / 256 : 1;
  static_assert(F::SEGS % PK == 0 && F::SEGS % PV == 0, "copy period must divide the copies per wave");
  __amdgpu_buffer_rsrc_t krs, vrs;
  uint32_t ko[PK], vo[PV];
  int wave;

  static __device__ __forceinline__ uint32_t sw(int lane, int g, bool is_v) {
    const int slot = g * 64 + lane;
    const int row = slot / F::NCH, pc = slot % F::NCH;
    const int c = pc ^ (is_v ? F::swz_v(row) : F::swz_k(row));
    return (uint32_t)(((row - g * 64 / F::NCH) * D + c * 8) * 2);
  }
  __device__ __forceinline__ void init(const uint16_t* kh, const uint16_t* vh, uint32_t head_bytes, int w, int lane) {
    wave = w;
    krs = __builtin_amdgcn_make_buffer_rsrc((void*)kh, (short)0, (int)head_bytes, 0x00020000);
    vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vh, (short)0, (int)head_bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < PK; ++i) ko[i] = (uint32_t)i * 1024u + sw(lane, i, false);
#pragma unroll
    for (int i = 0; i < PV; ++i) vo[i] = (uint32_t)i * 1024u + sw(lane, i, true);
  }
};

// Copy i (0 <= i < SEGS) of this wave's share of block j's tile of tensor
// WHAT (0 = K, 1 = V) into dst:
// global byte j*T + g*1024 + sw(lane, g) = soff + (i % P)*1024 + sw(lane, i % P)
// with g = wave*SEGS + i.
template <int WHAT, int D, int BLK>
__device__ __forceinline__ void copy_one(const Copier<D, BLK>& cp, unsigned char* dst, int j, int i) {
  // The builtin exists only in the device compilation; the host pass of this
  // HIP source never runs the kernel.
#if defined(__HIP_DEVICE_COMPILE__)
  using F = Fa<D, BLK>;
  const int g = cp.wave * F::SEGS + i;
  constexpr int P = WHAT == 1 ? Copier<D, BLK>::PV : Copier<D, BLK>::PK;
  const uint32_t soff = (uint32_t)j * (uint32_t)F::T + (uint32_t)(g - i % P) * 1024u;
  if constexpr (WHAT == 1)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(cp.vrs, (lds_void_t*)(dst + g * 1024), 16, cp.vo[i % P], soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(cp.krs, (lds_void_t*)(dst + g * 1024), 16, cp.ko[i % P], soff, 0, 0);
#endif
}

template <int WHAT, int D, int BLK>
__device__ __forceinline__ void copy_tile(const Copier<D, BLK>& cp, unsigned char* dst, int j) {
#pragma unroll
  for (int i = 0; i < Fa<D, BLK>::SEGS; ++i) copy_one<WHAT, D, BLK>(cp, dst, j, i);
}

// The four LDS slots of a workgroup: K and V of two blocks in flight.
struct Slots {
  unsigned char* k[2];
  unsigned char* v[2];
};

__device__ __forceinline__ bf16x8 lds_read_b128(const unsigned char* p) {
  const u32x4 x = *(const lds_u32x4_t*)p;
  bf16x8 r;
  __builtin_memcpy(&r, &x, 16);
  return r;
}

// Matrix-core products, written as inline assembly so that the register
// files are fixed: score accumulators in VGPRs (the softmax reads them), the
// Q fragments and the O accumulators in AGPRs.  The hazards the compiler
// would otherwise handle are handled here:
//  * a VALU write of a VGPR needs 2 wait states before an MFMA reads it: the
//    PV product (B operand = probabilities just converted by the VALU) starts
//    with s_nop 1;
//  * an MFMA result needs up to 18 wait states before a VALU or an AGPR read
//    uses it: fence_vgpr / fence_agpr wait that long and take the results as
//    asm operands, so that the compiler cannot schedule a read above the wait
//    (a plain asm with a memory clobber does not order register reads); in
//    the pipelined loop the scores of a block are read one iteration later,
//    after the PV MFMAs and a barrier, behind a fence that only orders;
//  * back-to-back accumulation into the same registers is interlocked by the
//    hardware, and every chain here interleaves at least three independent
//    accumulators anyway;
//  * the A and B operands are read when the MFMA issues, so their registers
//    may be refilled right after it; a result that does not accumulate is
//    early-clobber so that it never overlaps an operand.
__device__ __forceinline__ void mfma_score_first(f32x16& acc, const bf16x8& kfrag, const bf16x8& qfrag) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(kfrag), "a"(qfrag));
}
__device__ __forceinline__ void mfma_score(f32x16& acc, const bf16x8& kfrag, const bf16x8& qfrag) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(kfrag), "a"(qfrag));
}
__device__ __forceinline__ void mfma_pv(f32x16& acc, const bf16x8& vfrag, const bf16x8& pfrag) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(vfrag), "v"(pfrag));
}
// Wait (WAIT = true: 18 wait states) for the MFMAs that last wrote `acc`,
// as an asm that takes the accumulators as operands, so that no later read
// of them can be scheduled above it.  With WAIT = false it only orders the
// reads after this point (for results known to be complete).
template <bool WAIT, int N0, int N1>
__device__ __forceinline__ void fence_vgpr(f32x16 (&acc)[N0][N1]) {
  if (WAIT)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(acc[0][0])::"memory");
  else
    asm volatile("" : "+v"(acc[0][0])::"memory");
#pragma unroll
  for (int a = 0; a < N0; ++a)
#pragma unroll
    for (int b = 0; b < N1; ++b)
      if (a || b) asm volatile("" : "+v"(acc[a][b]));
}
template <int N0, int N1>
__device__ __forceinline__ void fence_agpr(f32x16 (&acc)[N0][N1]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+a"(acc[0][0])::"memory");
#pragma unroll
  for (int a = 0; a < N0; ++a)
#pragma unroll
    for (int b = 0; b < N1; ++b)
      if (a || b) asm volatile("" : "+a"(acc[a][b]));
}

// Per-wave state of the online softmax over this wave's key half.
template <int D, int BLK>
struct WaveState {
  using F = Fa<D, BLK>;
  bf16x8 qf[F::QT][F::DS];     // Q fragments (AGPRs): B operand of S^T = K Q^T
  f32x16 oacc[F::DT][F::QT];   // O^T accumulators (AGPRs)
  float m[F::QT];              // reference maximum (raw logits) of query qc of tile qt
  float l[F::QT];              // this lane's partial sum of probabilities
  bool bad;                    // a probability sum crossed kOverflowGuard
  // Per-lane LDS byte offsets within a tile; key tile, step and half are immediate offsets.
  uint32_t ko[F::DS];          // K fragment of d-step s, key tile 0
  uint32_t vo[F::DT];          // first V^T transpose read of d tile dt
};

template <int D, int BLK>
__device__ __forceinline__ bf16x8 k_fragment(const WaveState<D, BLK>& w, const unsigned char* kt_base, int s, int kt) {
  using F = Fa<D, BLK>;
  return lds_read_b128(kt_base + w.ko[s] + kt * 32 * F::NCH * 16);
}

// V^T operand for 16-key step ps and d tile dt: two transpose reads of keys
// kbase + 16ps + 8half + 4hh + 0..3, columns d = 32dt + 16gd + i.
template <int D, int BLK>
__device__ __forceinline__ bf16x8 v_fragment(const WaveState<D, BLK>& w, const unsigned char* vt_base, int ps, int dt) {
  using F = Fa<D, BLK>;
  i16x4 part[2];
#pragma unroll
  for (int half = 0; half < 2; ++half)
    part[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t*)(vt_base + w.vo[dt] + (16 * ps + 8 * half) * F::NCH * 16));
  bf16x8 a;
  __builtin_memcpy(&a, part, 16);
  return a;
}

// S^T = K Q^T for the KV tile in LDS at kt_base (this wave's key half), into
// sacc, with nothing else interleaved (prologue and rare paths).
template <int D, int BLK>
__device__ __forceinline__ void scores(const WaveState<D, BLK>& w, const unsigned char* kt_base,
                                       f32x16 (&sacc)[Fa<D, BLK>::KTW][Fa<D, BLK>::QT]) {
  using F = Fa<D, BLK>;
#pragma unroll
  for (int s = 0; s < F::DS; ++s) {
    bf16x8 kf[F::KTW];
#pragma unroll
    for (int kt = 0; kt < F::KTW; ++kt) kf[kt] = k_fragment<D, BLK>(w, kt_base, s, kt);
#pragma unroll
    for (int kt = 0; kt < F::KTW; ++kt)
#pragma unroll
      for (int qt = 0; qt < F::QT; ++qt) {
        if (s == 0)
          mfma_score_first(sacc[kt][qt], kf[kt], w.qf[qt][s]);
        else
          mfma_score(sacc[kt][qt], kf[kt], w.qf[qt][s]);
      }
  }
  fence_vgpr<true>(sacc);
}

// Per-query maximum of a score tile, over both lane halves.
template <int D, int BLK>
__device__ __forceinline__ void tile_max(const f32x16 (&sacc)[Fa<D, BLK>::KTW][Fa<D, BLK>::QT], float (&mx)[Fa<D, BLK>::QT]) {
  using F = Fa<D, BLK>;
#pragma unroll
  for (int qt = 0; qt < F::QT; ++qt) {
    float v = sacc[0][qt][0];
#pragma unroll
    for (int kt = 0; kt < F::KTW; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) v = fmaxf(v, sacc[kt][qt][r]);
    mx[qt] = fmaxf(v, __shfl_xor(v, 32));
  }
}

// Softmax element e of a score tile: query tile qt, 16-key step ps, register
// i of that step, e = (qt * PS + ps) * 8 + i.  pb[ps][qt] holds keys 16ps.. of
// the tile, i.e. accumulator registers 8(ps%2).. of key tile ps/2.
template <int D, int BLK, bool FAST>
struct Softmax {
  using F = Fa<D, BLK>;
  static constexpr int NE = F::QT * F::PS * 8;
  const f32x16 (&sacc)[F::KTW][F::QT];
  bf16x8 (&pb)[F::PS][F::QT];
  float mb[F::QT];
  float scale_log2;
  float p_even;  // probability of the last even element, packed with the next one
  __device__ __forceinline__ void element(int e) {
    const int i = e & 7, ps = (e >> 3) % F::PS, qt = (e >> 3) / F::PS;
    const float x = sacc[ps >> 1][qt][8 * (ps & 1) + i];
    const float p = __builtin_amdgcn_exp2f(FAST ? x : __builtin_fmaf(x, scale_log2, -mb[qt]));
    if ((i & 1) == 0) {
      p_even = p;
    } else {
      pb[ps][qt][i - 1] = (__bf16)p_even;
      pb[ps][qt][i] = (__bf16)p;
    }
  }
};

// Row sums of the bf16 probabilities of 16-key step ps (the weights the PV product uses).
template <int D, int BLK>
__device__ __forceinline__ void row_sums(const bf16x8 (&pb)[Fa<D, BLK>::PS][Fa<D, BLK>::QT], int ps,
                                         float (&lsum)[Fa<D, BLK>::QT]) {
  using F = Fa<D, BLK>;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int qt = 0; qt < F::QT; ++qt)
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const bf16x2 two = {pb[ps][qt][i], pb[ps][qt][i + 1]};
      lsum[qt] = __builtin_amdgcn_fdot2_f32_bf16(two, ones, lsum[qt], false);
    }
}

// The row's list, consumed in order, valid entries only (ids in [0, nk);
// anything else is skipped).  Entries come through a 64-entry window in one
// VGPR (lane i: entry base + i) with a wave-uniform mask of its valid lanes;
// an id is taken with v_readlane.  The next window is loaded one window
// ahead with a vector load, so no scalar memory load is outstanding in the
// block loop (it would force every LDS wait to drain completely).
struct ListStream {
  const int32_t* list;
  int cnt, nk;
  int cap;        // entries that may be read; cnt <= cap, and cap does not depend on the loaded count
  int base;       // list position of the window's first entry
  int win, ahead; // this window's entries and the next window's (per lane)
  uint64_t mask;  // valid lanes of this window not handed out yet
  static constexpr int PW = 4;  // windows loaded by prefetch (256 entries)
  int raw[PW];    // those windows as loaded (entries at or past cnt not yet dropped)

  __device__ __forceinline__ int load(int b, int lane) const {
    return b + lane < cnt ? list[b + lane] : -1;
  }
  // Issues the loads of the first PW windows: unconditional, straight-line
  // and independent of cnt (positions past cap read entry cap - 1; start()
  // drops everything at or past cnt <= cap), so that they go out together
  // with the loads of the count and of Q and are waited for once, in start().
  __device__ __forceinline__ void prefetch(int lane) {
    const int last = cap > 0 ? cap - 1 : 0;
#pragma unroll
    for (int i = 0; i < PW; ++i) raw[i] = list[min(64 * i + lane, last)];
  }
  // Starts the stream at the first window (after prefetch); returns the
  // number of valid entries in the whole list.
  __device__ __forceinline__ int start(int lane) {
    base = 0;
    win = lane < cnt ? raw[0] : -1;
    ahead = 64 + lane < cnt ? raw[1] : -1;
    mask = __builtin_amdgcn_ballot_w64((unsigned)win < (unsigned)nk);
    int c = 0;
#pragma unroll
    for (int i = 0; i < PW; ++i) c += (int)(64 * i + lane < cnt) & (int)((unsigned)raw[i] < (unsigned)nk);
    for (int t = 64 * PW + lane; t < cnt; t += 64) c += (unsigned)list[t] < (unsigned)nk;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
    return __builtin_amdgcn_readfirstlane(c);
  }
  // The next valid id, or -1 past the end.
  __device__ __forceinline__ int take(int lane) {
    while (mask == 0) {
      if (base + 64 >= cnt) return -1;
      base += 64;
      win = ahead;
      ahead = load(base + 64, lane);
      mask = __builtin_amdgcn_ballot_w64((unsigned)win < (unsigned)nk);
    }
    const int i = __builtin_ctzll(mask);
    mask &= mask - 1;
    return __builtin_amdgcn_readlane(win, i);
  }
};

// One software-pipelined pass over the row's listed blocks.  With FIRST the
// reference maximum comes from the first listed block; otherwise w.m is
// given.  Iteration t (block t of the valid entries, slots by parity):
//   copies  K(t+2) -> K slot t%2, V(t+1) -> V slot (t+1)%2
//   scores  S(t+1) from K slot (t+1)%2        (matrix cores)
//   softmax P(t) from S(t)                   (vector ALU, overlapping)
//   PV      O += V(t)^T P(t) from V slot t%2
//   wait for the copies, barrier.
template <int D, int BLK, bool FAST>
struct Pass {
  using F = Fa<D, BLK>;
  WaveState<D, BLK>& w;
  const Slots& sl;
  ListStream& ls;
  const Copier<D, BLK>& cp;
  float scale_log2;

  int fallback;  // a valid block id, copied for the phantom step past the end of the list

  // O += V^T P^T for the V tile in LDS at vb and the row sums of P after
  // each 16-key step.  V^T fragments are read kVAhead steps ahead through a
  // ring; the caller may have issued the first kVAhead reads (vf) already.
  static constexpr int NV = F::PS * F::DT;  // PV steps per block
  __device__ __forceinline__ void pv_prefetch(bf16x8 (&vf)[kVAhead + 1], const unsigned char* vb) {
#pragma unroll
    for (int n = 0; n < kVAhead && n < NV; ++n) vf[n] = v_fragment<D, BLK>(w, vb, n / F::DT, n % F::DT);
  }
  __device__ __forceinline__ void pv(const bf16x8 (&pb)[F::PS][F::QT], const unsigned char* vb,
                                     bf16x8 (&vf)[kVAhead + 1]) {
    float lsum[F::QT];
#pragma unroll
    for (int qt = 0; qt < F::QT; ++qt) lsum[qt] = 0.f;
#pragma unroll
    for (int ps = 0; ps < F::PS; ++ps) {
#pragma unroll
      for (int dt = 0; dt < F::DT; ++dt) {
        const int n = ps * F::DT + dt, na = n + kVAhead;
        if (na < NV) vf[na % (kVAhead + 1)] = v_fragment<D, BLK>(w, vb, na / F::DT, na % F::DT);
#pragma unroll
        for (int qt = 0; qt < F::QT; ++qt) mfma_pv(w.oacc[dt][qt], vf[n % (kVAhead + 1)], pb[ps][qt]);
        if (dt == 0) row_sums<D, BLK>(pb, ps, lsum);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int qt = 0; qt < F::QT; ++qt) {
      w.l[qt] += lsum[qt];
      w.bad |= lsum[qt] > (FAST ? kFastGuard : kOverflowGuard);
    }
  }

  // One block that has a successor.  ST: parity of t; jv: block id of t+1
  // (its V is copied now), jk: block id of t+2 (its K is copied now; past
  // the end of the list a valid block whose scores are never used).
  // Issue order (the sched_barrier fences keep it): each score MFMA of block
  // t+1 is followed by its share of the softmax of block t (NE / NS
  // elements), every d-step by the K fragment reads kKAhead steps
  // ahead, and its share of the 2 * SEGS copies (K first: it is needed
  // first); the last slots also start the V^T reads of the PV product; then
  // the PV MFMAs of block t with their V^T reads and the row sums.
  template <int ST>
  __device__ __forceinline__ void iter(f32x16 (&scur)[F::KTW][F::QT], f32x16 (&snext)[F::KTW][F::QT], int jv,
                                       int jk) {
    constexpr int NS = F::DS * F::KTW * F::QT;  // score MFMAs per block
    constexpr int NE = Softmax<D, BLK, FAST>::NE;  // softmax elements per lane and block
    static_assert(NE % NS == 0 && (NE / NS) % 2 == 0, "softmax share per slot must be whole pairs");
    constexpr int EPS = NE / NS;
    constexpr int NC = 2 * F::SEGS;             // copies per wave and block
    bf16x8 pb[F::PS][F::QT];
    Softmax<D, BLK, FAST> sm = {scur, pb, {}, scale_log2, 0.f};
#pragma unroll
    for (int qt = 0; qt < F::QT; ++qt) sm.mb[qt] = w.m[qt] * scale_log2;
    const unsigned char* kb = sl.k[ST ^ 1];
    // score MFMAs d-step major, m = (s * KTW + kt) * QT + qt: the K
    // fragments of step s feed QT MFMAs each
    bf16x8 kf[F::DS][F::KTW], vf[kVAhead + 1];
    auto read_step = [&](int st) {
#pragma unroll
      for (int kt = 0; kt < F::KTW; ++kt) kf[st][kt] = k_fragment<D, BLK>(w, kb, st, kt);
    };
#pragma unroll
    for (int st = 0; st < kKAhead && st < F::DS; ++st) read_step(st);
#pragma unroll
    for (int m = 0; m < NS; ++m) {
      const int s = m / (F::KTW * F::QT), kt = (m / F::QT) % F::KTW, qt = m % F::QT;
      if (kt == 0 && qt == 0 && s + kKAhead < F::DS) read_step(s + kKAhead);
      if (s == 0)
        mfma_score_first(snext[kt][qt], kf[s][kt], w.qf[qt][s]);
      else
        mfma_score(snext[kt][qt], kf[s][kt], w.qf[qt][s]);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c * NS / NC != m) continue;
        if (c < F::SEGS) {
          copy_one<0, D, BLK>(cp, sl.k[ST], jk, c);
        } else {
          copy_one<1, D, BLK>(cp, sl.v[ST ^ 1], jv, c - F::SEGS);
        }
      }
      if (m == NS - 1) pv_prefetch(vf, sl.v[ST]);
#pragma unroll
      for (int e = 0; e < EPS; ++e) sm.element(m * EPS + e);
      __builtin_amdgcn_sched_barrier(0);
    }
    pv(pb, sl.v[ST], vf);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // the scores of block t+1 are read by the VALU in the next iteration; the
    // PV MFMAs issued after them have drained the matrix pipe
    fence_vgpr<false>(snext);
  }

  // The last listed block: softmax and PV only (every copy has landed, so
  // the V slot may be a runtime pointer).
  __device__ __forceinline__ void last(f32x16 (&scur)[F::KTW][F::QT], const unsigned char* vb) {
    bf16x8 pb[F::PS][F::QT];
    Softmax<D, BLK, FAST> sm = {scur, pb, {}, scale_log2, 0.f};
#pragma unroll
    for (int qt = 0; qt < F::QT; ++qt) sm.mb[qt] = w.m[qt] * scale_log2;
    bf16x8 vf[kVAhead + 1];
    pv_prefetch(vf, vb);
#pragma unroll
    for (int e = 0; e < Softmax<D, BLK, FAST>::NE; ++e) sm.element(e);
    pv(pb, vb, vf);
    fence_agpr(w.oacc);  // O may be copied between registers after this point
    __syncthreads();
  }

  // One pass over the row's listed blocks.  With first the reference
  // maximum comes from the first listed block; otherwise w.m is given.
  // PREFETCHED: ls.prefetch has been called for this pass.  before_scores
  // runs once, after the first copies are issued and before any score is
  // computed (also for an empty list).
  template <class BeforeScores>
  __device__ __forceinline__ void run(int lane, bool first, bool prefetched, BeforeScores&& before_scores) {
    if (!prefetched) ls.prefetch(lane);
    const int nvalid = ls.start(lane);
    if (nvalid == 0) {
      before_scores();
      return;
    }
    const int j0 = ls.take(lane);
    int j1 = ls.take(lane), j2 = ls.take(lane);
    fallback = j0;
    // block ids of t+1 and t+2, taken an iteration ahead; past the end of
    // the list (the phantom step, the K copy for a block that does not
    // exist) the fallback is copied and never used
    if (j1 < 0) j1 = fallback;
    if (j2 < 0) j2 = fallback;
    f32x16 sa[F::KTW][F::QT], sb[F::KTW][F::QT];
    // block 0: K(0), K(1) and V(0) are copied together.  The scores of block 0
    // wait only for K(0): this wave's copies of it are the oldest, so
    // vmcnt(2 * SEGS) leaves K(1) and V(0) in flight, and the barrier covers
    // the other waves' copies.
    copy_tile<0, D, BLK>(cp, sl.k[0], j0);
    copy_tile<0, D, BLK>(cp, sl.k[1], j1);
    copy_tile<1, D, BLK>(cp, sl.v[0], j0);
    before_scores();
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * F::SEGS) : "memory");
    scores<D, BLK>(w, sl.k[0], sa);
    if (first) {
      tile_max<D, BLK>(sa, w.m);
      if constexpr (FAST) {
        // no reference maximum: the first block's maxima only decide whether
        // the pass is safe
#pragma unroll
        for (int qt = 0; qt < F::QT; ++qt) {
          w.bad |= !(__builtin_fabsf(w.m[qt]) <= kFastRange);
          w.m[qt] = 0.f;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Steady state, two blocks per turn so that slots are compile-time
    // constants.  Every block but the last computes its successor's scores;
    // when that count is odd one phantom step past the end keeps the turns
    // whole (it copies a valid block and its scores are never used), so the
    // last block always sits in slot 0 and there is a single loop exit.
    const int steps = nvalid - 1;
    const bool phantom = steps & 1;
    for (int turn = 0; turn < (steps + 1) / 2; ++turn) {
      int j3 = ls.take(lane);
      iter<0>(sa, sb, j1, j2);
      j1 = j2;
      j2 = j3 >= 0 ? j3 : fallback;
      j3 = ls.take(lane);
      iter<1>(sb, sa, j1, j2);
      j1 = j2;
      j2 = j3 >= 0 ? j3 : fallback;
    }
    fence_agpr(w.oacc);
    if (!phantom) last(sa, sl.v[0]);
  }

  // Rare path: the true maximum of every query over the listed blocks (no softmax, no V).
  __device__ __forceinline__ void max_sweep(int lane) {
    f32x16 sa[F::KTW][F::QT];
    ls.prefetch(lane);
    ls.start(lane);
    for (int j = ls.take(lane); j >= 0; j = ls.take(lane)) {
      copy_tile<0, D, BLK>(cp, sl.k[0], j);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      scores<D, BLK>(w, sl.k[0], sa);
      float mx[F::QT];
      tile_max<D, BLK>(sa, mx);
#pragma unroll
      for (int qt = 0; qt < F::QT; ++qt) w.m[qt] = fmaxf(w.m[qt], mx[qt]);
      __syncthreads();
    }
  }
};

// Split-KV: with `splits` > 0 workgroup g handles segment g % splits of row
// g / splits, the list positions [s*cnt/splits, (s+1)*cnt/splits), and
// writes a float32 partial result (normalised output and natural-log LSE of
// its segment) that merge_splits_kernel combines.  splits == 0: the whole
// row, written directly.
struct Segment {
  int row, begin, count, part;
};

// SPLIT = false: the whole row, at list position 0 (known before the count
// is loaded).
template <bool SPLIT>
__device__ __forceinline__ Segment segment_of(int g, int splits, const int32_t* __restrict__ kv_cnt, int top_k) {
  Segment sg;
  const int parts = SPLIT ? splits : 1;
  sg.row = SPLIT ? g / parts : g;
  sg.part = g;
  const int cnt = min(max(kv_cnt[sg.row], 0), top_k);
  if constexpr (SPLIT) {
    const int s = g % parts;
    sg.begin = (int)(((long long)s * cnt) / parts);
    sg.count = (int)(((long long)(s + 1) * cnt) / parts) - sg.begin;
  } else {
    sg.begin = 0;
    sg.count = cnt;
  }
  return sg;
}

// A query tile index as a type, so that code taking it indexes accumulator
// registers with a compile-time constant.
template <int I>
struct QTile {
  static constexpr int value = I;
};

// Arguments of one workgroup's row (or split segment): the kernel's, and
// g, the workgroup's index after the XCD regrouping.
struct RowArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_idx;
  const int32_t* kv_cnt;
  uint16_t* out;
  float* lse;
  float* part_o;
  float* part_lse;
  int nq, nk, top_k, splits, g;
  float scale_log2;
};

// One row (or split segment) of attention with the workgroup's LDS slots.
// FAST: Q is multiplied by log2(e)/sqrt(d) once, in bf16, so a score is
// already the exponent of its probability, and probabilities are exp2(s)
// with no reference maximum subtracted (one VALU operation less per score).
// That is the same softmax as long as nothing overflows or underflows; the
// pass returns false without writing anything when a query's maximum over
// the first listed block lies outside [-kFastRange, kFastRange] or a block's
// probability sum reaches kFastGuard.  Otherwise (FAST = false): unscaled Q,
// the first block's maximum as reference, and the rerun at the true maximum
// described in the file header; always returns true.
template <int D, int BLK, bool FAST, bool SPLIT>
__device__ __forceinline__ bool attend_row(const RowArgs a, const Slots sl) {
  using F = Fa<D, BLK>;
  const uint16_t* q = a.q;
  const int32_t* kv_idx = a.kv_idx;
  const int32_t* kv_cnt = a.kv_cnt;
  const int nq = a.nq, nk = a.nk, top_k = a.top_k, splits = a.splits;
  const float scale_log2 = a.scale_log2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = wave % F::NQG, kg = wave / F::NQG;
  const int qc = lane & 31, hh = lane >> 5;
  const int kbase = kg * F::KW;
  // The row's loads go out together: its count, its list, then its Q.  Each
  // is waited for where it is used, the count only after Q has been issued.
  Segment sg;
  int cnt_raw = 0;
  if constexpr (SPLIT) {
    sg = segment_of<true>(a.g, splits, kv_cnt, top_k);
  } else {
    sg.row = sg.part = a.g;
    sg.begin = 0;
    cnt_raw = kv_cnt[sg.row];
  }
  const int row = sg.row;
  const int bh = row / nq, iq = row % nq;
  const size_t N = (size_t)nk * BLK;
  const uint16_t* kh = a.k + (size_t)bh * N * D;
  const uint16_t* vh = a.v + (size_t)bh * N * D;
  ListStream ls;
  ls.list = kv_idx + (size_t)row * top_k + sg.begin;
  ls.nk = nk;
  ls.cap = SPLIT ? sg.count : top_k;
  ls.prefetch(lane);
  asm volatile("" ::: "memory");  // the list stays ahead of Q: the copies wait for it, not for Q

  WaveState<D, BLK> w;
  const size_t qrow0 = (size_t)bh * nq * BLK + (size_t)iq * BLK + qg * F::QW;
  // The row's Q is loaded now, right behind its list, and moved into the
  // B-operand fragments (take_q) only where the pass needs it, so that the
  // latencies of the list, Q and the first copies overlap.
  uint4 qraw[F::QT][F::DS];
#pragma unroll
  for (int qt = 0; qt < F::QT; ++qt) {
    // B operand of S^T = K Q^T: lane l holds query 32qt + l%32 of this wave's
    // group, d = 16s + 8(l/32) + 0..7
    const uint4* qrow = reinterpret_cast<const uint4*>(q + (qrow0 + 32 * qt + qc) * D);
#pragma unroll
    for (int s = 0; s < F::DS; ++s) qraw[qt][s] = qrow[2 * s + hh];
  }
  if constexpr (!SPLIT) {
    asm volatile("" : "+v"(cnt_raw));  // not used before this point
    sg.count = __builtin_amdgcn_readfirstlane(min(max(cnt_raw, 0), top_k));
  }
  ls.cnt = sg.count;
  auto take_q = [&]() {
#pragma unroll
    for (int qt = 0; qt < F::QT; ++qt)
#pragma unroll
      for (int s = 0; s < F::DS; ++s) {
        if constexpr (FAST) {
          bf16x8 raw;
          __builtin_memcpy(&raw, &qraw[qt][s], 16);
#pragma unroll
          for (int e = 0; e < 8; ++e) w.qf[qt][s][e] = (__bf16)((float)raw[e] * scale_log2);
        } else {
          __builtin_memcpy(&w.qf[qt][s], &qraw[qt][s], 16);
        }
        asm volatile("" : "+a"(w.qf[qt][s]));  // Q lives in AGPRs
      }
  };
#pragma unroll
  for (int qt = 0; qt < F::QT; ++qt) {
    w.m[qt] = -__builtin_inff();
    w.l[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < F::DT; ++dt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) w.oacc[dt][qt][r] = 0.f;
      asm volatile("" : "+a"(w.oacc[dt][qt]));  // O lives in AGPRs
    }
  }
#pragma unroll
  for (int s = 0; s < F::DS; ++s) {
    const int r = kbase + qc;
    w.ko[s] = (uint32_t)(r * F::NCH + ((2 * s + hh) ^ F::swz_k(r))) * 16u;
  }
  {
    const int grp = lane >> 4, j = lane & 15;
    const int gd = grp & 1;
    const int key0 = kbase + 4 * hh + (j >> 2);
    const int vsw = F::swz_v(key0);
#pragma unroll
    for (int dt = 0; dt < F::DT; ++dt) {
      const int c = (4 * dt + 2 * gd + ((j & 3) >> 1)) ^ vsw;
      w.vo[dt] = (uint32_t)(key0 * F::NCH * 16 + 8 * (j & 1) + c * 16);
    }
  }
  Copier<D, BLK> cp;
  cp.init(kh, vh, (uint32_t)(N * D * 2), wave, lane);
  w.bad = false;
  Pass<D, BLK, FAST> pass = {w, sl, ls, cp, scale_log2, 0};
  for (bool first = true;; first = false) {
    // Q is taken before the fast pass (it arrives together with the list the
    // pass waits for first) and, in the general pass, after its first copies;
    // these placements keep the block loop's code as tight as before and the
    // general pass free of AGPR rewrites next to its MFMAs.
    if (!first) {
      pass.run(lane, false, false, [] {});
    } else if constexpr (FAST) {
      take_q();
      pass.run(lane, true, true, [] {});
    } else {
      pass.run(lane, true, true, take_q);
    }
    if (!first) break;
    // Did any lane of any wave see an overflow?  One flag per wave in a free
    // slot (every copy has landed and every wave has passed the last barrier).
    int* flags = reinterpret_cast<int*>(sl.v[0]);
    if (lane == 0) flags[wave] = __builtin_amdgcn_ballot_w64(w.bad) != 0;
    __syncthreads();
    int any_bad = 0;
#pragma unroll
    for (int i = 0; i < F::NW; ++i) any_bad |= flags[i];
    __syncthreads();
    if (!any_bad) break;
    if constexpr (FAST) return false;
    // Rare: some logit exceeded the first block's maximum by more than 40
    // log2-units.  Find each query's true maximum, then redo the row at it.
#pragma unroll
    for (int qt = 0; qt < F::QT; ++qt) {
      w.m[qt] = -__builtin_inff();
      w.l[qt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < F::DT; ++dt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) w.oacc[dt][qt][r] = 0.f;
        asm volatile("" : "+a"(w.oacc[dt][qt]));
      }
    }
    pass.max_sweep(lane);
  }
  __syncthreads();
  fence_agpr(w.oacc);  // the last PV MFMAs have written O before it is read

  // Merge the two key halves.  The two waves of a query group split the work
  // by query tile: wave kg hands (m, l, O) of query tile 1 - kg to its
  // partner through LDS and merges query tile kg.  The handed-over O fills
  // both K slots exactly (2 * NQG waves * DT * 16 registers of 64 lanes =
  // 2 * BLK * D * 2 bytes).
  static_assert(F::QT == 2, "one query tile per key half");
  constexpr int HALF = F::NQG * F::DT * F::QT * 16 / 2;  // register slots per K slot
  float* xm = reinterpret_cast<float*>(sl.v[0]);       // m: [qg][qt][lane], then l: [qg][qt][lane]
  // registers 4rq..4rq+3 of accumulator (dt, qt): one 16-byte LDS access per lane
  auto xo_at = [&](int dt, int qt, int rq) -> float4* {
    const int f = ((qg * F::DT + dt) * F::QT + qt) * 4 + rq;
    return f < HALF / 4 ? reinterpret_cast<float4*>(sl.k[0]) + f * 64 + lane
                        : reinterpret_cast<float4*>(sl.k[1]) + (f - HALF / 4) * 64 + lane;
  };
  float lw[F::QT];
#pragma unroll
  for (int qt = 0; qt < F::QT; ++qt) lw[qt] = w.l[qt] + __shfl_xor(w.l[qt], 32);
  auto hand_over = [&](auto tile) {
    constexpr int qt = decltype(tile)::value;
    xm[(qg * F::QT + qt) * 64 + lane] = w.m[qt];
    xm[((F::NQG + qg) * F::QT + qt) * 64 + lane] = lw[qt];
#pragma unroll
    for (int dt = 0; dt < F::DT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *xo_at(dt, qt, rq) = make_float4(w.oacc[dt][qt][4 * rq], w.oacc[dt][qt][4 * rq + 1],
                                         w.oacc[dt][qt][4 * rq + 2], w.oacc[dt][qt][4 * rq + 3]);
  };
  auto merge = [&](auto tile) {
    constexpr int qt = decltype(tile)::value;
    const float m1 = xm[(qg * F::QT + qt) * 64 + lane];
    const float l1 = xm[((F::NQG + qg) * F::QT + qt) * 64 + lane];
    const float m0 = w.m[qt];
    const float mm = fmaxf(m0, m1);
    const float msc = FAST ? 1.0f : scale_log2;  // reference maxima to log2 units
    const float a0 = m0 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((m0 - mm) * msc);
    const float a1 = m1 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((m1 - mm) * msc);
    const float lt = lw[qt] * a0 + l1 * a1;
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const size_t tq = qrow0 + 32 * qt + qc;
    // split mode: float32 partial result of this segment, token t of the block
    const size_t pt = ((size_t)sg.part * BLK + qg * F::QW + 32 * qt + qc);
    uint16_t* orow = a.out + tq * D;
    float* prow = a.part_o + pt * D;
#pragma unroll
    for (int dt = 0; dt < F::DT; ++dt) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const float4 x = *xo_at(dt, qt, rq);
        const float xe[4] = {x.x, x.y, x.z, x.w};
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (w.oacc[dt][qt][4 * rq + e] * a0 + xe[e] * a1) * inv;
        if constexpr (SPLIT) {
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
        lt > 0.f ? (mm * msc + __builtin_log2f(lt)) * 0.69314718055994531f : -__builtin_inff();
    if (hh == 0) {
      if constexpr (SPLIT)
        a.part_lse[pt] = row_lse;
      else if (a.lse)
        a.lse[tq] = row_lse;
    }
  };
  if (kg == 0)
    hand_over(QTile<1>{});
  else
    hand_over(QTile<0>{});
  __syncthreads();
  if (kg == 0)
    merge(QTile<0>{});
  else
    merge(QTile<1>{});
  return true;
}

// The general pass, compiled as a function of its own so that its registers
// do not constrain the fast pass inlined in the kernel.
template <int D, int BLK, bool SPLIT>
__device__ __attribute__((noinline)) void attend_row_general(const RowArgs a, const Slots sl) {
  attend_row<D, BLK, false, SPLIT>(a, sl);
}

// SPLIT: split-KV segments (splits > 0) instead of whole rows.
template <int D, int BLK, bool SPLIT>
__global__ __launch_bounds__(2 * BLK) __attribute__((amdgpu_waves_per_eu(1, 1))) void sparse_fa_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ kv_cnt, uint16_t* __restrict__ out,
    float* __restrict__ lse, int nq, int nk, int top_k, float scale_log2, int splits, float* __restrict__ part_o,
    float* __restrict__ part_lse) {
  using F = Fa<D, BLK>;
  __shared__ __attribute__((aligned(1024))) unsigned char k_slot0[F::T];
  __shared__ __attribute__((aligned(1024))) unsigned char k_slot1[F::T];
  __shared__ __attribute__((aligned(1024))) unsigned char v_slot0[F::T];
  __shared__ __attribute__((aligned(1024))) unsigned char v_slot1[F::T];
  const Slots sl = {{k_slot0, k_slot1}, {v_slot0, v_slot1}};
  const RowArgs a = {q, k, v, kv_idx, kv_cnt, out, lse, part_o, part_lse, nq, nk, top_k, splits,
                     xcd_grouped(blockIdx.x, gridDim.x), scale_log2};
  if (!attend_row<D, BLK, true, SPLIT>(a, sl)) attend_row_general<D, BLK, SPLIT>(a, sl);
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
  const Segment sg = splits > 0 ? segment_of<true>(blockIdx.x, splits, kv_cnt, top_k)
                                 : segment_of<false>(blockIdx.x, splits, kv_cnt, top_k);
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
  auto kern = splits > 0 ? sparse_fa_bf16_kernel<D, BLK, true> : sparse_fa_bf16_kernel<D, BLK, false>;
  hipLaunchKernelGGL(kern, dim3(rows * (splits > 0 ? splits : 1)), dim3(Fa<D, BLK>::NT), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
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
