/*
 * velox.h -- C ABI of the Velox routed block-sparse attention layer for
 * AMD Instinct MI355X (CDNA4, gfx950).
 *
 * The method (sns.style, "Velox: spatial memory speeds up video world
 * models", section Deep analysis, all four language editions): a chunked
 * video-diffusion model keeps a KV cache that grows by one chunk per step.
 * In every attention layer Velox takes the block importance the model
 * already computes, softly modulates it by how much each past chunk's
 * camera-frustum slice overlaps the query region, leaves regions that the
 * history does not cover on the model's native routing, keeps the most
 * important KV blocks per query block, and runs tiled attention that
 * skips the other blocks.  Routing decisions are made at the kernel's tile
 * size so that skipped blocks are really skipped (same section, paragraph
 * on token-block granularity).
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers to contiguous row-major arrays,
 *    owned by the caller.  Q, K, V and Out must be 16-byte aligned.
 *  - The library never allocates, frees, synchronises or prints.  Calls
 *    enqueue work on `stream` (a hipStream_t; NULL = the default stream)
 *    and return immediately.
 *  - Arguments are validated on the host before any launch; on an error
 *    nothing is launched and nothing is written.
 *  - Device data is trusted apart from block lists: NaN or Inf in Q, K,
 *    V, scores or overlap give unspecified (but memory-safe) results.
 *  - Functions are thread-safe; the library holds no state except the
 *    thread-local HIP error code of the last failed launch.
 *
 * Shapes (notation of the problem struct below):
 *   nq = T / blk query blocks, nk = N / blk KV blocks with N = (C+1)*T,
 *   ncur = T / blk current-chunk blocks (the last ncur KV blocks),
 *   chunk(j) = floor(j*blk / T) is the chunk of KV block j (C = current),
 *   k_eff = min(top_k, nk); a "row" is one (b, h, i) query block.
 */
#ifndef VELOX_H_
#define VELOX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t *velox_stream_t;

typedef enum velox_status {
  VELOX_OK = 0,
  VELOX_ERR_NULL_POINTER = 1, /* a required pointer is NULL                                  */
  VELOX_ERR_BAD_SHAPE = 2,    /* sizes < 1, T % blk != 0, top_k < ncur, alpha < 0 or not finite,
                                 unknown modulation                                          */
  VELOX_ERR_UNSUPPORTED = 3,  /* (dtype, d, blk) not built, or nq / nk above the limits below */
  VELOX_ERR_MISALIGNED = 4,   /* Q, K, V or Out not 16-byte aligned                          */
  VELOX_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than velox_route_workspace_bytes  */
  VELOX_ERR_HIP = 6           /* a launch failed; velox_last_hip_error() holds the hipError_t */
} velox_status;

typedef enum velox_dtype { VELOX_F32 = 0, VELOX_BF16 = 1 } velox_dtype;

/* How the overlap modulates the importance of a past block j of a covered
 * row (both readings of the article's Deep analysis: the overlap softly
 * modulates, and does not replace, the model's own block importance):
 *   VELOX_MOD_SCALE     m_j = s_j * (1 + alpha * o)       the literal reading;
 *                       for s_j < 0 a larger overlap lowers m_j.
 *   VELOX_MOD_LOG_PROB  m_j = s_j + log1p(alpha * o)      the importance read as
 *                       the softmax probability p_j of s_j: p_j*(1 + alpha*o)
 *                       ranks exactly like this, so a larger overlap never
 *                       lowers a block's rank whatever the sign of s_j.
 * In float32: alpha*o, then log1p in float64 rounded once to float32, then
 * one float32 addition. */
typedef enum velox_modulation { VELOX_MOD_SCALE = 0, VELOX_MOD_LOG_PROB = 1 } velox_modulation;

/* Built configurations: d in {64, 128}, blk in {64, 128}, both dtypes.
 * Limits: nq <= VELOX_MAX_QUERY_BLOCKS, nk <= VELOX_MAX_KV_BLOCKS, B*H <= VELOX_MAX_HEADS_TOTAL
 * (the scoring kernels put the (b,h) pair on the second grid axis). */
#define VELOX_MAX_QUERY_BLOCKS 64
#define VELOX_MAX_KV_BLOCKS 8192
#define VELOX_MAX_HEADS_TOTAL 65535

typedef struct velox_problem {
  int32_t batch;        /* B: independent rollouts                                         */
  int32_t heads;        /* H: heads, equal for Q and KV                                    */
  int32_t head_dim;     /* d                                                               */
  int32_t chunk_tokens; /* T: query tokens = tokens per chunk                              */
  int32_t past_chunks;  /* C >= 0: number of past chunks; N = (C+1)*T KV tokens, the
                           current chunk being the last T of them                          */
  int32_t block;        /* blk: routing block = attention tile, for queries and keys       */
  int32_t top_k;        /* kept KV blocks per row including the ncur current blocks
                           (top_k >= ncur); values above nk keep every block               */
  float alpha;          /* modulation strength, finite and >= 0                            */
  int32_t dtype;        /* a velox_dtype: element type of Q, K, V and Out (an int32, so
                           that any value a caller passes can be checked)                  */
  int32_t modulation;   /* a velox_modulation (0 = VELOX_MOD_SCALE when zero-initialised);
                           used by routing, must be valid everywhere                       */
} velox_problem;

/* Validate a problem on the host (no GPU needed).  Returns VELOX_OK,
 * VELOX_ERR_NULL_POINTER (p == NULL), VELOX_ERR_BAD_SHAPE or
 * VELOX_ERR_UNSUPPORTED. */
velox_status velox_check(const velox_problem *p);

/* Bytes of device workspace velox_route needs for this problem (pooled
 * queries and, when `scores` is NULL, the score matrix); 0 if p is invalid. */
size_t velox_route_workspace_bytes(const velox_problem *p);

/* Routing: block importance, overlap modulation and per-row top-k
 * (sns.style "Velox" article, Deep analysis, third and fourth steps).
 *
 *   q        [B,H,T,d]  dtype         queries of the current chunk
 *   k        [B,H,N,d]  dtype         keys of the whole cache (past chunks, then current)
 *   overlap  [B,nq,C]   float32       frustum-slice overlap of query block i with past
 *                                     chunk c, expected in [0,1] (not clamped); may be
 *                                     NULL when C == 0
 *   covered  [B,nq]     uint8         0 = history does not cover the region: native
 *                                     routing (no modulation); non-zero = covered
 *   kv_idx   [B,H,nq,top_k] int32 out kept KV block ids of each row, ascending; the
 *                                     entries after the first k_eff are -1
 *   kv_cnt   [B,H,nq]   int32   out   k_eff for every row
 *   scores   [B,H,nq,nk] float32 out  optional: the raw importance s (NULL = not written)
 *   workspace, workspace_bytes        device scratch of at least
 *                                     velox_route_workspace_bytes(p) bytes, 256-byte aligned
 *
 * Per row (b,h,i): qbar_i and kbar_j are the means of Q over query block i
 * and of K over KV block j (float32 sums); s_j = <qbar_i, kbar_j>/sqrt(d)
 * (float32 matrix-core products and sums);
 * m_j = +inf for current-chunk blocks, the modulated importance of
 * p->modulation with o = overlap[b,i,chunk(j)] for past blocks of covered
 * rows (s_j*(1 + alpha*o) by default), s_j otherwise (every operation a
 * separately rounded float32 operation).  The kept set is the k_eff largest
 * m_j, ties broken toward the lower block index (-0 equals +0). */
velox_status velox_route(const velox_problem *p, const void *q, const void *k, const float *overlap,
                         const uint8_t *covered, int32_t *kv_idx, int32_t *kv_cnt, float *scores,
                         void *workspace, size_t workspace_bytes, velox_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): velox_route
 * with its workspace taken from a scratch array the library holds per GPU
 * (VELOX_NOALLOC_SCRATCH_BYTES, held by each GPU the call runs on until the
 * process ends).  Arguments and results as velox_route, without `workspace`;
 * the same kernels run, so kv_idx, kv_cnt and scores are identical to
 * velox_route's.  The call allocates nothing (no hipMalloc or hipFree); its
 * first call on a device looks the array's address up there.
 * Errors: velox_route's, and VELOX_ERR_WORKSPACE when the pooled queries plus,
 * if `scores` is NULL, the score matrix exceed VELOX_NOALLOC_SCRATCH_BYTES
 * (checked before any device work).  The array is shared by every call on one
 * GPU and keeps the last call's contents (every byte a call reads it wrote
 * first): calls that overlap on one GPU, e.g. on two streams, race. */
#define VELOX_NOALLOC_SCRATCH_BYTES (24u << 20)
velox_status velox_route_noalloc(const velox_problem *p, const void *q, const void *k, const float *overlap,
                                 const uint8_t *covered, int32_t *kv_idx, int32_t *kv_cnt, float *scores,
                                 velox_stream_t stream);

/* The scoring step of velox_route alone: writes the raw importance
 * s [B,H,nq,nk] float32 (same values as velox_route's `scores`) for a later
 * velox_select.  Lets a caller build the overlap concurrently (below) and
 * join before the selection.  workspace: at least
 * velox_route_workspace_bytes(p) bytes, 256-byte aligned. */
velox_status velox_score(const velox_problem *p, const void *q, const void *k, float *scores, void *workspace,
                         size_t workspace_bytes, velox_stream_t stream);

/* Overlap of past chunks' camera-frustum slices with the current view's
 * query strips (the article's Deep analysis, first and third steps; the
 * slices are built asynchronously next to denoising, same section).  The
 * article gives no geometry; here chunk c sees horizontal angles
 * yaw_c +- fov/2 and depths [near_c, far_c], query block i is the i-th of nq
 * equal angular strips of the current view (yaw_C) with depths
 * [qnear_i, qfar_i], and
 *   overlap[b,i,c] = (fraction of strip i's angle inside chunk c's range)
 *                  * (fraction of [qnear_i, qfar_i] inside [near_c, far_c])
 * with angle differences wrapped to (-180, 180]; covered[b,i] = 1 if any
 * overlap of the row is > 0, else 0.  float32 arithmetic.
 *   yaw          [B, C+1] float32 degrees, yaw[b, C] = the current view
 *   past_depth   [B, C, 2] float32 (near, far) of each past chunk
 *   query_depth  [B, nq, 2] float32 (near, far) of each query strip
 *   fov_deg      horizontal field of view, in (0, 180] (else VELOX_ERR_BAD_SHAPE)
 *   overlap      [B, nq, C] float32 out (may be NULL when C == 0)
 *   covered      [B, nq] uint8 out
 * Only batch, chunk_tokens, block and past_chunks of p are used (the rest
 * must be valid). */
velox_status velox_frustum_overlap(const velox_problem *p, const float *yaw, const float *past_depth,
                                   const float *query_depth, float fov_deg, float *overlap, uint8_t *covered,
                                   velox_stream_t stream);

/* Incremental pooled-key cache (the article's Outlook section: behaviour for
 * rollouts far longer than 48 chunks; with the cache kept per layer, past
 * chunks' keys, which do not change, are pooled once instead of on every
 * routing call).
 *
 * velox_pool_keys writes the float32 means of K over KV blocks
 * [first_block, first_block + num_blocks) of every (b,h) into the cache:
 *   k     [B,H,N,d] dtype   keys (N = (C+1)*T from p; top_k and alpha of p are
 *                           not used but must be valid, top_k >= 1)
 *   kbar  [B,H,cache_blocks,d] float32 out, 16-byte aligned; only the rows of
 *                           the pooled blocks are written
 * Requires 0 <= first_block, 0 <= num_blocks, first_block + num_blocks <= nk
 * and <= cache_blocks (else VELOX_ERR_BAD_SHAPE).  num_blocks == 0 is a no-op.
 * The values are bit-identical to the pooled keys velox_route computes. */
velox_status velox_pool_keys(const velox_problem *p, const void *k, float *kbar, int32_t cache_blocks,
                             int32_t first_block, int32_t num_blocks, velox_stream_t stream);

/* velox_route with the pooled keys read from a cache filled by
 * velox_pool_keys instead of pooled from K.  Rows [0, C*nq) of kbar (the
 * past chunks) must hold the pooled keys; rows [C*nq, nk) (the current
 * chunk) are read only when `scores` is requested, since the current chunk is
 * always kept.  cache_blocks is kbar's row stride in blocks and must cover
 * the rows read (else VELOX_ERR_BAD_SHAPE).  Other arguments, the workspace
 * size and the outputs are those of velox_route, and for the same pooled
 * keys the outputs are bit-identical to it. */
velox_status velox_route_cached(const velox_problem *p, const void *q, const float *kbar, int32_t cache_blocks,
                                const float *overlap, const uint8_t *covered, int32_t *kv_idx, int32_t *kv_cnt,
                                float *scores, void *workspace, size_t workspace_bytes, velox_stream_t stream);

/* The modulation and top-k steps of velox_route alone, from importance
 * scores the caller provides (`scores` [B,H,nq,nk] float32, device; read
 * only).  Same outputs and rules as velox_route; q and k are not needed. */
velox_status velox_select(const velox_problem *p, const float *scores, const float *overlap,
                          const uint8_t *covered, int32_t *kv_idx, int32_t *kv_cnt, velox_stream_t stream);

/* Block-skipping tiled attention (sns.style "Velox" article, Deep analysis,
 * paragraph on token-block granularity and FlashAttention-style tiles).
 * p->top_k is the row stride of kv_idx (any value >= 1; the routing bound
 * top_k >= ncur does not apply here) and p->alpha is ignored but must be
 * valid.
 *
 *   q [B,H,T,d], k and v [B,H,N,d]      dtype
 *   kv_idx [B,H,nq,top_k] int32, kv_cnt [B,H,nq] int32: per row the KV blocks
 *        to attend; the first min(max(kv_cnt,0), top_k) entries are used and
 *        entries outside [0, nk) are skipped, so a bad list never reads out
 *        of bounds.  Lists need not be sorted; a block listed twice counts twice.
 *   out [B,H,T,d] dtype out: for query token t of block i,
 *        softmax(q_t K_U^T / sqrt(d)) V_U over the tokens U of the listed
 *        blocks (no causal mask); bf16 output is rounded to nearest even.
 *        A row with no valid block gets zeros.
 *   lse [B,H,T] float32 out, optional (NULL = not written): natural-log
 *        sum of exp of the scaled logits (-inf for an empty row).
 * Arithmetic: bf16 MFMA products with float32 accumulation, float32 softmax;
 * the probabilities are rounded to bf16 before the PV product.  float32
 * problems use float32 throughout. */
velox_status velox_sparse_attn(const velox_problem *p, const void *q, const void *k, const void *v,
                               const int32_t *kv_idx, const int32_t *kv_cnt, void *out, float *lse,
                               velox_stream_t stream);

/* Split-KV attention for problems with few rows (fewer rows than compute
 * units leave most of the GPU idle: the Small workload has 64 rows for 256
 * CUs).  Each row's block list is cut into num_splits contiguous segments,
 * list positions [s*cnt/num_splits, (s+1)*cnt/num_splits) for s = 0..num_splits-1;
 * every segment is attended by its own workgroup, which writes a float32
 * partial result (its normalised output and natural-log LSE) to the
 * workspace, and a merge launch combines them exactly:
 *   LSE = log sum_s exp(LSE_s),  out = sum_s exp(LSE_s - LSE) * out_s,
 * segments without a valid block having weight 0.  Arguments and results
 * are those of velox_sparse_attn (same kernels per segment; rounding may
 * differ from the unsplit call in the last bits), plus:
 *   num_splits   1 .. VELOX_MAX_SPLITS (else VELOX_ERR_BAD_SHAPE)
 *   workspace    device scratch, 256-byte aligned, of at least
 *                velox_sparse_attn_split_workspace_bytes(p, num_splits) bytes
 *                (else VELOX_ERR_WORKSPACE).  Same article section as
 *                velox_sparse_attn; the split itself is this library's
 *                scheduling choice, not the article's. */
#define VELOX_MAX_SPLITS 64
size_t velox_sparse_attn_split_workspace_bytes(const velox_problem *p, int32_t num_splits);

/* Host-only heuristic: a split count that gives about two workgroups per
 * compute unit (num_cus, e.g. 256 on MI355X) with at least 4 listed blocks
 * per segment; 1 when the rows alone fill the GPU or p is invalid. */
int32_t velox_sparse_attn_auto_splits(const velox_problem *p, int32_t num_cus);

velox_status velox_sparse_attn_split(const velox_problem *p, const void *q, const void *k, const void *v,
                                     const int32_t *kv_idx, const int32_t *kv_cnt, int32_t num_splits, void *out,
                                     float *lse, void *workspace, size_t workspace_bytes, velox_stream_t stream);

/* Static English description of a status code. */
const char *velox_status_string(int32_t status);

/* hipError_t of the last failed launch on the calling thread (0 = none). */
int velox_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VELOX_H_ */
