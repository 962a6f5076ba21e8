/*
 * velox_oracle.c -- TEST INFRASTRUCTURE, not product code.
 *
 * A plain, slow, obviously correct CPU definition of the Velox routed
 * attention layer, used only to check the GPU path: by the tests, by the
 * package's smoke check and by the benchmark's CPU-baseline leg.  Nothing
 * in the product path may load it.  It shares no source with the HIP
 * kernels and includes none of their headers.
 *
 * Every input element is widened exactly to double and all arithmetic is
 * fp64 (except velox_oracle_modulate_f32, which takes the selection
 * decision in fp32 on purpose).  OpenMP parallelises over independent
 * rows / query tokens only; no blocking, fusion or reordering of the sums.
 *
 * Source: the Velox article (sns.style, "Velox: spatial memory speeds up
 * video world models", section Deep analysis in each language edition).
 * The article describes the steps in words and gives no formula; the
 * formulas below are the plain reading of those words:
 *   1. the model's own block importance, taken as the dot product of the
 *      mean-pooled query block and mean-pooled key block scaled by
 *      1/sqrt(d);
 *   2. soft modulation of that importance by frustum-slice overlap,
 *      m = s * (1 + alpha * overlap), only for query regions that history
 *      covers; uncovered regions keep the plain score (native routing);
 *      blocks of the current chunk are always kept;
 *   3. per query block, keep the k highest modulated scores (ties go to
 *      the lowest block index);
 *   4. FlashAttention-style attention of every query token of the block
 *      over the tokens of the kept KV blocks only (softmax with scale
 *      1/sqrt(d), no causal mask).
 *
 * Parity pins (tests/test_oracle.py): closed forms for pooling, the
 * blk = 1 reduction of the score to token logits, hand-computed worked
 * examples for modulation and selection (tests/golden/), brute-force
 * subset enumeration for the selection, keep-all against brute-force
 * dense attention, closed-form two-key and zero-query attention, and the
 * skipped-block poison invariant; closed forms over several batch
 * elements, heads and query blocks (every (b,h), query block and KV block
 * carrying its own constant) for pooling, scores, listed and dense
 * attention, so that every row and head stride is pinned; for the
 * sign-safe modulation a worked example and a brute-force softmax check;
 * for the frustum overlap closed forms and a Monte Carlo estimate.  Every
 * function here has such a pin.
 * Against Velox as published, parity unpinned: the article prints no
 * formula, worked example or intermediate value for these steps.
 *
 * dtype codes: 0 = float32, 1 = bfloat16 bit patterns (uint16).
 * All functions return 0 on success and a negative value on bad arguments.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double elem(const void *x, int dtype, int64_t i) {
  if (dtype == 0) return (double)((const float *)x)[i];
  uint32_t u = (uint32_t)((const uint16_t *)x)[i] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int velox_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count for the following calls (n >= 1); no effect on the results,
 * every parallel loop writes disjoint outputs. */
void velox_oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Mean of each group of `blk` consecutive rows of x, viewed as
 * [nblocks * blk, d].  out: [nblocks, d]. */
int velox_oracle_pool(const void *x, int dtype, int64_t nblocks, int blk, int d, double *out) {
  if (!x || !out || nblocks < 0 || blk < 1 || d < 1) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nblocks; ++b) {
    for (int e = 0; e < d; ++e) {
      double sum = 0.0;
      for (int t = 0; t < blk; ++t) sum += elem(x, dtype, (b * blk + t) * (int64_t)d + e);
      out[b * d + e] = sum / (double)blk;
    }
  }
  return 0;
}

/* s[bh, i, j] = <qbar[bh, i, :], kbar[bh, j, :]> / sqrt(d). */
int velox_oracle_scores(const double *qbar, const double *kbar, int64_t BH, int nq, int nk, int d,
                        double *s) {
  if (!qbar || !kbar || !s || BH < 0 || nq < 0 || nk < 0 || d < 1) return -1;
  const double scale = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < BH * nq; ++r) {
    const int64_t bh = r / nq;
    const double *qi = qbar + r * d;
    for (int j = 0; j < nk; ++j) {
      const double *kj = kbar + (bh * nk + j) * d;
      double dot = 0.0;
      for (int e = 0; e < d; ++e) dot += qi[e] * kj[e];
      s[r * nk + j] = dot * scale;
    }
  }
  return 0;
}

/* Modulated importance m[b,h,i,j] (rows = (b,h,i)):
 *   chunk(j) = floor(j*blk / T); chunk(j) == C is the current chunk;
 *   current chunk                  -> +infinity (always kept)
 *   past chunk, covered[b,i] != 0  -> s * (1 + alpha * overlap[b,i,chunk(j)])
 *   past chunk, uncovered          -> s            (native routing)      */
int velox_oracle_modulate(const double *s, const float *overlap, const uint8_t *covered, int B, int H,
                          int nq, int nk, int blk, int T, int C, double alpha, double *m) {
  if (!s || !m || !covered || (C > 0 && !overlap) || B < 0 || H < 0 || blk < 1 || T < blk) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < (int64_t)B * H * nq; ++r) {
    const int64_t b = r / ((int64_t)H * nq);
    const int i = (int)(r % nq);
    for (int j = 0; j < nk; ++j) {
      const int c = (int)(((int64_t)j * blk) / T);
      const double sv = s[r * nk + j];
      double mv;
      if (c >= C)
        mv = INFINITY;
      else if (covered[b * nq + i])
        mv = sv * (1.0 + alpha * (double)overlap[(b * nq + i) * (int64_t)C + c]);
      else
        mv = sv;
      m[r * nk + j] = mv;
    }
  }
  return 0;
}

/* The same modulation with the decision taken in fp32: s, overlap and
 * alpha are float32 and every operation is a separately rounded float32
 * operation (1 + alpha*o first, then the product).  Built with
 * -ffp-contract=off so that no fused multiply-add changes the rounding. */
int velox_oracle_modulate_f32(const float *s, const float *overlap, const uint8_t *covered, int B, int H,
                              int nq, int nk, int blk, int T, int C, float alpha, double *m) {
  if (!s || !m || !covered || (C > 0 && !overlap) || B < 0 || H < 0 || blk < 1 || T < blk) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < (int64_t)B * H * nq; ++r) {
    const int64_t b = r / ((int64_t)H * nq);
    const int i = (int)(r % nq);
    for (int j = 0; j < nk; ++j) {
      const int c = (int)(((int64_t)j * blk) / T);
      const float sv = s[r * nk + j];
      float mv;
      if (c >= C) {
        mv = INFINITY;
      } else if (covered[b * nq + i]) {
        const float ao = alpha * overlap[(b * nq + i) * (int64_t)C + c];
        const float f = 1.0f + ao;
        mv = sv * f;
      } else {
        mv = sv;
      }
      m[r * nk + j] = (double)mv;
    }
  }
  return 0;
}

/* Sign-safe variant of the modulation.  The article says the overlap softly
 * modulates the model's own importance; read as a probability, that
 * importance is p_j = softmax_j(s_j) over the row's blocks, and the soft
 * modulation multiplies it: p_j * (1 + alpha * overlap).  Because the log is
 * increasing and log p_j = s_j - log(sum_l exp(s_l)) differs from s_j by a
 * per-row constant, the ranking is the ranking of
 *   m_j = s_j + log1p(alpha * overlap)
 * for past blocks of covered rows (current blocks +inf, uncovered rows s_j).
 * Unlike s * (1 + alpha*o), this never lowers a negative score's rank when
 * the overlap grows.  fp64 throughout. */
int velox_oracle_modulate_logprob(const double *s, const float *overlap, const uint8_t *covered, int B, int H,
                                  int nq, int nk, int blk, int T, int C, double alpha, double *m) {
  if (!s || !m || !covered || (C > 0 && !overlap) || B < 0 || H < 0 || blk < 1 || T < blk) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < (int64_t)B * H * nq; ++r) {
    const int64_t b = r / ((int64_t)H * nq);
    const int i = (int)(r % nq);
    for (int j = 0; j < nk; ++j) {
      const int c = (int)(((int64_t)j * blk) / T);
      const double sv = s[r * nk + j];
      double mv;
      if (c >= C)
        mv = INFINITY;
      else if (covered[b * nq + i])
        mv = sv + log1p(alpha * (double)overlap[(b * nq + i) * (int64_t)C + c]);
      else
        mv = sv;
      m[r * nk + j] = mv;
    }
  }
  return 0;
}

/* The sign-safe variant with the decision in fp32: a = alpha*o in float32,
 * the log term log1p(a) evaluated in fp64 and rounded once to float32, then
 * m = s + that term as one float32 addition. */
int velox_oracle_modulate_logprob_f32(const float *s, const float *overlap, const uint8_t *covered, int B,
                                      int H, int nq, int nk, int blk, int T, int C, float alpha, double *m) {
  if (!s || !m || !covered || (C > 0 && !overlap) || B < 0 || H < 0 || blk < 1 || T < blk) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < (int64_t)B * H * nq; ++r) {
    const int64_t b = r / ((int64_t)H * nq);
    const int i = (int)(r % nq);
    for (int j = 0; j < nk; ++j) {
      const int c = (int)(((int64_t)j * blk) / T);
      const float sv = s[r * nk + j];
      float mv;
      if (c >= C) {
        mv = INFINITY;
      } else if (covered[b * nq + i]) {
        const float ao = alpha * overlap[(b * nq + i) * (int64_t)C + c];
        const float lt = (float)log1p((double)ao);
        mv = sv + lt;
      } else {
        mv = sv;
      }
      m[r * nk + j] = (double)mv;
    }
  }
  return 0;
}

/* Frustum-slice overlap (the article, Deep analysis, first and third steps:
 * each past chunk is a camera frustum slice with a depth interval; the
 * router asks which past slices overlap the region being drawn).  The
 * article gives no geometry; the reading used here: chunk c sees the
 * horizontal angles yaw_c +- fov/2 and depths [near_c, far_c]; query block
 * i is the i-th of nq equal angular strips of the current view (yaw_C) with
 * depths [qnear_i, qfar_i]; the overlap is the covered fraction of the
 * strip's angle times the covered fraction of its depth interval:
 *   O[b,i,c] = |strip_i ∩ (rel_c +- fov/2)| / |strip_i| *
 *              |[qnear_i, qfar_i] ∩ [near_c, far_c]| / max(qfar_i - qnear_i, 1e-12)
 * with rel_c = yaw_c - yaw_C wrapped to (-180, 180] and strip_i =
 * [-fov/2 + fov*i/nq, -fov/2 + fov*(i+1)/nq]; covered[b,i] = (O[b,i,c] > 0
 * for some c).  Inputs: yaw [B, C+1], past_depth [B, C, 2], query_depth
 * [B, nq, 2] (float32, widened exactly); fp64 throughout. */
int velox_oracle_frustum_overlap(const float *yaw, const float *past_depth, const float *query_depth, double fov,
                                 int B, int nq, int C, double *overlap, uint8_t *covered) {
  if (!yaw || !query_depth || !covered || (C > 0 && (!past_depth || !overlap)) || B < 0 || nq < 1 || C < 0 ||
      !(fov > 0.0))
    return -1;
  const double half = fov / 2.0;
  for (int b = 0; b < B; ++b) {
    const double ycur = yaw[(int64_t)b * (C + 1) + C];
    for (int i = 0; i < nq; ++i) {
      const double s0 = -half + fov * i / nq, s1 = -half + fov * (i + 1) / nq;
      const double q0 = query_depth[((int64_t)b * nq + i) * 2], q1 = query_depth[((int64_t)b * nq + i) * 2 + 1];
      const double qlen = fmax(q1 - q0, 1e-12);
      int any = 0;
      for (int c = 0; c < C; ++c) {
        double rel = fmod((double)yaw[(int64_t)b * (C + 1) + c] - ycur + 180.0, 360.0);
        if (rel < 0.0) rel += 360.0;
        rel -= 180.0;
        if (rel == -180.0) rel = 180.0;
        const double ang = fmax(0.0, fmin(s1, rel + half) - fmax(s0, rel - half)) / (s1 - s0);
        const double n0 = past_depth[((int64_t)b * C + c) * 2], n1 = past_depth[((int64_t)b * C + c) * 2 + 1];
        const double dep = fmax(0.0, fmin(q1, n1) - fmax(q0, n0)) / qlen;
        const double o = ang * dep;
        overlap[((int64_t)b * nq + i) * C + c] = o;
        any |= o > 0.0;
      }
      covered[(int64_t)b * nq + i] = (uint8_t)any;
    }
  }
  return 0;
}

typedef struct {
  double m;
  int j;
} scored;

/* Strict order: larger m first; equal m (including -0 == +0 and equal
 * infinities) -> lower block index first. */
static int by_m_desc_then_j(const void *pa, const void *pb) {
  const scored *a = (const scored *)pa, *b = (const scored *)pb;
  if (a->m > b->m) return -1;
  if (a->m < b->m) return 1;
  return (a->j > b->j) - (a->j < b->j);
}

/* Per row keep the first k_eff = min(k, nk) blocks of the strict order,
 * written in ascending block index; entries past k_eff are -1.
 * kv_idx: [rows, k]; kv_cnt: [rows]; kth (optional): [rows] = m of the
 * k_eff-th kept block (the selection threshold used by the gap rule). */
int velox_oracle_select(const double *m, int64_t rows, int nk, int k, int32_t *kv_idx, int32_t *kv_cnt,
                        double *kth) {
  if (!m || !kv_idx || !kv_cnt || rows < 0 || nk < 1 || k < 1) return -1;
  const int keff = k < nk ? k : nk;
  int fail = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : fail)
  for (int64_t r = 0; r < rows; ++r) {
    scored *order = (scored *)malloc(sizeof(scored) * (size_t)nk);
    unsigned char *kept = (unsigned char *)calloc((size_t)nk, 1);
    if (!order || !kept) {
      free(order);
      free(kept);
      fail = 1;
      continue;
    }
    for (int j = 0; j < nk; ++j) {
      order[j].m = m[r * nk + j];
      order[j].j = j;
    }
    qsort(order, (size_t)nk, sizeof(scored), by_m_desc_then_j);
    for (int t = 0; t < keff; ++t) kept[order[t].j] = 1;
    if (kth) kth[r] = order[keff - 1].m;
    int n = 0;
    for (int j = 0; j < nk; ++j)
      if (kept[j]) kv_idx[r * k + n++] = j;
    for (; n < k; ++n) kv_idx[r * k + n] = -1;
    kv_cnt[r] = keff;
    free(order);
    free(kept);
  }
  return fail ? -2 : 0;
}

/* Softmax attention of listed query tokens over the tokens of their row's
 * kept KV blocks.
 *   q: [B,H,T,d]; k, v: [B,H,N,d]; kv_idx: [B,H,T/blk,kmax]; kv_cnt: [B,H,T/blk]
 *   tok: flat token indices f = (b*H + h)*T + t (NULL = all B*H*T tokens
 *        in order, ntok must then equal B*H*T)
 *   out: [ntok, d]; lse (optional): [ntok]
 * For a token t of query block i = t / blk, with U the union of the kept
 * blocks' tokens: l_u = <q_t, k_u>/sqrt(d), M = max l_u, w_u = exp(l_u - M),
 * out = sum w_u v_u / sum w_u, lse = M + log(sum w_u).  No causal mask.
 * Lists follow the library's contract for caller-made lists: the first
 * min(max(kv_cnt, 0), kmax) entries are read and an entry outside
 * [0, N/blk) names no block and is skipped; a row left with no block gets
 * out = 0 and lse = -inf. */
int velox_oracle_attn(const void *q, const void *k, const void *v, int dtype, int B, int H, int T, int64_t N,
                      int d, int blk, const int32_t *kv_idx, const int32_t *kv_cnt, int kmax, int64_t ntok,
                      const int64_t *tok, double *out, double *lse) {
  if (!q || !k || !v || !kv_idx || !kv_cnt || !out || B < 0 || H < 0 || d < 1 || blk < 1 || T % blk)
    return -1;
  if (!tok && ntok != (int64_t)B * H * T) return -1;
  if (kmax < 1 || N % blk) return -1;
  const int nq = T / blk;
  const int64_t nkb = N / blk;
  const double scale = 1.0 / sqrt((double)d);
  int fail = 0;
#pragma omp parallel for schedule(dynamic, 8) reduction(| : fail)
  for (int64_t n = 0; n < ntok; ++n) {
    const int64_t f = tok ? tok[n] : n;
    const int64_t bh = f / T;
    const int t = (int)(f % T);
    const int64_t row = bh * nq + t / blk;
    const int cnt = kv_cnt[row] < 0 ? 0 : (kv_cnt[row] > kmax ? kmax : kv_cnt[row]);
    const int32_t *list = kv_idx + row * kmax;
    double *logit = (double *)malloc(sizeof(double) * (size_t)(cnt > 0 ? cnt : 1) * blk);
    if (!logit) {
      fail = 1;
      continue;
    }
    double M = -INFINITY;
    for (int c = 0; c < cnt; ++c) {
      if (list[c] < 0 || list[c] >= nkb) continue;
      for (int u = 0; u < blk; ++u) {
        const int64_t key = (int64_t)list[c] * blk + u;
        double dot = 0.0;
        for (int e = 0; e < d; ++e) dot += elem(q, dtype, f * d + e) * elem(k, dtype, (bh * N + key) * d + e);
        logit[c * blk + u] = dot * scale;
        if (logit[c * blk + u] > M) M = logit[c * blk + u];
      }
    }
    double wsum = 0.0;
    for (int e = 0; e < d; ++e) out[n * d + e] = 0.0;
    for (int c = 0; c < cnt; ++c) {
      if (list[c] < 0 || list[c] >= nkb) continue;
      for (int u = 0; u < blk; ++u) {
        const int64_t key = (int64_t)list[c] * blk + u;
        const double w = exp(logit[c * blk + u] - M);
        wsum += w;
        for (int e = 0; e < d; ++e) out[n * d + e] += w * elem(v, dtype, (bh * N + key) * d + e);
      }
    }
    if (wsum > 0.0)
      for (int e = 0; e < d; ++e) out[n * d + e] /= wsum;
    if (lse) lse[n] = wsum > 0.0 ? M + log(wsum) : -INFINITY;
    free(logit);
  }
  return fail ? -2 : 0;
}

/* Brute-force dense softmax attention of every query token over all N keys
 * (self-check reference for the keep-all case).  out: [B,H,T,d]; lse: [B,H,T]. */
int velox_oracle_dense_attn(const void *q, const void *k, const void *v, int dtype, int B, int H, int T,
                            int64_t N, int d, double *out, double *lse) {
  if (!q || !k || !v || !out || B < 0 || H < 0 || T < 0 || N < 1 || d < 1) return -1;
  const double scale = 1.0 / sqrt((double)d);
  int fail = 0;
#pragma omp parallel for schedule(dynamic, 8) reduction(| : fail)
  for (int64_t f = 0; f < (int64_t)B * H * T; ++f) {
    const int64_t bh = f / T;
    double *logit = (double *)malloc(sizeof(double) * (size_t)N);
    if (!logit) {
      fail = 1;
      continue;
    }
    double M = -INFINITY;
    for (int64_t u = 0; u < N; ++u) {
      double dot = 0.0;
      for (int e = 0; e < d; ++e) dot += elem(q, dtype, f * d + e) * elem(k, dtype, (bh * N + u) * d + e);
      logit[u] = dot * scale;
      if (logit[u] > M) M = logit[u];
    }
    double wsum = 0.0;
    for (int e = 0; e < d; ++e) out[f * d + e] = 0.0;
    for (int64_t u = 0; u < N; ++u) {
      const double w = exp(logit[u] - M);
      wsum += w;
      for (int e = 0; e < d; ++e) out[f * d + e] += w * elem(v, dtype, (bh * N + u) * d + e);
    }
    for (int e = 0; e < d; ++e) out[f * d + e] /= wsum;
    if (lse) lse[f] = M + log(wsum);
    free(logit);
  }
  return fail ? -2 : 0;
}
