/*
 * csa_oracle.c -- plain, slow, fp64 CPU reference for the CSA / HCA hybrid
 * compressed attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * Sources (cited by page and section; the pages have no code for this path):
 *   [shareware]  shareware.cn, "DeepSeek V4 Hybrid Attention" architecture
 *                article, sections 一 .. 十六
 *   [trdm]       trdm.cn, "从 MLA 到 CSA，聊聊大模型 Attention 的瘦身与闪送",
 *                sections 2.1 (MQA), 3.1 (Flash), 4.2 (DSA), 4.3 (V4 Hybrid)
 *   [aimodeling] aimodeling.com news item on V4 hybrid attention at 1M tokens
 *                (the CSA and HCA paragraphs)
 *   [tomwong]    tomwong001.github.io notes, section 一 (the MHA formula)
 *
 * Every floating-point quantity is accumulated in double.  Storage-precision
 * inputs (bf16 / fp32) convert to double exactly, so the only rounding here is
 * fp64 rounding.  Readings of points the pages leave open are marked READING.
 *
 * Parallelism: OpenMP over independent output units only (entries, queries);
 * it does not change the arithmetic of any unit.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Entry counts and causal visibility                                        */
/* ------------------------------------------------------------------------ */

/* Number of compressed entries for n tokens merged m at a time.
 * [shareware] 二: CSA maps n -> n/4, HCA maps n -> n/128; section 三.3 gives
 * 1,000,000 / 128 ~ 7813.  READING: a trailing partial block still yields an
 * entry (ceil), which is what makes the 7813 figure come out. */
int64_t oracle_num_entries(int64_t n, int64_t m) { return (n + m - 1) / m; }

/* Number of compressed entries visible to the query at position t.
 * [shareware] 十: a query may read only blocks that lie strictly before it and
 * are already complete.  Block s covers tokens [s*m, (s+1)*m); it is complete
 * and strictly earlier iff its last token (s+1)*m - 1 < t, i.e. (s+1)*m <= t. */
int64_t oracle_num_visible(int64_t t, int64_t m) { return t / m; }

/* ------------------------------------------------------------------------ */
/* Block-weighted compression                                                 */
/* ------------------------------------------------------------------------ */

/* One compressed entry is, per channel c, a softmax-weighted sum of the raw
 * rows of its block; the weights are dynamic (token dependent) and per
 * dimension ([shareware] 四).  The learned logits are the input z (same shape
 * as x).  Two-path ([shareware] 五; [trdm] 4.3 改进二): the current block is
 * read through stream A (x_a, z_a) and the previous block through stream B
 * (x_b, z_b); both compete in one joint softmax per channel.  Optional
 * additive per-position logit bias (READING of the position biases of
 * [trdm] 4.3 改进二): bias[span][D] with span = m for one path, 2m for two;
 * rows 0..m-1 belong to the B-path positions and rows m..2m-1 to the A path.
 *
 * Raw arrays are [B][n_raw][D] holding positions p0 .. p0+n_raw-1 of a
 * sequence of n tokens.  Entries e0 .. e1-1 are produced into out[B][e1-e0][D].
 * READING (partial block): the softmax runs over the tokens present.
 * Returns 0 on success, -1 when a needed raw row is not held. */
int oracle_compress(const double *x_a, const double *z_a, const double *x_b,
                    const double *z_b, const double *bias, int64_t B, int64_t n,
                    int64_t D, int64_t m, int64_t p0, int64_t n_raw, int64_t e0,
                    int64_t e1, double *out) {
  const int two_path = (x_b != NULL);
  const int64_t ne = e1 - e0;
  if (ne < 0) return -1;
  for (int64_t j = e0; j < e1; ++j) {
    int64_t lo = j * m;
    int64_t hi = (j + 1) * m < n ? (j + 1) * m : n;
    if (two_path && j >= 1) lo = (j - 1) * m;
    if (lo < p0 || hi > p0 + n_raw) return -1;
  }
  int err = 0;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t jj = 0; jj < ne; ++jj) {
      const int64_t j = e0 + jj;
      const int64_t a_lo = j * m;
      const int64_t a_hi = (j + 1) * m < n ? (j + 1) * m : n;
      const int64_t b_lo = (two_path && j >= 1) ? (j - 1) * m : 0;
      const int64_t b_hi = (two_path && j >= 1) ? j * m : 0;
      const int64_t cap = 2 * m;
      double *lg = (double *)malloc(sizeof(double) * cap);
      double *val = (double *)malloc(sizeof(double) * cap);
      if (!lg || !val) {
        err = 1;
        free(lg);
        free(val);
        continue;
      }
      for (int64_t c = 0; c < D; ++c) {
        int64_t cnt = 0;
        /* stream B: previous block, bias rows 0..m-1 */
        for (int64_t u = b_lo; u < b_hi; ++u) {
          const int64_t r = (b * n_raw + (u - p0)) * D + c;
          double l = z_b[r];
          if (bias) l += bias[(u - b_lo) * D + c];
          lg[cnt] = l;
          val[cnt] = x_b[r];
          ++cnt;
        }
        /* stream A: current block; bias rows m..2m-1 for two-path, 0..m-1 else */
        for (int64_t u = a_lo; u < a_hi; ++u) {
          const int64_t r = (b * n_raw + (u - p0)) * D + c;
          double l = z_a[r];
          if (bias) l += bias[((two_path ? m : 0) + (u - a_lo)) * D + c];
          lg[cnt] = l;
          val[cnt] = x_a[r];
          ++cnt;
        }
        /* softmax over the candidates, then the weighted sum */
        double mx = -INFINITY;
        for (int64_t i = 0; i < cnt; ++i)
          if (lg[i] > mx) mx = lg[i];
        double den = 0.0;
        for (int64_t i = 0; i < cnt; ++i) den += exp(lg[i] - mx);
        double acc = 0.0;
        for (int64_t i = 0; i < cnt; ++i) acc += exp(lg[i] - mx) / den * val[i];
        out[(b * ne + jj) * D + c] = acc;
      }
      free(lg);
      free(val);
    }
  }
  return err ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Lightning Indexer scores                                                   */
/* ------------------------------------------------------------------------ */

/* I(t, s) = sum_h w[t][h] * max(0, q_I[t][h] . k_I[s]) for visible s.
 * [shareware] 六-七: few heads, small head dim, per-head ReLU before the
 * sum over heads (the 8 / -7 example).  [trdm] 4.2: relu(q_idx . k_idx) with
 * the index key shared by all indexer heads and no softmax or scale.
 * READING: w is an optional per-query head weight, 1 when NULL.
 * q [B][T][HI][dI], w [B][T][HI], k [B][L][dI], tpos[T] query positions.
 * scores [B][T][L]; entries that are not visible are -inf. */
void oracle_index_scores(const double *q, const double *w, const double *k,
                         int64_t B, int64_t T, const int64_t *tpos, int64_t L,
                         int64_t HI, int64_t dI, int64_t m, double *scores) {
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t t = 0; t < T; ++t) {
      int64_t nv = oracle_num_visible(tpos[t], m);
      if (nv > L) nv = L;
      double *row = scores + (b * T + t) * L;
      for (int64_t s = 0; s < L; ++s) {
        if (s >= nv) {
          row[s] = -INFINITY;
          continue;
        }
        const double *ks = k + (b * L + s) * dI;
        double tot = 0.0;
        for (int64_t h = 0; h < HI; ++h) {
          const double *qh = q + ((b * T + t) * HI + h) * dI;
          double dot = 0.0;
          for (int64_t c = 0; c < dI; ++c) dot += qh[c] * ks[c];
          const double r = dot > 0.0 ? dot : 0.0;
          const double wh = w ? w[(b * T + t) * HI + h] : 1.0;
          tot += wh * r;
        }
        row[s] = tot;
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Top-k selection                                                            */
/* ------------------------------------------------------------------------ */

typedef struct {
  double v;
  int64_t s;
} scored_t;

/* Order: higher score first; equal scores (and -0 == +0) by lower index. */
static int by_score_then_index(const void *pa, const void *pb) {
  const scored_t *a = (const scored_t *)pa, *b = (const scored_t *)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->s < b->s) ? -1 : (a->s > b->s);
}

static int by_index(const void *pa, const void *pb) {
  const int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  return (a > b) - (a < b);
}

/* For each of R rows keep the min(k, nvis[r]) highest scores among the
 * first nvis[r] entries ([shareware] 六: score, then keep the top-k; the
 * aimodeling CSA paragraph: 1024 entries per query).  Ordering by
 * (score desc, index asc) is a stable sort by score of the index-ordered row,
 * so equal scores go to the lower index.  The kept indices are written in
 * ascending order; the remaining slots are -1.  Scores must not be NaN. */
void oracle_topk(const double *scores, const int64_t *nvis, int64_t R, int64_t L,
                 int64_t k, int32_t *idx) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < R; ++r) {
    int64_t nv = nvis[r] < L ? nvis[r] : L;
    if (nv < 0) nv = 0;
    scored_t *tmp = (scored_t *)malloc(sizeof(scored_t) * (nv > 0 ? nv : 1));
    for (int64_t s = 0; s < nv; ++s) {
      tmp[s].v = scores[r * L + s];
      tmp[s].s = s;
    }
    qsort(tmp, (size_t)nv, sizeof(scored_t), by_score_then_index);
    const int64_t keep = nv < k ? nv : k;
    int32_t *o = idx + r * k;
    for (int64_t i = 0; i < keep; ++i) o[i] = (int32_t)tmp[i].s;
    qsort(o, (size_t)keep, sizeof(int32_t), by_index);
    for (int64_t i = keep; i < k; ++i) o[i] = -1;
    free(tmp);
  }
}

/* ------------------------------------------------------------------------ */
/* Attention with a sink over a list of rows                                  */
/* ------------------------------------------------------------------------ */

/* MQA ([trdm] 2.1; [shareware] 十一): all H query heads read one shared K/V.
 * Per head: logits l_i = scale * q . key_i, plus a sink logit sigma_h with no
 * value vector ([shareware] 十二); the sink takes part in the normalisation
 * only.  out = sum_i softmax_i * val_i; lse = log(exp(sigma) + sum exp(l_i)).
 * A NULL sink means sigma = -inf (plain softmax, [tomwong] 一).
 * rows: nr pointers to key rows and nr to value rows, each d long. */
static void attend_rows(const double *qv, int64_t H, int64_t d,
                        const double *const *krow, const double *const *vrow,
                        int64_t nr, const double *sink, double scale,
                        double *out, double *lse, double *lg) {
  for (int64_t h = 0; h < H; ++h) {
    const double *qh = qv + h * d;
    const double sig = sink ? sink[h] : -INFINITY;
    double mx = sig;
    for (int64_t i = 0; i < nr; ++i) {
      double dot = 0.0;
      for (int64_t c = 0; c < d; ++c) dot += qh[c] * krow[i][c];
      lg[i] = scale * dot;
      if (lg[i] > mx) mx = lg[i];
    }
    double *oh = out + h * d;
    for (int64_t c = 0; c < d; ++c) oh[c] = 0.0;
    if (mx == -INFINITY) { /* no rows and no sink: empty softmax */
      if (lse) lse[h] = -INFINITY;
      continue;
    }
    double den = (sig == -INFINITY) ? 0.0 : exp(sig - mx);
    for (int64_t i = 0; i < nr; ++i) den += exp(lg[i] - mx);
    for (int64_t i = 0; i < nr; ++i) {
      const double p = exp(lg[i] - mx) / den;
      for (int64_t c = 0; c < d; ++c) oh[c] += p * vrow[i][c];
    }
    if (lse) lse[h] = mx + log(den);
  }
}

/* Sliding window rows for query position t: raw tokens
 * max(0, t-W+1) .. t ([shareware] 三.1 keeps the last 128 raw tokens; 十:
 * the window covers the same-block history that compressed entries cannot).
 * READING: the window ends at and includes t.  Raw rows kr/vr [B][R][d] hold
 * positions n_ctx-R .. n_ctx-1.  Returns the number of rows appended, or -1 if
 * a needed position is not held. */
static int64_t window_rows(const double *kr, const double *vr, int64_t b,
                           int64_t R, int64_t n_ctx, int64_t W, int64_t t,
                           int64_t d, const double **kp, const double **vp) {
  if (W <= 0) return 0;
  int64_t lo = t - W + 1;
  if (lo < 0) lo = 0;
  const int64_t base = n_ctx - R;
  int64_t cnt = 0;
  for (int64_t u = lo; u <= t; ++u) {
    if (u < base || u >= n_ctx) return -1;
    kp[cnt] = kr + (b * R + (u - base)) * d;
    vp[cnt] = vr + (b * R + (u - base)) * d;
    ++cnt;
  }
  return cnt;
}

/* CSA main attention ([shareware] 六 flow: score -> top-k -> exact attention;
 * [trdm] 4.3 改进三: the selected compressed entries are concatenated with the
 * uncompressed window).  READING: rows are the kept entries (idx != -1) then
 * the window rows, with no de-duplication.
 * q [B][T][H][d]; kc, vc [B][L][d]; idx [B][T][k]; out [B][T][H][d];
 * lse [B][T][H] (may be NULL); tpos[T] query positions.
 * Returns 0, or -1 on a bad index / window position. */
int oracle_sparse_attn(const double *q, const double *kc, const double *vc,
                       int64_t L, const int32_t *idx, int64_t k,
                       const double *kr, const double *vr, int64_t R, int64_t W,
                       const double *sink, double scale, int64_t B, int64_t T,
                       const int64_t *tpos, int64_t n_ctx, int64_t H, int64_t d,
                       double *out, double *lse) {
  int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t t = 0; t < T; ++t) {
      const int64_t cap = k + (W > 0 ? W : 0);
      const double **kp = (const double **)malloc(sizeof(double *) * (cap + 1));
      const double **vp = (const double **)malloc(sizeof(double *) * (cap + 1));
      double *lg = (double *)malloc(sizeof(double) * (cap + 1));
      int64_t nr = 0;
      for (int64_t j = 0; j < k; ++j) {
        const int32_t s = idx[(b * T + t) * k + j];
        if (s < 0) continue;
        if (s >= L) {
          err = 1;
          continue;
        }
        kp[nr] = kc + (b * L + s) * d;
        vp[nr] = vc + (b * L + s) * d;
        ++nr;
      }
      const int64_t nw = window_rows(kr, vr, b, R, n_ctx, W, tpos[t], d,
                                     kp + nr, vp + nr);
      if (nw < 0) err = 1;
      else nr += nw;
      attend_rows(q + (b * T + t) * H * d, H, d, kp, vp, nr, sink, scale,
                  out + (b * T + t) * H * d, lse ? lse + (b * T + t) * H : NULL,
                  lg);
      free(kp);
      free(vp);
      free(lg);
    }
  }
  return err ? -1 : 0;
}

/* HCA attention: dense over every visible compressed entry, no indexer and no
 * top-k ([shareware] 八; the aimodeling HCA paragraph), plus the optional raw
 * window ([trdm] 4.3, HCA paragraph).  Visibility as oracle_num_visible. */
int oracle_dense_attn(const double *q, const double *kc, const double *vc,
                      int64_t L, int64_t m, const double *kr, const double *vr,
                      int64_t R, int64_t W, const double *sink, double scale,
                      int64_t B, int64_t T, const int64_t *tpos, int64_t n_ctx,
                      int64_t H, int64_t d, double *out, double *lse) {
  int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t t = 0; t < T; ++t) {
      int64_t nv = oracle_num_visible(tpos[t], m);
      if (nv > L) nv = L;
      const int64_t cap = nv + (W > 0 ? W : 0);
      const double **kp = (const double **)malloc(sizeof(double *) * (cap + 1));
      const double **vp = (const double **)malloc(sizeof(double *) * (cap + 1));
      double *lg = (double *)malloc(sizeof(double) * (cap + 1));
      int64_t nr = 0;
      for (int64_t s = 0; s < nv; ++s) {
        kp[nr] = kc + (b * L + s) * d;
        vp[nr] = vc + (b * L + s) * d;
        ++nr;
      }
      const int64_t nw = window_rows(kr, vr, b, R, n_ctx, W, tpos[t], d,
                                     kp + nr, vp + nr);
      if (nw < 0) err = 1;
      else nr += nw;
      attend_rows(q + (b * T + t) * H * d, H, d, kp, vp, nr, sink, scale,
                  out + (b * T + t) * H * d, lse ? lse + (b * T + t) * H : NULL,
                  lg);
      free(kp);
      free(vp);
      free(lg);
    }
  }
  return err ? -1 : 0;
}
