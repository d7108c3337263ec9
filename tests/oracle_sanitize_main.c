/*
 * Driver for a sanitizer build of the CPU oracle (test infrastructure).
 *
 * Built by tests/test_oracle_sanitizers.py with gcc and AddressSanitizer +
 * UndefinedBehaviorSanitizer, single-threaded (no OpenMP), together with
 * oracle/csa_oracle.c.  It calls every oracle entry point on small inputs that
 * reach its edge cases (a trailing partial block, two-path compression with a
 * position bias, the first entry without a stream-B block, queries with no
 * visible entry, k above the visible count, ties and signed zeros, -1 index
 * padding, a window reaching position 0, an empty row list with and without a
 * sink) and checks a few invariants, so that an out-of-bounds access, a leak
 * or undefined behaviour in the oracle ends the run with a report.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int64_t oracle_num_entries(int64_t n, int64_t m);
int64_t oracle_num_visible(int64_t t, int64_t m);
int oracle_compress(const double *x_a, const double *z_a, const double *x_b, const double *z_b,
                    const double *bias, int64_t B, int64_t n, int64_t D, int64_t m, int64_t p0,
                    int64_t n_raw, int64_t e0, int64_t e1, double *out);
void oracle_index_scores(const double *q, const double *w, const double *k, int64_t B, int64_t T,
                         const int64_t *tpos, int64_t L, int64_t HI, int64_t dI, int64_t m,
                         double *scores);
void oracle_topk(const double *scores, const int64_t *nvis, int64_t R, int64_t L, int64_t k,
                 int32_t *idx);
int oracle_sparse_attn(const double *q, const double *kc, const double *vc, int64_t L,
                       const int32_t *idx, int64_t k, const double *kr, const double *vr, int64_t R,
                       int64_t W, const double *sink, double scale, int64_t B, int64_t T,
                       const int64_t *tpos, int64_t n_ctx, int64_t H, int64_t d, double *out,
                       double *lse);
int oracle_dense_attn(const double *q, const double *kc, const double *vc, int64_t L, int64_t m,
                      const double *kr, const double *vr, int64_t R, int64_t W, const double *sink,
                      double scale, int64_t B, int64_t T, const int64_t *tpos, int64_t n_ctx,
                      int64_t H, int64_t d, double *out, double *lse);

static uint64_t state = 0x9e3779b97f4a7c15ull;

/* xorshift64*: a uniform draw in [-1, 1) (input values only). */
static double draw(void) {
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  const uint64_t r = state * 0x2545f4914f6cdd1dull;
  return (double)(r >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

static double *fill(size_t n, double scale) {
  double *p = (double *)malloc(sizeof(double) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) p[i] = scale * draw();
  return p;
}

static int failures = 0;
#define CHECK(c)                                            \
  do {                                                      \
    if (!(c)) {                                             \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                           \
    }                                                       \
  } while (0)

static void test_compress(void) {
  const int64_t B = 2, n = 19, D = 5, m = 4;
  const int64_t L = oracle_num_entries(n, m);
  CHECK(L == 5);
  double *xa = fill(B * n * D, 1.0), *za = fill(B * n * D, 2.0);
  double *xb = fill(B * n * D, 1.0), *zb = fill(B * n * D, 2.0);
  double *bias = fill(2 * m * D, 0.5);
  double *out = (double *)malloc(sizeof(double) * B * L * D);
  /* single path, then two-path with a bias, over whole sequences */
  CHECK(oracle_compress(xa, za, NULL, NULL, bias, B, n, D, m, 0, n, 0, L, out) == 0);
  CHECK(oracle_compress(xa, za, xb, zb, bias, B, n, D, m, 0, n, 0, L, out) == 0);
  for (int64_t i = 0; i < B * L * D; ++i) CHECK(isfinite(out[i]) && fabs(out[i]) <= 1.0);
  /* one entry from a window of raw rows (decode-time write) */
  const int64_t p0 = 8, nr = n - p0;
  CHECK(oracle_compress(xa + p0 * D, za + p0 * D, xb + p0 * D, zb + p0 * D, NULL, 1, n, D, m, p0, nr, 3,
                        4, out) == 0);
  /* raw rows that do not cover the entry are rejected, nothing read */
  CHECK(oracle_compress(xa, za, xb, zb, NULL, 1, n, D, m, 8, 4, 2, 3, out) == -1);
  free(xa), free(za), free(xb), free(zb), free(bias), free(out);
}

static void test_index_topk(void) {
  const int64_t B = 2, T = 3, L = 37, HI = 3, dI = 8, m = 4, k = 7;
  const int64_t tpos[3] = {2, 60, 147};  /* nothing visible, 15 visible, all 37 */
  double *q = fill(B * T * HI * dI, 1.0), *w = fill(B * T * HI, 1.0), *kk = fill(B * L * dI, 1.0);
  double *sc = (double *)malloc(sizeof(double) * B * T * L);
  oracle_index_scores(q, w, kk, B, T, tpos, L, HI, dI, m, sc);
  oracle_index_scores(q, NULL, kk, B, T, tpos, L, HI, dI, m, sc);
  int64_t nv[6];
  for (int64_t r = 0; r < B * T; ++r) {
    int64_t v = oracle_num_visible(tpos[r % T], m);
    nv[r] = v < L ? v : L;
  }
  /* ties and signed zeros: a coarse grid */
  for (int64_t r = 0; r < B * T; ++r)
    for (int64_t s = 0; s < nv[r]; ++s) sc[r * L + s] = floor(3.0 * draw());
  sc[4 * L + 1] = -0.0;
  int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * B * T * k);
  oracle_topk(sc, nv, B * T, L, k, idx);
  for (int64_t r = 0; r < B * T; ++r) {
    const int64_t keep = nv[r] < k ? nv[r] : k;
    for (int64_t i = 0; i < k; ++i) {
      if (i < keep) {
        CHECK(idx[r * k + i] >= 0 && idx[r * k + i] < nv[r]);
        if (i) CHECK(idx[r * k + i] > idx[r * k + i - 1]);
      } else {
        CHECK(idx[r * k + i] == -1);
      }
    }
  }
  /* a k larger than every row */
  int32_t *big = (int32_t *)malloc(sizeof(int32_t) * B * T * 64);
  oracle_topk(sc, nv, B * T, L, 64, big);
  free(big);
  free(q), free(w), free(kk), free(sc), free(idx);
}

static void test_attention(void) {
  const int64_t B = 2, T = 3, H = 4, d = 6, L = 9, k = 5, W = 4, m = 4, n_ctx = 40;
  const int64_t R = T + W - 1;
  const int64_t tpos[3] = {37, 38, 39};
  double *q = fill(B * T * H * d, 1.0), *kc = fill(B * L * d, 1.0), *vc = fill(B * L * d, 1.0);
  double *kr = fill(B * R * d, 1.0), *vr = fill(B * R * d, 1.0), *sink = fill(H, 1.0);
  int32_t idx[2 * 3 * 5];
  for (int i = 0; i < 30; ++i) idx[i] = (i % 3 == 2) ? -1 : (int32_t)(i % 9);
  double *out = (double *)malloc(sizeof(double) * B * T * H * d);
  double *lse = (double *)malloc(sizeof(double) * B * T * H);
  CHECK(oracle_sparse_attn(q, kc, vc, L, idx, k, kr, vr, R, W, sink, 0.4, B, T, tpos, n_ctx, H, d, out, lse) == 0);
  CHECK(oracle_sparse_attn(q, kc, vc, L, idx, k, kr, vr, R, W, NULL, 0.4, B, T, tpos, n_ctx, H, d, out, NULL) == 0);
  CHECK(oracle_dense_attn(q, kc, vc, L, m, kr, vr, R, W, sink, 0.4, B, T, tpos, n_ctx, H, d, out, lse) == 0);
  for (int64_t i = 0; i < B * T * H; ++i) CHECK(isfinite(lse[i]));
  /* an out-of-range index and a window position not held are rejected */
  idx[0] = 9;
  CHECK(oracle_sparse_attn(q, kc, vc, L, idx, k, kr, vr, R, W, sink, 0.4, B, T, tpos, n_ctx, H, d, out, lse) == -1);
  const int64_t early[3] = {30, 31, 32};
  CHECK(oracle_dense_attn(q, kc, vc, L, m, kr, vr, R, W, sink, 0.4, B, T, early, n_ctx, H, d, out, lse) == -1);
  /* no row at all: no visible entry, no window; with a sink the output is 0 */
  int32_t none[2 * 3 * 5];
  for (int i = 0; i < 30; ++i) none[i] = -1;
  CHECK(oracle_sparse_attn(q, kc, vc, L, none, k, NULL, NULL, 0, 0, sink, 0.4, B, T, tpos, n_ctx, H, d, out, lse) == 0);
  for (int64_t i = 0; i < B * T * H * d; ++i) CHECK(out[i] == 0.0);
  CHECK(oracle_sparse_attn(q, kc, vc, L, none, k, NULL, NULL, 0, 0, NULL, 0.4, B, T, tpos, n_ctx, H, d, out, lse) == 0);
  for (int64_t i = 0; i < B * T * H; ++i) CHECK(isinf(lse[i]) && lse[i] < 0);
  /* a window that reaches position 0 (t < W - 1) */
  const int64_t first[1] = {1};
  CHECK(oracle_dense_attn(q, kc, vc, L, m, kr, vr, 2, W, sink, 0.4, 1, 1, first, 2, H, d, out, lse) == 0);
  free(q), free(kc), free(vc), free(kr), free(vr), free(sink), free(out), free(lse);
}

int main(void) {
  test_compress();
  test_index_topk();
  test_attention();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle sanitizer run ok\n");
  return 0;
}
