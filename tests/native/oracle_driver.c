/*
 * Sanitizer driver for the CPU oracle (built with -fsanitize=address,undefined by
 * tests/test_sanitizers.py).  Calls every oracle function on small seeded inputs,
 * edge cases included (empty sets, k above the visible count, masked slots, window 0,
 * first block), and checks properties that hold at any size, so that a run is both a
 * memory/UB check and a light self-test.  Exit status: 0 = all checks passed.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static unsigned long long g_state = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*, uniform in [0, 1) */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (double)((g_state * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0);
}
static double nrand(void) { return (urand() + urand() + urand() + urand() - 2.0) * 1.7; }
static double* vec(long n) {
  double* p = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (long i = 0; i < n; ++i) p[i] = nrand();
  return p;
}

static int g_fail = 0;
#define CHECK(cond, ...)                    \
  do {                                      \
    if (!(cond)) {                          \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");                \
      g_fail = 1;                           \
    }                                       \
  } while (0)

static void t_compress(void) {
  const int cs[3] = {1, 3, 8}, ms[3] = {1, 2, 4};
  for (int ci = 0; ci < 3; ++ci)
    for (int mi = 0; mi < 3; ++mi)
      for (int zmode = 0; zmode < 2; ++zmode)
        for (int bias = 0; bias < 2; ++bias) {
          const int c = cs[ci], m = ms[mi], zc = zmode ? c : 1;
          const long n_rows = 5 * m, tok_base = 0, e0 = 0, e1 = 5;
          double *A = vec(n_rows * c), *B = vec(n_rows * c), *za = vec(n_rows * zc), *zb = vec(n_rows * zc);
          double *ba = bias ? vec((long)m * zc) : NULL, *bb = bias ? vec((long)m * zc) : NULL;
          double* out = (double*)malloc(sizeof(double) * (size_t)(e1 - e0) * c);
          int rc = oracle_compress(A, B, za, zb, ba, bb, tok_base, n_rows, c, m, zc, e0, e1, out);
          CHECK(rc == 0, "compress rc %d (c %d m %d zc %d)", rc, c, m, zc);
          /* each output is a convex combination of the 2m rows it pools */
          for (long j = e0; j < e1 && rc == 0; ++j)
            for (int ch = 0; ch < c; ++ch) {
              double lo = INFINITY, hi = -INFINITY;
              for (long u = m * j; u < m * (j + 1); ++u) {
                lo = fmin(lo, A[u * c + ch]);
                hi = fmax(hi, A[u * c + ch]);
              }
              for (long u = m * (j - 1); j > 0 && u < m * j; ++u) {
                lo = fmin(lo, B[u * c + ch]);
                hi = fmax(hi, B[u * c + ch]);
              }
              double v = out[(j - e0) * c + ch];
              CHECK(isfinite(v) && v >= lo - 1e-12 && v <= hi + 1e-12, "compress entry %ld ch %d outside its rows", j, ch);
            }
          /* rows that do not cover the entries, and bad shapes, are rejected */
          CHECK(oracle_compress(A, B, za, zb, ba, bb, 1, n_rows - 1, c, m, zc, e0, e1, out) != 0, "compress coverage");
          CHECK(oracle_compress(A, B, za, zb, ba, bb, 0, n_rows, c, 0, zc, e0, e1, out) != 0, "compress m 0");
          free(A); free(B); free(za); free(zb); free(ba); free(bb); free(out);
        }
}

static void t_rmsnorm_visible(void) {
  double* x = vec(4 * 16);
  double* y = (double*)malloc(sizeof(double) * 64);
  oracle_rmsnorm(x, 4, 16, NULL, 0.0, y);
  for (int r = 0; r < 4; ++r) {
    double ms = 0.0;
    for (int i = 0; i < 16; ++i) ms += y[r * 16 + i] * y[r * 16 + i];
    CHECK(fabs(ms / 16.0 - 1.0) < 1e-12, "rmsnorm mean square %g", ms / 16.0);
  }
  free(x); free(y);
  for (long t = -3; t < 40; ++t)
    for (int m = 1; m <= 5; ++m) {
      long v = oracle_visible(t, 7, m);
      CHECK(v >= 0 && v <= 7 && (t < 0 || v == ((t + 1) / m < 7 ? (t + 1) / m : 7)), "visible t %ld m %d", t, m);
    }
}

static void t_index_topk(void) {
  const int H = 4, d = 8;
  const long n = 37;
  double *q = vec(H * d), *K = vec(n * d), *w = (double*)malloc(sizeof(double) * H);
  for (int h = 0; h < H; ++h) w[h] = urand();
  double* sc = (double*)malloc(sizeof(double) * n);
  oracle_index_scores(q, w, K, H, d, n, sc);
  for (long s = 0; s < n; ++s) CHECK(isfinite(sc[s]) && sc[s] >= 0.0, "index score %ld", s);
  sc[3] = sc[5]; /* a tie */
  const long Vs[4] = {0, 1, 20, 37};
  const int ks[4] = {1, 8, 37, 50};
  for (int a = 0; a < 4; ++a)
    for (int b = 0; b < 4; ++b) {
      int32_t* out = (int32_t*)malloc(sizeof(int32_t) * (size_t)ks[b]);
      oracle_topk(sc, Vs[a], ks[b], out);
      const long take = Vs[a] < ks[b] ? Vs[a] : ks[b];
      for (int i = 0; i < ks[b]; ++i) {
        if (i >= take) {
          CHECK(out[i] == -1, "topk pad");
          continue;
        }
        CHECK(out[i] >= 0 && out[i] < Vs[a], "topk index range");
        for (int j = 0; j < i; ++j) CHECK(out[j] != out[i], "topk duplicate");
        if (i > 0) CHECK(sc[out[i - 1]] > sc[out[i]] || (sc[out[i - 1]] == sc[out[i]] && out[i - 1] < out[i]), "topk order");
      }
      free(out);
    }
  free(q); free(K); free(w); free(sc);
}

static void t_mqa(void) {
  const int H = 3, d = 16, m = 4;
  const long n_entries = 9, n_raw = 12, raw_base = 20;
  double *q = vec(H * d), *kv = vec(n_entries * d), *raw = vec(n_raw * d), *g = vec(d), *sink = vec(H);
  double* out = (double*)malloc(sizeof(double) * H * d);
  double* lse = (double*)malloc(sizeof(double) * H);
  const int32_t idx[6] = {4, -1, 0, 8, -1, 2};
  for (int win = 0; win <= 8; win += 4)
    for (int wg = 0; wg < 2; ++wg)
      for (int ws = 0; ws < 2; ++ws) {
        const long t = raw_base + n_raw - 1;
        int rc = oracle_sparse_mqa(q, kv, n_entries, idx, 6, raw, n_raw, raw_base, t, win, H, d, 0.25, 1e-6,
                                   wg ? g : NULL, ws ? sink : NULL, out, lse);
        CHECK(rc == 0, "sparse rc");
        for (int i = 0; i < H * d; ++i) CHECK(isfinite(out[i]), "sparse out finite");
        for (int h = 0; h < H; ++h) CHECK(isfinite(lse[h]), "sparse lse finite");
        rc = oracle_dense_mqa(q, kv, n_entries, m, raw, n_raw, raw_base, t, win, H, d, 0.25, 1e-6, wg ? g : NULL,
                              ws ? sink : NULL, out, lse);
        CHECK(rc == 0, "dense rc");
        for (int h = 0; h < H; ++h) CHECK(isfinite(lse[h]), "dense lse finite");
      }
  /* nothing to attend: zero output, lse -inf (or the sink alone) */
  const int32_t none[2] = {-1, -1};
  CHECK(oracle_sparse_mqa(q, kv, n_entries, none, 2, raw, n_raw, raw_base, raw_base, 0, H, d, 0.25, 1e-6, NULL, NULL,
                          out, lse) == 0, "empty rc");
  for (int h = 0; h < H; ++h) CHECK(isinf(lse[h]) && lse[h] < 0, "empty lse");
  CHECK(oracle_dense_mqa(q, kv, n_entries, m, raw, n_raw, raw_base, 2, 0, H, d, 0.25, 1e-6, NULL, sink, out, lse) == 0,
        "dense V=0 rc");
  for (int h = 0; h < H; ++h) CHECK(fabs(lse[h] - sink[h]) < 1e-12, "sink-only lse");
  /* slots and window rows outside their buffers are rejected */
  const int32_t bad[1] = {(int32_t)n_entries};
  CHECK(oracle_sparse_mqa(q, kv, n_entries, bad, 1, raw, n_raw, raw_base, raw_base, 1, H, d, 0.25, 1e-6, NULL, NULL,
                          out, lse) != 0, "bad slot");
  CHECK(oracle_dense_mqa(q, kv, n_entries, m, raw, n_raw, raw_base, raw_base + n_raw, 1, H, d, 0.25, 1e-6, NULL, NULL,
                         out, lse) != 0, "window past the raw rows");
  free(q); free(kv); free(raw); free(g); free(sink); free(out); free(lse);
}

static void t_formats_rope(void) {
  const long nb = 6;
  double* x = vec(nb * 32);
  for (int i = 0; i < 32; ++i) x[i] = 0.0;           /* an all-zero block */
  x[40] = 1e30; x[41] = -1e-30;                      /* a block with a huge range */
  uint8_t codes[6 * 16], scales[6];
  oracle_mxfp4_quantize(x, nb, codes, scales);
  double* y = (double*)malloc(sizeof(double) * nb * 32);
  oracle_mxfp4_dequantize(codes, scales, nb, y);
  for (long i = 0; i < nb * 32; ++i) CHECK(isfinite(y[i]), "mxfp4 finite");
  for (int i = 0; i < 32; ++i) CHECK(y[i] == 0.0, "mxfp4 zero block");
  uint8_t f8[64];
  double z[64], back[64];
  for (int i = 0; i < 64; ++i) z[i] = ldexp(nrand(), (i % 12) - 6);
  z[0] = 1e9; z[1] = -1e9; z[2] = 0.0;
  oracle_fp8_quantize(z, 64, f8);
  oracle_fp8_dequantize(f8, 64, back);
  CHECK(back[0] == 448.0 && back[1] == -448.0 && back[2] == 0.0, "fp8 saturation");
  for (int i = 3; i < 64; ++i)
    CHECK(fabs(back[i] - z[i]) <= fabs(z[i]) * 0.0625 + 1.0 / 1024.0, "fp8 roundtrip %d", i);
  const int H = 2, d = 80;
  double* o = vec(H * d);
  double* o0 = (double*)malloc(sizeof(double) * H * d);
  memcpy(o0, o, sizeof(double) * H * d);
  double cs[128];
  for (int p = 0; p < 32; ++p) {
    double a = 6.283185307179586 * urand();
    cs[2 * p] = cs[2 * p + 1] = cos(a);
    cs[64 + 2 * p] = cs[64 + 2 * p + 1] = sin(a);
  }
  oracle_rope_conjugate(o, H, d, cs);
  for (int h = 0; h < H; ++h) {
    for (int i = 0; i < d - 64; ++i) CHECK(o[h * d + i] == o0[h * d + i], "rope leaves the leading dims");
    for (int p = 0; p < 32; ++p) {
      const double* a = o + h * d + d - 64 + 2 * p;
      const double* b = o0 + h * d + d - 64 + 2 * p;
      CHECK(fabs(a[0] * a[0] + a[1] * a[1] - b[0] * b[0] - b[1] * b[1]) < 1e-12, "rope pair norm");
    }
  }
  free(x); free(y); free(o); free(o0);
}

int main(void) {
  t_compress();
  t_rmsnorm_visible();
  t_index_topk();
  t_mqa();
  t_formats_rope();
  if (!g_fail) printf("oracle driver: all checks passed\n");
  return g_fail;
}
