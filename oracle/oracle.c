/*
 * CPU oracle for Compressed Sparse Attention (CSA) and Heavily Compressed
 * Attention (HCA): a plain, slow, single-threaded reference.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no source with the GPU library.
 *
 * Every value is carried in IEEE double.  Inputs arrive as doubles holding
 * the exact stored values (fp32, bf16 or dequantised MXFP4), so nothing is
 * rounded on the way in.  No blocking, fusion or reordering: each function is
 * the definition written out, loop by loop.
 *
 * Sources (web pages describing DeepSeek-V4):
 *  [P2] "DeepSeek-AI (2026) - ARXIV-2606.19348", anthology record, Key takeaways
 *       (two latent KV streams pooled over overlapping 2m windows; RMSNorm on
 *       every query head and on the single compressed KV head).
 *  [P3] "DeepSeek v4" (Korean summary), section "Compressed Sparse Attention",
 *       sub-parts on compressed KV entries and on the lightning indexer; and
 *       section on the hybrid CSA/HCA attention.
 *  [P4] "DeepSeek-V4-Pro" model techniques map, entries "Grouped-query
 *       attention", "Sliding-window attention", "Indexer-selected sparse
 *       attention", "QK normalization".
 *  [MX] OCP Microscaling Formats (MX) v1.0 specification, MXFP4 (e2m1 elements,
 *       e8m0 shared scale per block of 32) -- format named by the workload, the
 *       pages say only "FP4" ([P1] forum post "DeepSeek V4 paper full version is
 *       out", and [P4] "FP4 precision for the attention indexer").
 *
 * Readings taken where the pages are silent are listed beside each function.
 * Parity pins for every function live in the CPU test-suite; none is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

#define ORC_OK 0
#define ORC_EINVAL 1

/* ------------------------------------------------------------------------ */
/* Compression.  [P3] "Compressed Sparse Attention", compressed KV entries:
 * two series of token-level entries C_a, C_b with weights Z_a, Z_b and
 * learnable positional biases B_a, B_b; each compressed entry is a row-wise
 * softmax over 2m elements; for the first block the previous block's Z_b is
 * padded with -inf and C_b with 0; adjacent entries overlap, so the length
 * shrinks to 1/m.  [P2] Key takeaways: each entry pools an overlapping window
 * of 2m tokens drawn from two latent streams.
 *
 * Reading (not printed on the pages): entry j takes the A stream over tokens
 * [m*j, m*j+m) and the B stream over the previous block [m*(j-1), m*j); the
 * 2m logits are z + positional bias; weights s = softmax over those 2m logits
 * (per channel when zc == c, shared when zc == 1); C_j = sum s*row.
 *
 * Arrays hold token rows [tok_base, tok_base + n_rows):
 *   A, Bv   [n_rows, c]     za, zb [n_rows, zc]
 *   bias_a, bias_b [m, zc] or NULL (= 0)
 *   out     [entry_end - entry_begin, c]
 * ------------------------------------------------------------------------ */
int oracle_compress(const double* A, const double* Bv, const double* za, const double* zb,
                    const double* bias_a, const double* bias_b, long tok_base, long n_rows,
                    int c, int m, int zc, long entry_begin, long entry_end, double* out) {
  if (m < 1 || c < 1 || !(zc == 1 || zc == c) || entry_begin < 0 || entry_end < entry_begin)
    return ORC_EINVAL;
  double* logit = (double*)malloc(sizeof(double) * 2 * m);
  double* weight = (double*)malloc(sizeof(double) * 2 * m);
  for (long j = entry_begin; j < entry_end; ++j) {
    long a0 = (long)m * j;         /* first token of the A half */
    long b0 = (long)m * (j - 1);   /* first token of the B half (previous block) */
    if (a0 + m - tok_base > n_rows || a0 < tok_base || (j > 0 && b0 < tok_base)) {
      free(logit); free(weight);
      return ORC_EINVAL;
    }
    double* o = out + (j - entry_begin) * (long)c;
    for (int ch = 0; ch < c; ++ch) {
      int zi = (zc == 1) ? 0 : ch;
      for (int r = 0; r < m; ++r) {
        logit[r] = za[(a0 + r - tok_base) * zc + zi] + (bias_a ? bias_a[r * zc + zi] : 0.0);
        if (j > 0)
          logit[m + r] = zb[(b0 + r - tok_base) * zc + zi] + (bias_b ? bias_b[r * zc + zi] : 0.0);
        else
          logit[m + r] = -INFINITY;
      }
      double mx = -INFINITY;
      for (int r = 0; r < 2 * m; ++r) if (logit[r] > mx) mx = logit[r];
      double den = 0.0;
      for (int r = 0; r < 2 * m; ++r) {
        weight[r] = (logit[r] == -INFINITY) ? 0.0 : exp(logit[r] - mx);
        den += weight[r];
      }
      double acc = 0.0;
      for (int r = 0; r < m; ++r) acc += (weight[r] / den) * A[(a0 + r - tok_base) * c + ch];
      if (j > 0)
        for (int r = 0; r < m; ++r) acc += (weight[m + r] / den) * Bv[(b0 + r - tok_base) * c + ch];
      /* j == 0: the B half is padded with zero rows and weight 0. */
      o[ch] = acc;
    }
  }
  free(logit); free(weight);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm.  [P2] Key takeaways: an extra RMSNorm on each query head and on
 * the single compressed-KV head just before the core attention.  [P4] "QK
 * normalization": queries and kv pass through RMSNorm before the product.
 * x_hat = x * gamma / sqrt(mean(x^2) + eps), per row of length d.
 * ------------------------------------------------------------------------ */
void oracle_rmsnorm(const double* x, long rows, int d, const double* gamma, double eps, double* out) {
  for (long r = 0; r < rows; ++r) {
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss += x[r * d + i] * x[r * d + i];
    double inv = 1.0 / sqrt(ss / d + eps);
    for (int i = 0; i < d; ++i) out[r * d + i] = x[r * d + i] * inv * (gamma ? gamma[i] : 1.0);
  }
}

/* ------------------------------------------------------------------------ */
/* Causal visibility.  [P3] lightning indexer: scores are taken for the
 * preceding compressed blocks only; [P4] "Indexer-selected sparse attention":
 * indices at or past a per-query causal threshold are invalid.
 * Reading: only complete blocks exist; entry s (covering tokens up to
 * m*(s+1)-1) is visible to the query at absolute position t iff
 * m*(s+1)-1 <= t, so V(t) = min(N, floor((t+1)/m)).
 * ------------------------------------------------------------------------ */
long oracle_visible(long t, long n_entries, int m) {
  long v = (t + 1) / m;
  if (v > n_entries) v = n_entries;
  if (v < 0) v = 0;
  return v;
}

/* ------------------------------------------------------------------------ */
/* Lightning indexer score.  [P3] lightning indexer: for query t, several
 * indexer query heads; the score of a preceding compressed block s is the sum
 * over heads of a per-head weight times ReLU(q . K).  No scale (any positive
 * scale leaves the ranking unchanged).
 *   q [H_I, d_I], w [H_I], K [n, d_I]  ->  scores [n]
 * ------------------------------------------------------------------------ */
void oracle_index_scores(const double* q, const double* w, const double* K, int H_I, int d_I,
                         long n, double* scores) {
  for (long s = 0; s < n; ++s) {
    double total = 0.0;
    for (int h = 0; h < H_I; ++h) {
      double dot = 0.0;
      for (int i = 0; i < d_I; ++i) dot += q[(long)h * d_I + i] * K[s * d_I + i];
      total += w[h] * (dot > 0.0 ? dot : 0.0);
    }
    scores[s] = total;
  }
}

/* ------------------------------------------------------------------------ */
/* Top-k selector.  [P3] each query keeps only the top-k entries chosen by the
 * selector; [P4] "Indexer-selected sparse attention": index_topk entries,
 * invalid slots marked -1.  Reading of the order: score descending, ties by
 * lower index; take min(k, V) and pad with -1.
 * ------------------------------------------------------------------------ */
static const double* g_sort_scores; /* single-threaded by contract */
static int cmp_desc(const void* a, const void* b) {
  long i = *(const long*)a, j = *(const long*)b;
  double si = g_sort_scores[i], sj = g_sort_scores[j];
  if (si > sj) return -1;
  if (si < sj) return 1;
  return (i < j) ? -1 : (i > j);
}
void oracle_topk(const double* scores, long n_visible, int k, int32_t* out) {
  long* order = (long*)malloc(sizeof(long) * (n_visible > 0 ? n_visible : 1));
  for (long s = 0; s < n_visible; ++s) order[s] = s;
  g_sort_scores = scores;
  qsort(order, (size_t)n_visible, sizeof(long), cmp_desc);
  for (int i = 0; i < k; ++i) out[i] = (i < n_visible) ? (int32_t)order[i] : -1;
  free(order);
}

/* ------------------------------------------------------------------------ */
/* Core attention over an explicit set of rows.  [P4] "Grouped-query
 * attention": H query heads share one KV head (multi-query attention); the
 * compressed entry serves as both key and value.  One softmax over the whole
 * set (top-k entries and sliding-window tokens together).
 *   q [H, d] raw; rows [S, d] raw; RMSNorm applied here to both sides.
 *   out [H, d]; lse [H] (natural log of the softmax denominator incl. max).
 * [P4] "Learnable attention sink": a per-head sink logit is concatenated to
 * the logits before the softmax and its column dropped after, i.e. it adds
 * exp(sink[h]) to the denominator and nothing to the numerator.  sink [H] or
 * NULL.
 * ------------------------------------------------------------------------ */
static void attend(const double* q, const double* const* rows, long S, int H, int d,
                   double scale, double eps, const double* gamma, const double* sink, double* out,
                   double* lse) {
  double* qn = (double*)malloc(sizeof(double) * d);
  double* kn = (double*)malloc(sizeof(double) * (S > 0 ? S : 1) * d);
  double* logit = (double*)malloc(sizeof(double) * (S > 0 ? S : 1));
  for (long j = 0; j < S; ++j) oracle_rmsnorm(rows[j], 1, d, gamma, eps, kn + j * d);
  for (int h = 0; h < H; ++h) {
    oracle_rmsnorm(q + (long)h * d, 1, d, gamma, eps, qn);
    double mx = -INFINITY;
    for (long j = 0; j < S; ++j) {
      double dot = 0.0;
      for (int i = 0; i < d; ++i) dot += qn[i] * kn[j * d + i];
      logit[j] = scale * dot;
      if (logit[j] > mx) mx = logit[j];
    }
    if (sink && sink[h] > mx) mx = sink[h];
    double den = 0.0;
    for (long j = 0; j < S; ++j) den += exp(logit[j] - mx);
    if (sink) den += exp(sink[h] - mx);
    for (int i = 0; i < d; ++i) {
      double acc = 0.0;
      for (long j = 0; j < S; ++j) acc += (exp(logit[j] - mx) / den) * kn[j * d + i];
      out[(long)h * d + i] = (S > 0) ? acc : 0.0;
    }
    if (lse) lse[h] = (S > 0 || sink) ? mx + log(den) : -INFINITY;
  }
  free(qn); free(kn); free(logit);
}

/* Sliding-window rows.  [P3] a small set of sliding-window KV entries is
 * appended to the selected compressed entries; [P4] "Sliding-window
 * attention": window 128, the cache keeps the last w-1 tokens plus the current
 * one.  Reading: raw tokens u with max(0, t-w+1) <= u <= t; kv_raw row 0 holds
 * absolute position raw_base.  Returns the number of rows appended, or -1 if
 * a needed row is outside kv_raw. */
static long window_rows(const double* kv_raw, long n_raw, long raw_base, long t, int window, int d,
                        const double** rows, long pos) {
  long lo = t - window + 1;
  if (lo < 0) lo = 0;
  long cnt = 0;
  for (long u = lo; u <= t && window > 0; ++u) {
    long r = u - raw_base;
    if (r < 0 || r >= n_raw) return -1;
    rows[pos + cnt++] = kv_raw + r * d;
  }
  return cnt;
}

/* ------------------------------------------------------------------------ */
/* CSA sparse MQA for one query.  [P3] "Compressed Sparse Attention": the
 * query attends to its top-k compressed entries plus the sliding window.
 *   q [H,d]; kv [n_entries, d]; idx [k] (-1 skipped); kv_raw [n_raw, d]
 * ------------------------------------------------------------------------ */
int oracle_sparse_mqa(const double* q, const double* kv, long n_entries, const int32_t* idx, int k,
                      const double* kv_raw, long n_raw, long raw_base, long t, int window, int H, int d,
                      double scale, double eps, const double* gamma, const double* sink, double* out,
                      double* lse) {
  const double** rows = (const double**)malloc(sizeof(double*) * (size_t)(k + window + 1));
  long S = 0;
  for (int i = 0; i < k; ++i) {
    if (idx[i] < 0) continue;
    if (idx[i] >= n_entries) { free(rows); return ORC_EINVAL; }
    rows[S++] = kv + (long)idx[i] * d;
  }
  long w = window_rows(kv_raw, n_raw, raw_base, t, window, d, rows, S);
  if (w < 0) { free(rows); return ORC_EINVAL; }
  S += w;
  attend(q, rows, S, H, d, scale, eps, gamma, sink, out, lse);
  free(rows);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* HCA dense MQA for one query.  [P3] hybrid CSA/HCA: HCA merges every m'
 * tokens (m' >> m) into one entry and keeps attention dense.  Reading: the
 * query attends to every visible compressed entry s < V(t) plus the same
 * sliding window as CSA, one softmax.
 * ------------------------------------------------------------------------ */
int oracle_dense_mqa(const double* q, const double* kv, long n_entries, int m, const double* kv_raw,
                     long n_raw, long raw_base, long t, int window, int H, int d, double scale,
                     double eps, const double* gamma, const double* sink, double* out, double* lse) {
  long V = oracle_visible(t, n_entries, m);
  const double** rows = (const double**)malloc(sizeof(double*) * (size_t)(V + window + 1));
  long S = 0;
  for (long s = 0; s < V; ++s) rows[S++] = kv + s * d;
  long w = window_rows(kv_raw, n_raw, raw_base, t, window, d, rows, S);
  if (w < 0) { free(rows); return ORC_EINVAL; }
  S += w;
  attend(q, rows, S, H, d, scale, eps, gamma, sink, out, lse);
  free(rows);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* MXFP4 quantisation [MX]: blocks of 32 consecutive values share one e8m0
 * scale 2^E with E = floor(log2(max|x|)) - 2 (2 = exponent of e2m1's largest
 * normal, 6 = 1.5 * 2^2), clamped to [-127, 127]; an all-zero block takes
 * E = -127.  Each element is x / 2^E rounded to the nearest e2m1 value
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6} (ties to the even code), saturating at 6; the
 * sign bit copies the sign of x.  Code layout: 4-bit code = sign<<3 | mag,
 * two per byte, even element in the low nibble.  Scale byte = E + 127.
 * ------------------------------------------------------------------------ */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

static int e2m1_code(double v /* >= 0, already scaled */) {
  if (v >= 6.0) return 7;
  /* nearest grid value; on an exact midpoint take the even code */
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    double dc = fabs(v - kE2M1[c]), db = fabs(v - kE2M1[best]);
    if (dc < db || (dc == db && (c & 1) == 0 && (best & 1) == 1)) best = c;
  }
  return best;
}

void oracle_mxfp4_quantize(const double* x, long n_blocks, uint8_t* codes, uint8_t* scales) {
  for (long b = 0; b < n_blocks; ++b) {
    const double* xb = x + b * 32;
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) if (fabs(xb[i]) > amax) amax = fabs(xb[i]);
    int E;
    if (amax == 0.0) {
      E = -127;
    } else {
      int e2;
      frexp(amax, &e2);          /* amax = f * 2^e2, f in [0.5, 1) => floor(log2 amax) = e2 - 1 */
      E = (e2 - 1) - 2;
      if (E < -127) E = -127;
      if (E > 127) E = 127;
    }
    scales[b] = (uint8_t)(E + 127);
    for (int i = 0; i < 32; i += 2) {
      int cc[2];
      for (int h = 0; h < 2; ++h) {
        double v = xb[i + h];
        int mag = e2m1_code(fabs(ldexp(v, -E)));
        cc[h] = (signbit(v) ? 8 : 0) | mag;
      }
      codes[b * 16 + i / 2] = (uint8_t)(cc[0] | (cc[1] << 4));
    }
  }
}

void oracle_mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, long n_blocks, double* x) {
  for (long b = 0; b < n_blocks; ++b) {
    int E = (int)scales[b] - 127;
    for (int i = 0; i < 32; ++i) {
      int code = (codes[b * 16 + i / 2] >> (4 * (i & 1))) & 0xF;
      double v = kE2M1[code & 7];
      x[b * 32 + i] = ldexp((code & 8) ? -v : v, E);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 (OCP 8-bit floating point, "E4M3FN"): sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 is subnormal (m * 2^-9); the code
 * S.1111.111 is NaN and there is no infinity, so the largest finite value is
 * 1.75 * 2^8 = 448.  [Techniques, Inference quantization]: the compressed KV
 * cache is kept in FP8.  Reading: per element, no scale; x is clamped to
 * [-448, 448] and rounded to the nearest finite value, ties to the even code;
 * the sign bit copies the sign of x (-0 kept).
 * ------------------------------------------------------------------------ */
static double e4m3_value(int mag) { /* mag = code & 0x7f, 0..126 */
  int e = mag >> 3, m = mag & 7;
  return (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
}
void oracle_fp8_quantize(const double* x, long n, uint8_t* codes) {
  for (long i = 0; i < n; ++i) {
    double a = fabs(x[i]);
    if (a > 448.0) a = 448.0;
    int best = 0; /* nearest of the 127 finite magnitudes; ties to the even code */
    for (int mag = 1; mag < 127; ++mag) {
      double d = fabs(e4m3_value(mag) - a), db = fabs(e4m3_value(best) - a);
      if (d < db || (d == db && (mag & 1) == 0)) best = mag;
    }
    codes[i] = (uint8_t)(best | (signbit(x[i]) ? 0x80 : 0));
  }
}
void oracle_fp8_dequantize(const uint8_t* codes, long n, double* x) {
  for (long i = 0; i < n; ++i) {
    double v = e4m3_value(codes[i] & 0x7f);
    x[i] = (codes[i] & 0x80) ? -v : v;
  }
}

/* ------------------------------------------------------------------------ */
/* Rope-conjugate rotation of the attention output ([P4] techniques map,
 * "Gated attention output": the output passes through the conjugate of the
 * rotary rotation before the output projection; "Partial RoPE": only the
 * trailing 64 dims of each 512-dim head are rotated, by
 * x*cos + rotate_half(x)*sin).  The pages print that formula but not
 * rotate_half; V4's rotary is interleaved: it rotates consecutive pairs
 * (x_{2j}, x_{2j+1}) of the slice, rotate_half(x)_{2j} = -x_{2j+1} and
 * rotate_half(x)_{2j+1} = x_{2j}, with one angle per pair.  The conjugate
 * rotation uses the query's cos and sin with the sine negated.
 * cs [128] = cos[64] then sin[64], one value per rotated dim (a pair's two dims
 * carry the same angle); out [H, d] is rotated in place over dims d-64 .. d-1
 * of every head.
 * ------------------------------------------------------------------------ */
void oracle_rope_conjugate(double* out, int H, int d, const double* cs) {
  const double* c = cs;
  const double* s = cs + 64;
  double y[64];
  for (int h = 0; h < H; ++h) {
    double* x = out + (long)h * d + (d - 64);
    for (int i = 0; i < 64; ++i) {
      double rot_half = (i % 2 == 0) ? -x[i + 1] : x[i - 1];
      y[i] = x[i] * c[i] - rot_half * s[i];
    }
    for (int i = 0; i < 64; ++i) x[i] = y[i];
  }
}
