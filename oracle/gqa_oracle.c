/*
 * CPU oracle for grouped-query decode attention and the grouped mean-pool
 * conversion.  TEST INFRASTRUCTURE: only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code with the
 * HIP path and must never be used as a fallback for it.
 *
 * Sources (the pages; cited by title and section):
 *  - wikillm "Grouped-query attention (GQA)", Overview: H query heads are split
 *    into G groups; every head in a group attends with that group's single key
 *    head and value head; a decode step reads the whole cache.
 *  - same page, Implementation sketch, decode-step block: for each query head
 *    i, scores = q[i] . K[:, g(i), :] / sqrt(h); probs = softmax(scores);
 *    out[i] = probs . V[:, g(i), :].  The block's comment says the head-to-group
 *    assignment is not stated and that blocks are assumed: g(i) = i / (H/G).
 *  - same page, Implementation sketch, conversion block, and Variants
 *    ("Converted and uptrained checkpoints"): the K and V projections of the
 *    heads in one group are mean-pooled; head i owns columns i*h .. (i+1)*h-1.
 *  - elemedex glossary "grouped-query attention", paragraph "Grouped (GQA)":
 *    GQA-1 is multi-query attention, GQA-H is multi-head attention.
 *
 * Arithmetic: every input element is widened exactly to binary64 and all work
 * is done in binary64, in the plain order of the definition (no splitting, no
 * online softmax, no fusion).  Build with -O2 -ffp-contract=off.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

/* Exact widening of one stored element to binary64.  bfloat16 is the upper
 * half of an IEEE binary32, so its value is that binary32 with 16 zero bits
 * appended. */
static double widen(const void *base, size_t i, int elem) {
  if (elem == ORACLE_F64) return ((const double *)base)[i];
  if (elem == ORACLE_F32) return (double)((const float *)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

typedef struct {
  const void *q, *k, *v;
  int elem;
  const int32_t *seq_lens;
  int B, H, G, d, Lmax;
  int window; /* > 0: attend only the last `window` cached positions */
  double scale;
  double *out;
  int nthreads, tid;
} decode_job;

/* One query head of one sequence: the decode-step block of the
 * Implementation sketch, over the positions lo .. n-1 held in the cache
 * (lo = 0, or n - window for the sliding-window variant that the wikillm
 * page's Variants section names for Mistral 7B: only the last `window`
 * positions are attended). */
static void decode_head(const decode_job *J, int b, int h, double *s) {
  const int r = J->H / J->G;      /* query heads per K/V head */
  const int g = h / r;            /* block assignment of heads to groups */
  const int d = J->d;
  long n = J->seq_lens[b];
  if (n < 0) n = 0;
  if (n > J->Lmax) n = J->Lmax;
  long lo = 0;
  if (J->window > 0 && n > J->window) lo = n - J->window;
  double *o = J->out + ((size_t)b * J->H + h) * d;
  for (int c = 0; c < d; ++c) o[c] = 0.0;
  if (n == 0) return; /* empty cache: the empty weighted sum is zero */

  const size_t q_off = ((size_t)b * J->H + h) * d;
  const size_t kv_off = ((size_t)b * J->G + g) * (size_t)J->Lmax * d;

  /* scores[t] = scale * sum_i q[i] * K[t, i] */
  for (long t = lo; t < n; ++t) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i)
      acc += widen(J->q, q_off + i, J->elem) * widen(J->k, kv_off + (size_t)t * d + i, J->elem);
    s[t] = J->scale * acc;
  }
  /* softmax: subtracting the maximum leaves the quotient unchanged and only
   * keeps exp() in range */
  double m = s[lo];
  for (long t = lo + 1; t < n; ++t)
    if (s[t] > m) m = s[t];
  double Z = 0.0;
  for (long t = lo; t < n; ++t) {
    s[t] = exp(s[t] - m);
    Z += s[t];
  }
  /* out = sum_t (w[t] / Z) * V[t, :] */
  for (long t = lo; t < n; ++t) {
    const double p = s[t] / Z;
    for (int c = 0; c < d; ++c)
      o[c] += p * widen(J->v, kv_off + (size_t)t * d + c, J->elem);
  }
}

static void *decode_worker(void *arg) {
  const decode_job *J = (const decode_job *)arg;
  double *s = (double *)malloc(sizeof(double) * (size_t)(J->Lmax > 0 ? J->Lmax : 1));
  if (!s) return (void *)1;
  const long total = (long)J->B * J->H;
  for (long job = J->tid; job < total; job += J->nthreads)
    decode_head(J, (int)(job / J->H), (int)(job % J->H), s);
  free(s);
  return NULL;
}

/*
 * out[B,H,d] (binary64) = grouped-query decode attention of q[B,H,d] over
 * k_cache/v_cache[B,G,Lmax,d], all stored as `elem` (0 binary32, 1 bfloat16
 * bits, 2 binary64), attending to positions 0 .. clamp(seq_lens[b],0,Lmax)-1.
 * Returns 0, or -1 on a shape error (H % G != 0, non-positive sizes), -2 if a
 * worker could not allocate.
 */
int gqa_oracle_decode_window(const void *q, const void *k_cache, const void *v_cache, int elem,
                             const int32_t *seq_lens, int B, int H, int G, int d, int Lmax, int window,
                             double scale, double *out, int nthreads) {
  if (B < 0 || H <= 0 || G <= 0 || d <= 0 || Lmax <= 0 || H % G != 0 || window < 0) return -1;
  if (elem < ORACLE_F32 || elem > ORACLE_F64) return -1;
  if (B == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  decode_job base = {q, k_cache, v_cache, elem, seq_lens, B, H, G, d, Lmax, window, scale, out, nthreads, 0};
  decode_job jobs[256];
  pthread_t th[256];
  int rc = 0;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = base;
    jobs[t].tid = t;
  }
  for (int t = 1; t < nthreads; ++t)
    if (pthread_create(&th[t], NULL, decode_worker, &jobs[t]) != 0) {
      /* run the stripe inline if a thread cannot start */
      if (decode_worker(&jobs[t])) rc = -2;
      th[t] = 0;
    }
  if (decode_worker(&jobs[0])) rc = -2;
  for (int t = 1; t < nthreads; ++t)
    if (th[t]) {
      void *res = NULL;
      pthread_join(th[t], &res);
      if (res) rc = -2;
    }
  return rc;
}

int gqa_oracle_decode(const void *q, const void *k_cache, const void *v_cache, int elem,
                      const int32_t *seq_lens, int B, int H, int G, int d, int Lmax,
                      double scale, double *out, int nthreads) {
  return gqa_oracle_decode_window(q, k_cache, v_cache, elem, seq_lens, B, H, G, d, Lmax, 0, scale, out,
                                  nthreads);
}

static size_t elem_size(int elem) { return elem == ORACLE_F64 ? 8 : (elem == ORACLE_F32 ? 4 : 2); }

/*
 * The decode-step block with its cache append: the new token's key and value
 * (k_new, v_new [B,G,d]) are appended - written at position len-1 of each
 * sequence's cache, where len = clamp(seq_lens[b], 0, Lmax) counts the new
 * token - and then attended with the rest (gqa_oracle_decode_window).
 * k_cache / v_cache are updated in place; len = 0 appends nothing.
 */
int gqa_oracle_decode_append(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                             int elem, const int32_t *seq_lens, int B, int H, int G, int d, int Lmax,
                             int window, double scale, double *out, int nthreads) {
  if (B < 0 || H <= 0 || G <= 0 || d <= 0 || Lmax <= 0 || H % G != 0 || window < 0) return -1;
  if (elem < ORACLE_F32 || elem > ORACLE_F64) return -1;
  const size_t es = elem_size(elem);
  for (int b = 0; b < B; ++b) {
    long n = seq_lens[b];
    if (n < 0) n = 0;
    if (n > Lmax) n = Lmax;
    if (n == 0) continue;
    for (int g = 0; g < G; ++g) {
      const size_t dst = (((size_t)b * G + g) * (size_t)Lmax + (size_t)(n - 1)) * d;
      const size_t src = ((size_t)b * G + g) * d;
      memcpy((char *)k_cache + dst * es, (const char *)k_new + src * es, d * es);
      memcpy((char *)v_cache + dst * es, (const char *)v_new + src * es, d * es);
    }
  }
  return gqa_oracle_decode_window(q, k_cache, v_cache, elem, seq_lens, B, H, G, d, Lmax, window, scale, out,
                                  nthreads);
}

/*
 * y[M,N] (binary64) = x[M,K] @ W[K,N]: the projections of the decode-step
 * block (q = x @ Wq, key = x @ Wk, val = x @ Wv, and y = out @ Wo), one row
 * of x per token.  x and W are stored as `elem`, row-major; the sum over k is
 * taken in ascending order.  Returns 0, or -1 on a shape error.
 */
int gqa_oracle_matmul(const void *x, const void *w, int elem, int M, int K, int N, double *y) {
  if (M < 0 || K <= 0 || N <= 0 || elem < ORACLE_F32 || elem > ORACLE_F64) return -1;
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k)
        acc += widen(x, (size_t)m * K + k, elem) * widen(w, (size_t)k * N + n, elem);
      y[(size_t)m * N + n] = acc;
    }
  return 0;
}

/*
 * Grouped mean-pool of a projection matrix w[d_model, H*h] (binary32, head i
 * owns columns i*h .. (i+1)*h-1) into w_out[d_model, G*h]: column block g is
 * the mean of the column blocks of heads g*r .. g*r+r-1, r = H/G.
 * The mean is taken as: binary64 sum in ascending head order, starting from
 * the first member, one binary64 division by r, one rounding to binary32.
 * Returns 0, or -1 on a shape error.
 */
int gqa_oracle_meanpool(const float *w, int d_model, int H, int G, int h, float *w_out) {
  if (d_model < 0 || H <= 0 || G <= 0 || h <= 0 || H % G != 0) return -1;
  const int r = H / G;
  const size_t in_cols = (size_t)H * h, out_cols = (size_t)G * h;
  for (int row = 0; row < d_model; ++row)
    for (int g = 0; g < G; ++g)
      for (int c = 0; c < h; ++c) {
        const float *wr = w + (size_t)row * in_cols;
        double acc = (double)wr[(size_t)(g * r) * h + c];
        for (int i = g * r + 1; i < g * r + r; ++i) acc += (double)wr[(size_t)i * h + c];
        w_out[(size_t)row * out_cols + (size_t)g * h + c] = (float)(acc / (double)r);
      }
  return 0;
}
