/*
 * attn_oracle.c -- plain fp64 reference for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this
 * file; only the tests, the smoke check and the benchmark's CPU-baseline leg do.
 *
 * What it computes is the plain definition of attention given on the FlashAttention-3
 * pages (zenmind digest, section 3.1 "computation definition", the paper's section 2.1):
 * S = alpha * Q K^T, P = softmax(S) taken along the keys, O = P V, with the row maximum
 * subtracted before exponentiating, and the log-sum-exp L = m + log(l) that the forward
 * pass writes for the backward pass (same digest, section 3.2, epilogue of Algorithm 1).
 *
 * It is written as the definition, not as the tiled algorithm: for every query row it
 * takes two plain passes over that row's keys (the maximum, then the sum of exponentials
 * and the weighted sum of V rows), in fp64, with no blocking and no online rescaling.
 *
 * Indexing (all from the problem statement; readings where the pages are silent):
 *   - tokens are packed as [T, H, d] with d contiguous; a dense [B, N, H, d] batch is the
 *     same thing with cu_seqlens = {0, N, 2N, ..., BN}; cu_seqlens marks where each
 *     sequence starts (the varlen interface of the guijiagi overview, "variable length").
 *   - grouped-query attention: query head h reads key/value head h / (Hq / Hkv), the
 *     FlashAttention-2 style index adjustment the digest mentions in section 3.2 (K and V
 *     are never replicated).
 *   - causal: query i of a sequence sees keys j <= i of the same sequence.
 *   - sliding window of W keys (window > 0; the guijiagi overview's "sliding window
 *     attention" paragraph, which only says attention is taken inside a local window):
 *     query i sees keys j > i - W as well, i.e. with causal the W most recent positions,
 *     itself included.  window <= 0 means no window.
 *   - a row with no visible key gets O = 0 and L = -inf.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* Sequence that holds global token t: the b with cu[b] <= t < cu[b+1]. */
static int64_t seq_of_token(const int64_t* cu, int64_t nseq, int64_t t) {
  int64_t lo = 0, hi = nseq - 1;
  while (lo < hi) {
    int64_t mid = (lo + hi + 1) / 2;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

/* One query row (head h, global token t).  o_row receives d values, *lse one value. */
static void attention_row(const double* q, const double* k, const double* v,
                          int64_t Hq, int64_t Hkv, int64_t d,
                          const int64_t* cu, int64_t nseq, int causal, int64_t window, double alpha,
                          int64_t h, int64_t t, double* o_row, double* lse) {
  const int64_t b = seq_of_token(cu, nseq, t);
  const int64_t start = cu[b];
  const int64_t n = cu[b + 1] - start;
  const int64_t i = t - start;
  const int64_t g = h / (Hq / Hkv);
  const int64_t last = causal ? i : n - 1; /* keys start+first .. start+last are visible */
  const int64_t lo = i - window + 1;       /* oldest key inside a window of W keys */
  const int64_t first = (window > 0 && lo > 0) ? lo : 0;
  const double* qrow = q + (t * Hq + h) * d;

  for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
  if (last < first || n <= 0) { *lse = -INFINITY; return; }

  /* pass 1: scores s_j = alpha * <q, k_j> and their maximum */
  double* s = (double*)malloc(sizeof(double) * (size_t)(last - first + 1));
  double m = -INFINITY;
  for (int64_t j = first; j <= last; ++j) {
    const double* krow = k + ((start + j) * Hkv + g) * d;
    double dot = 0.0;
    for (int64_t c = 0; c < d; ++c) dot += qrow[c] * krow[c];
    s[j - first] = alpha * dot;
    if (s[j - first] > m) m = s[j - first];
  }
  /* pass 2: l = sum_j exp(s_j - m), o = sum_j exp(s_j - m) v_j / l */
  double l = 0.0;
  for (int64_t j = first; j <= last; ++j) {
    const double p = exp(s[j - first] - m);
    const double* vrow = v + ((start + j) * Hkv + g) * d;
    l += p;
    for (int64_t c = 0; c < d; ++c) o_row[c] += p * vrow[c];
  }
  for (int64_t c = 0; c < d; ++c) o_row[c] /= l;
  *lse = m + log(l);
  free(s);
}

/*
 * Selected rows.  q: [T, Hq, d], k and v: [T, Hkv, d] (fp64, host).  cu: nseq+1 int64
 * prefix offsets with cu[0] = 0 and cu[nseq] = T.  rows_h[r], rows_t[r] name row r.
 * o: [n_rows, d], lse: [n_rows].  Returns 0, or -1 on an argument it cannot use.
 */
int oracle_attention_rows(const double* q, const double* k, const double* v,
                          int64_t Hq, int64_t Hkv, int64_t d,
                          const int64_t* cu, int64_t nseq, int causal, int64_t window, double alpha,
                          const int64_t* rows_h, const int64_t* rows_t, int64_t n_rows,
                          double* o, double* lse) {
  if (!q || !k || !v || !cu || !o || !lse || Hq <= 0 || Hkv <= 0 || d <= 0 || nseq <= 0 ||
      Hq % Hkv != 0 || (n_rows > 0 && (!rows_h || !rows_t)))
    return -1;
  const int64_t T = cu[nseq];
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows_h[r] < 0 || rows_h[r] >= Hq || rows_t[r] < 0 || rows_t[r] >= T) return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < n_rows; ++r)
    attention_row(q, k, v, Hq, Hkv, d, cu, nseq, causal, window, alpha, rows_h[r], rows_t[r],
                  o + r * d, lse + r);
  return 0;
}

/* Every row: o is [T, Hq, d]; lse is [Hq, T]. */
int oracle_attention(const double* q, const double* k, const double* v,
                     int64_t Hq, int64_t Hkv, int64_t d,
                     const int64_t* cu, int64_t nseq, int causal, int64_t window, double alpha,
                     double* o, double* lse) {
  if (!q || !k || !v || !cu || !o || !lse || Hq <= 0 || Hkv <= 0 || d <= 0 || nseq <= 0 ||
      Hq % Hkv != 0)
    return -1;
  const int64_t T = cu[nseq];
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t h = 0; h < Hq; ++h)
      attention_row(q, k, v, Hq, Hkv, d, cu, nseq, causal, window, alpha, h, t,
                    o + (t * Hq + h) * d, lse + h * T + t);
  return 0;
}

/* Number of OpenMP threads the calls above use from now on (n >= 1); the benchmark's CPU
 * baseline takes a one-core figure with n = 1. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Number of OpenMP threads the calls above use (reported next to oracle timings). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
