/*
 * oracle_entmax.c — plain fp64 CPU oracle for alpha-entmax attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code with the GPU
 * path.
 *
 * What it computes
 * ----------------
 * The AdaSplash-2 explainer (technical summary, section 1) replaces softmax
 * by alpha-entmax, whose normaliser tau has no closed form and is found by
 * root finding.  For query row i with allowed keys A(i) (keys of the same
 * sequence, j <= i under causal masking) and scores z_j = scale * q_i . k_j:
 *
 *   p_j = [(alpha - 1) z_j - tau]_+ ^ (1 / (alpha - 1)),   j in A(i)
 *   tau is the root of  g(tau) = sum_j p_j(tau) - 1,        alpha > 1
 *   O_i = sum_j p_j v_j
 *
 * g is continuous and strictly decreasing where positive; with m = max_j z_j
 * and n = |A(i)| the root lies in [(alpha-1) m - 1, (alpha-1) m - n^(1-alpha)]
 * (at the left end the largest score alone gives p = 1, at the right end
 * every p is at most 1/n).  The oracle bisects that bracket in fp64 until it
 * stops shrinking, so tau is exact to rounding; it then forms p and O
 * (divided by sum p, which is 1 to rounding).  An empty row gives O = 0 and
 * tau = -inf.
 *
 * Histogram lower bound (the same explainer, section 2: solving for tau on a
 * histogram of the scores gives tau_h <= tau*): only scores above
 * m - 1/(alpha-1) can carry weight once tau >= (alpha-1) m - 1, so only the
 * window [m - W, m], W = 1/(alpha-1), is binned.  The bins have width
 * bw = W / (B - 1) on the grid of integer multiples of bw (bin k holds
 * k bw <= z < (k + 1) bw); with top = floor(m / bw), the B bins top - B + 1
 * .. top cover the window, and each score in them is counted at its bin's
 * lower edge k bw (lower scores are dropped).  Every score is then replaced
 * by something no larger, so the histogram's g_h <= g everywhere and its
 * root tau_h <= tau*; placing them at upper edges instead would raise each
 * by at most bw, so tau* <= tau_h + (alpha-1) bw = tau_h + 1/(B-1).  (A grid
 * fixed in z, rather than one anchored at m - W, lets a single pass over the
 * scores bin them while it is still finding m.)
 *
 * Block mask: bit kb % 32 of word kb / 32 of query block qb's row (for each
 * sequence and query head) is set when some row of the query block gives
 * some key of block kb a weight p > 0 (blocks of blk rows / keys).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { ENT_OK = 0, ENT_EINVAL = -1, ENT_ENOMEM = -2 };

typedef struct {
  const double *q, *k, *v;
  const int32_t *cu;
  int n_seqs, hq, hkv, d, causal;
  double scale, alpha;
  int bins, blk, n_qblk, words;
  double *out, *tau, *tau_hist;
  uint32_t *mask;  /* [n_seqs][hq][n_qblk][words] or NULL */
  int nthreads;
  int status;
} ejob_t;

typedef struct {
  ejob_t *job;
  int tid;
} eworker_t;

/* g(tau) + 1 = sum_j [(alpha-1) z_j - tau]_+^(1/(alpha-1)) */
static double mass(const double *z, int64_t n, double alpha, double tau) {
  const double e = 1.0 / (alpha - 1.0);
  double s = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    const double u = (alpha - 1.0) * z[j] - tau;
    if (u > 0.0) s += pow(u, e);
  }
  return s;
}

/* exact root of mass(tau) = 1 by bisection of the bracket */
static double solve_tau(const double *z, int64_t n, double alpha, double m) {
  double lo = (alpha - 1.0) * m - 1.0;
  double hi = (alpha - 1.0) * m - pow((double)n, 1.0 - alpha);
  for (int it = 0; it < 400; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (!(mid > lo && mid < hi)) break;
    if (mass(z, n, alpha, mid) >= 1.0)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

/* root of the histogram's mass: bins counted at their lower edges */
static double solve_tau_hist(const double *z, int64_t n, double alpha, double m, int bins,
                             double *cnt) {
  const double W = 1.0 / (alpha - 1.0);
  const double bw = W / (bins - 1);
  const double top = floor(m / bw);
  const double k0 = top - (bins - 1); /* grid index of the lowest bin */
  for (int b = 0; b < bins; ++b) cnt[b] = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    const double k = floor(z[j] / bw);
    if (k < k0) continue;
    cnt[(int)(k - k0)] += 1.0;
  }
  const double e = 1.0 / (alpha - 1.0);
  /* the histogram's root lies between (alpha-1) m - 2 (where the top bin
     alone, at most bw below m, already has mass >= 1) and (alpha-1) m */
  double lo = (alpha - 1.0) * m - 2.0;
  double hi = (alpha - 1.0) * m;
  for (int it = 0; it < 400; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (!(mid > lo && mid < hi)) break;
    double s = 0.0;
    for (int b = 0; b < bins; ++b) {
      const double u = (alpha - 1.0) * ((k0 + b) * bw) - mid;
      if (u > 0.0 && cnt[b] > 0.0) s += cnt[b] * pow(u, e);
    }
    if (s >= 1.0)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

static void one_row(ejob_t *J, int b, int h, int64_t i, double *z, double *cnt) {
  const int64_t base = J->cu[b];
  const int64_t L = (int64_t)J->cu[b + 1] - base;
  const int c = h / (J->hq / J->hkv);
  const int d = J->d;
  const double *qi = J->q + ((size_t)(base + i) * J->hq + h) * d;
  double *oi = J->out + ((size_t)(base + i) * J->hq + h) * d;
  const int64_t n = J->causal ? i + 1 : L;
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j) {
    const double *kj = J->k + ((size_t)(base + j) * J->hkv + c) * d;
    double dot = 0.0;
    for (int x = 0; x < d; ++x) dot += qi[x] * kj[x];
    z[j] = J->scale * dot;
    if (z[j] > m) m = z[j];
  }
  for (int x = 0; x < d; ++x) oi[x] = 0.0;
  const size_t ti = (size_t)(base + i) * J->hq + h;
  if (n == 0) {
    J->tau[ti] = -INFINITY;
    if (J->tau_hist) J->tau_hist[ti] = -INFINITY;
    return;
  }
  const double tau = solve_tau(z, n, J->alpha, m);
  J->tau[ti] = tau;
  if (J->tau_hist) J->tau_hist[ti] = solve_tau_hist(z, n, J->alpha, m, J->bins, cnt);
  const double e = 1.0 / (J->alpha - 1.0);
  double psum = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    const double u = (J->alpha - 1.0) * z[j] - tau;
    const double p = u > 0.0 ? pow(u, e) : 0.0;
    if (p > 0.0) {
      psum += p;
      const double *vj = J->v + ((size_t)(base + j) * J->hkv + c) * d;
      for (int x = 0; x < d; ++x) oi[x] += p * vj[x];
      if (J->mask) {
        const int64_t kb = j / J->blk, qb = i / J->blk;
        uint32_t *w = J->mask + (((size_t)b * J->hq + h) * J->n_qblk + qb) * J->words + kb / 32;
        __atomic_fetch_or(w, 1u << (kb % 32), __ATOMIC_RELAXED);
      }
    }
  }
  for (int x = 0; x < d; ++x) oi[x] /= psum;
}

static void *eworker(void *arg) {
  eworker_t *W = (eworker_t *)arg;
  ejob_t *J = W->job;
  int64_t maxl = 1;
  for (int b = 0; b < J->n_seqs; ++b)
    if ((int64_t)J->cu[b + 1] - J->cu[b] > maxl) maxl = (int64_t)J->cu[b + 1] - J->cu[b];
  double *z = (double *)malloc(sizeof(double) * (size_t)maxl);
  double *cnt = (double *)malloc(sizeof(double) * (size_t)(J->bins > 0 ? J->bins : 1));
  if (!z || !cnt) {
    J->status = ENT_ENOMEM;
  } else {
    /* rows dealt round-robin: (sequence, head, row) flattened */
    int64_t u = 0;
    for (int b = 0; b < J->n_seqs; ++b) {
      const int64_t L = (int64_t)J->cu[b + 1] - J->cu[b];
      for (int h = 0; h < J->hq; ++h)
        for (int64_t i = 0; i < L; ++i, ++u)
          if (u % J->nthreads == W->tid) one_row(J, b, h, i, z, cnt);
    }
  }
  free(z);
  free(cnt);
  return NULL;
}

/*
 * oracle_entmax_fwd — exact alpha-entmax attention forward.
 *   q [T][hq][d], k, v [T][hkv][d] float64; cu [n_seqs+1] int32 (host)
 *   alpha > 1; bins >= 2 (histogram of tau_hist)
 *   out [T][hq][d], tau [T][hq] (exact normaliser), tau_hist [T][hq] or NULL
 *   mask NULL or uint32 [n_seqs][hq][n_qblk][words] (zeroed here), blocks of blk
 */
int oracle_entmax_fwd(const double *q, const double *k, const double *v, const int32_t *cu,
                      int n_seqs, int hq, int hkv, int d, int causal, double scale, double alpha,
                      int bins, double *out, double *tau, double *tau_hist, uint32_t *mask,
                      int blk, int n_qblk, int words, int nthreads) {
  if (!q || !k || !v || !cu || !out || !tau || n_seqs < 1 || hq < 1 || hkv < 1 || d < 1 ||
      hq % hkv != 0 || !(alpha > 1.0) || bins < 2)
    return ENT_EINVAL;
  if (mask && (blk < 1 || n_qblk < 1 || words < 1)) return ENT_EINVAL;
  if (mask) memset(mask, 0, sizeof(uint32_t) * (size_t)n_seqs * hq * n_qblk * words);
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads < 1) nthreads = 1;
  ejob_t J;
  memset(&J, 0, sizeof(J));
  J.q = q; J.k = k; J.v = v; J.cu = cu; J.n_seqs = n_seqs; J.hq = hq; J.hkv = hkv; J.d = d;
  J.causal = causal; J.scale = scale; J.alpha = alpha; J.bins = bins; J.blk = blk;
  J.n_qblk = n_qblk; J.words = words; J.out = out; J.tau = tau; J.tau_hist = tau_hist;
  J.mask = mask; J.nthreads = nthreads;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  eworker_t *ws = (eworker_t *)malloc(sizeof(eworker_t) * (size_t)nthreads);
  if (!th || !ws) {
    free(th);
    free(ws);
    return ENT_ENOMEM;
  }
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    ws[t].job = &J;
    ws[t].tid = t;
    if (pthread_create(&th[t], NULL, eworker, &ws[t]) != 0) break;
    ++started;
  }
  for (int t = started; t < nthreads; ++t) eworker(&ws[t]);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  free(th);
  free(ws);
  return J.status;
}
