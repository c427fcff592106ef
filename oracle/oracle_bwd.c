/*
 * oracle_bwd.c — plain fp64 CPU oracle for the softmax-attention backward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite may load this library.  It
 * shares no code, header, table or helper with the GPU path.
 *
 * What it computes (the plain derivative of the forward definition)
 * -----------------------------------------------------------------
 * Forward, for sequence b (length L), query head h, kv head c = floor(h/g),
 * query position i, allowed set A(i) (causal: j <= i):
 *   s_ij = scale * q_i . k_j,   LSE_i = ln sum_{j in A(i)} exp(s_ij),
 *   P_ij = exp(s_ij - LSE_i),   O_i = sum_j P_ij v_j.
 * Given dO (the gradient of a scalar loss with respect to O):
 *   dV_j  = sum_{h in group c} sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   D_i   = sum_j P_ij dP_ij                       ( = dO_i . O_i )
 *   dS_ij = P_ij (dP_ij - D_i)                      (softmax Jacobian)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_{h in group c} sum_i dS_ij q_i
 * A(i) is the forward's allowed set: keys of the same sequence, j <= i under
 * causal masking, and, with a bit-packed block mask, only keys whose 128-key
 * block has its bit set in the row of the query's 128-query block (bit kb%32
 * of word kb/32; one mask per sequence and kv head, strides in words, 0 =
 * shared).  Rows with an empty allowed set contribute nothing.
 *
 * Source on the pages: the AdaSplash-2 explainer (section 2) names a backward
 * pass that navigates only the visited blocks, and (section 4) training with
 * forward and backward; the formulas above are the chain rule of the forward
 * definition in oracle_attn.c, not taken from the pages.
 *
 * Every score row is materialised in full (LSE and P recomputed here from the
 * definition, independent of any forward output); plain ascending loops, no
 * tiling.  Work is split over (sequence, kv head) pairs, so each thread owns
 * the dK and dV rows it accumulates.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { BWD_OK = 0, BWD_EINVAL = -1, BWD_ENOMEM = -2 };

typedef struct {
  const double *q, *k, *v, *dout;
  const int32_t *cu;
  const uint32_t *mask;
  int64_t mask_ss, mask_sh;
  int mask_words, blk;
  int n_seqs, hq, hkv, d, causal;
  double scale;
  double *dq, *dk, *dv;
  int nthreads;
  int status;
} bjob_t;

typedef struct {
  bjob_t *job;
  int tid;
} bworker_t;

/* Is key j of this sequence in the allowed set of query i (causal bound aside)? */
static int mask_allows(const bjob_t *J, int b, int c, int64_t i, int64_t j) {
  if (!J->mask) return 1;
  const uint32_t *row = J->mask + (int64_t)b * J->mask_ss + (int64_t)c * J->mask_sh +
                        (i / J->blk) * (int64_t)J->mask_words;
  const int64_t kb = j / J->blk;
  return (row[kb / 32] >> (kb % 32)) & 1u;
}

static void one_unit(bjob_t *J, int b, int c, double *s, double *p, double *dp, char *ok) {
  const int64_t base = J->cu[b];
  const int64_t L = (int64_t)J->cu[b + 1] - base;
  const int g = J->hq / J->hkv;
  const int d = J->d;
  for (int h = c * g; h < (c + 1) * g; ++h) {
    for (int64_t i = 0; i < L; ++i) {
      const double *qi = J->q + ((size_t)(base + i) * J->hq + h) * d;
      const double *gi = J->dout + ((size_t)(base + i) * J->hq + h) * d;
      const int64_t n = J->causal ? i + 1 : L;  /* keys 0 .. n-1 pass the causal bound */
      double m = -INFINITY;
      int64_t n_ok = 0;
      for (int64_t j = 0; j < n; ++j) {
        ok[j] = (char)mask_allows(J, b, c, i, j);
        if (!ok[j]) continue;
        ++n_ok;
        const double *kj = J->k + ((size_t)(base + j) * J->hkv + c) * d;
        double dot = 0.0;
        for (int e = 0; e < d; ++e) dot += qi[e] * kj[e];
        s[j] = J->scale * dot;
        if (s[j] > m) m = s[j];
      }
      if (n_ok == 0) continue;
      double l = 0.0;
      for (int64_t j = 0; j < n; ++j)
        if (ok[j]) l += exp(s[j] - m);
      const double lse = m + log(l);
      double D = 0.0;
      for (int64_t j = 0; j < n; ++j) {
        if (!ok[j]) continue;
        p[j] = exp(s[j] - lse);
        const double *vj = J->v + ((size_t)(base + j) * J->hkv + c) * d;
        double dot = 0.0;
        for (int e = 0; e < d; ++e) dot += gi[e] * vj[e];
        dp[j] = dot;
        D += p[j] * dot;
      }
      double *dqi = J->dq + ((size_t)(base + i) * J->hq + h) * d;
      for (int64_t j = 0; j < n; ++j) {
        if (!ok[j]) continue;
        const double ds = p[j] * (dp[j] - D);
        const double *kj = J->k + ((size_t)(base + j) * J->hkv + c) * d;
        double *dkj = J->dk + ((size_t)(base + j) * J->hkv + c) * d;
        double *dvj = J->dv + ((size_t)(base + j) * J->hkv + c) * d;
        for (int e = 0; e < d; ++e) {
          dqi[e] += J->scale * ds * kj[e];
          dkj[e] += J->scale * ds * qi[e];
          dvj[e] += p[j] * gi[e];
        }
      }
    }
  }
}

static void *bworker(void *arg) {
  bworker_t *W = (bworker_t *)arg;
  bjob_t *J = W->job;
  int64_t maxl = 1;
  for (int b = 0; b < J->n_seqs; ++b)
    if ((int64_t)J->cu[b + 1] - J->cu[b] > maxl) maxl = (int64_t)J->cu[b + 1] - J->cu[b];
  double *s = (double *)malloc(sizeof(double) * (size_t)maxl);
  double *p = (double *)malloc(sizeof(double) * (size_t)maxl);
  double *dp = (double *)malloc(sizeof(double) * (size_t)maxl);
  char *ok = (char *)malloc((size_t)maxl);
  if (!s || !p || !dp || !ok) {
    J->status = BWD_ENOMEM;
  } else {
    const int n_units = J->n_seqs * J->hkv;
    for (int u = W->tid; u < n_units; u += J->nthreads) one_unit(J, u / J->hkv, u % J->hkv, s, p, dp, ok);
  }
  free(s);
  free(p);
  free(dp);
  free(ok);
  return NULL;
}

/*
 * oracle_attn_bwd — exact fp64 gradients of softmax attention (dense, causal, block mask).
 *   q, dout        float64 [T][hq][d];  k, v float64 [T][hkv][d]
 *   cu             int32 [n_seqs+1] prefix sums of sequence lengths (host)
 *   mask           NULL, or the bit-packed block mask (host uint32); row of
 *                  query block qb for sequence b, kv head c at
 *                  mask + b*mask_ss + c*mask_sh + qb*mask_words; blocks of
 *                  blk keys / queries
 *   dq             float64 [T][hq][d];  dk, dv float64 [T][hkv][d]  (overwritten)
 * Returns 0, or a negative code on bad arguments / allocation failure.
 */
int oracle_attn_bwd(const double *q, const double *k, const double *v, const double *dout,
                    const int32_t *cu, int n_seqs, int hq, int hkv, int d, int causal,
                    double scale, const uint32_t *mask, int64_t mask_ss, int64_t mask_sh,
                    int mask_words, int blk, double *dq, double *dk, double *dv, int nthreads) {
  if (!q || !k || !v || !dout || !cu || !dq || !dk || !dv || n_seqs < 1 || hq < 1 || hkv < 1 ||
      d < 1 || hq % hkv != 0)
    return BWD_EINVAL;
  if (mask && (blk < 1 || mask_words < 1 || mask_ss < 0 || mask_sh < 0)) return BWD_EINVAL;
  for (int b = 0; b < n_seqs; ++b)
    if (cu[b + 1] < cu[b]) return BWD_EINVAL;
  const int64_t T = cu[n_seqs];
  memset(dq, 0, sizeof(double) * (size_t)T * hq * d);
  memset(dk, 0, sizeof(double) * (size_t)T * hkv * d);
  memset(dv, 0, sizeof(double) * (size_t)T * hkv * d);
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads < 1) nthreads = 1;
  bjob_t J;
  memset(&J, 0, sizeof(J));
  J.q = q; J.k = k; J.v = v; J.dout = dout; J.cu = cu; J.n_seqs = n_seqs; J.hq = hq;
  J.mask = mask; J.mask_ss = mask_ss; J.mask_sh = mask_sh; J.mask_words = mask_words; J.blk = blk;
  J.hkv = hkv; J.d = d; J.causal = causal; J.scale = scale; J.dq = dq; J.dk = dk; J.dv = dv;
  J.nthreads = nthreads;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  bworker_t *ws = (bworker_t *)malloc(sizeof(bworker_t) * (size_t)nthreads);
  if (!th || !ws) { free(th); free(ws); return BWD_ENOMEM; }
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    ws[t].job = &J;
    ws[t].tid = t;
    if (pthread_create(&th[t], NULL, bworker, &ws[t]) != 0) break;
    ++started;
  }
  for (int t = started; t < nthreads; ++t) bworker(&ws[t]);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  free(th);
  free(ws);
  return J.status;
}
