/*
 * oracle_osk.c — plain fp64 CPU oracle for ordered skipping along a block list.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code with the GPU
 * path.
 *
 * The CoSA explainer (lay summary) describes a kernel that reads the KV blocks
 * of a query block in the proxy's priority order, builds a cumulative score
 * from the most important blocks first, and then skips the later blocks it no
 * longer needs.  The page states no rule for when to stop; the rule here is
 * the builder's reading of "cumulative score":
 *
 *   Walk the entries e = 1, 2, ... of query block qb's list (n entries) in
 *   order.  For each row i of the block let L_i(e) = sum of exp(s_ij) over
 *   the allowed keys of entries 1..e (its cumulative softmax mass) and d_i(e)
 *   the part of it that entry e added.  If the list ranks blocks by their
 *   mass, each of the n - e entries still to come adds at most d_i(e), so
 *   (n - e) d_i(e) bounds the mass the row would still gain.  After entry e,
 *   if e >= min_visit and (n - e) d_i(e) <= tau * L_i(e) for every row i of
 *   the block, stop: the visited prefix is entries 1..e, and tau bounds the
 *   fraction of each row's mass left out when the ranking holds.  Otherwise
 *   go on; a list that runs out is visited whole.  (A row that has seen no key
 *   yet has L = d = 0 and meets the test.)
 *   The result is exact softmax attention over the keys of the visited
 *   prefix (the allowed set of the block-list definition in oracle_attn.c,
 *   with the list cut at the prefix).
 *
 * The decision is shared by the rows of one query block and one query head
 * (the unit of work of the kernel).  Everything here is fp64; sums of
 * exponentials are kept relative to a per-row running maximum (the ratio
 * d/L does not depend on that reference).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { OSK_OK = 0, OSK_EINVAL = -1, OSK_ENOMEM = -2 };

typedef struct {
  const double *q, *k, *v;
  int64_t T;
  int hq, hkv, d, causal;
  double scale;
  const int32_t *row_ptr, *col_idx;
  int n_qblk, blk;
  double tau;
  int min_visit;
  const int32_t *qblocks;  /* selected query blocks */
  int n_sel;
  const int64_t *row_off;  /* first output row of each selected block */
  double *out, *lse;       /* [rows of the selected blocks][hq][d], [rows][hq] */
  int32_t *visited;        /* [hq][n_sel] */
  double *ratio;           /* [hq][nnz] or NULL: max_i d_i/L_i after each entry */
  int nthreads;
  int status;
} ojob_t;

typedef struct {
  ojob_t *job;
  int tid;
} oworker_t;

static int key_allowed(const ojob_t *J, int64_t i, int64_t j) {
  return j < J->T && (!J->causal || j <= i);
}

/* one (query head, selected query block) unit */
static void one_unit(ojob_t *J, int h, int si, double *m, double *L, double *srow) {
  const int qb = J->qblocks[si];
  const int c = h / (J->hq / J->hkv);
  const int d = J->d;
  const int64_t r0 = (int64_t)qb * J->blk;
  const int64_t r1 = r0 + J->blk < J->T ? r0 + J->blk : J->T;
  const int e0 = J->row_ptr[qb], e1 = J->row_ptr[qb + 1];
  const int64_t nkb = (J->T + J->blk - 1) / J->blk;
  for (int64_t i = r0; i < r1; ++i) {
    m[i - r0] = -INFINITY;
    L[i - r0] = 0.0;
  }
  int visited = e1 - e0;
  for (int e = e0; e < e1; ++e) {
    const int kb = J->col_idx[e];
    double worst = 0.0;
    for (int64_t i = r0; i < r1; ++i) {
      double delta = 0.0;
      if (kb >= 0 && kb < nkb) {
        const double *qi = J->q + ((size_t)i * J->hq + h) * d;
        double mb = -INFINITY;
        int64_t n = 0;
        for (int64_t j = (int64_t)kb * J->blk; j < (int64_t)(kb + 1) * J->blk; ++j) {
          if (!key_allowed(J, i, j)) continue;
          const double *kj = J->k + ((size_t)j * J->hkv + c) * d;
          double dot = 0.0;
          for (int x = 0; x < d; ++x) dot += qi[x] * kj[x];
          srow[n++] = J->scale * dot;
          if (J->scale * dot > mb) mb = J->scale * dot;
        }
        if (n > 0) {
          const double m_new = mb > m[i - r0] ? mb : m[i - r0];
          for (int64_t t = 0; t < n; ++t) delta += exp(srow[t] - m_new);
          L[i - r0] = L[i - r0] * exp(m[i - r0] - m_new) + delta;
          m[i - r0] = m_new;
        }
      }
      const double r = L[i - r0] > 0.0 ? (double)(e1 - e - 1) * delta / L[i - r0] : 0.0;
      if (r > worst) worst = r;
    }
    if (J->ratio) J->ratio[(size_t)h * J->row_ptr[J->n_qblk] + e] = worst;
    if (e - e0 + 1 >= J->min_visit && worst <= J->tau) {
      visited = e - e0 + 1;
      break;
    }
  }
  J->visited[(size_t)h * J->n_sel + si] = visited;

  /* exact softmax attention over the keys of the visited prefix */
  for (int64_t i = r0; i < r1; ++i) {
    const double *qi = J->q + ((size_t)i * J->hq + h) * d;
    const int64_t orow = J->row_off[si] + (i - r0);
    double *oi = J->out + ((size_t)orow * J->hq + h) * d;
    double mx = -INFINITY;
    int64_t n = 0;
    for (int e = e0; e < e0 + visited; ++e) {
      const int kb = J->col_idx[e];
      if (kb < 0 || kb >= nkb) continue;
      for (int64_t j = (int64_t)kb * J->blk; j < (int64_t)(kb + 1) * J->blk; ++j) {
        if (!key_allowed(J, i, j)) continue;
        const double *kj = J->k + ((size_t)j * J->hkv + c) * d;
        double dot = 0.0;
        for (int x = 0; x < d; ++x) dot += qi[x] * kj[x];
        srow[n++] = J->scale * dot;
        if (J->scale * dot > mx) mx = J->scale * dot;
      }
    }
    for (int x = 0; x < d; ++x) oi[x] = 0.0;
    if (n == 0) {
      J->lse[(size_t)orow * J->hq + h] = -INFINITY;
      continue;
    }
    double l = 0.0;
    for (int64_t t = 0; t < n; ++t) l += exp(srow[t] - mx);
    const double lse = mx + log(l);
    J->lse[(size_t)orow * J->hq + h] = lse;
    int64_t t = 0;
    for (int e = e0; e < e0 + visited; ++e) {
      const int kb = J->col_idx[e];
      if (kb < 0 || kb >= nkb) continue;
      for (int64_t j = (int64_t)kb * J->blk; j < (int64_t)(kb + 1) * J->blk; ++j) {
        if (!key_allowed(J, i, j)) continue;
        const double p = exp(srow[t++] - lse);
        const double *vj = J->v + ((size_t)j * J->hkv + c) * d;
        for (int x = 0; x < d; ++x) oi[x] += p * vj[x];
      }
    }
  }
}

static void *oworker(void *arg) {
  oworker_t *W = (oworker_t *)arg;
  ojob_t *J = W->job;
  int max_len = 1;
  for (int r = 0; r < J->n_qblk; ++r)
    if (J->row_ptr[r + 1] - J->row_ptr[r] > max_len) max_len = J->row_ptr[r + 1] - J->row_ptr[r];
  const size_t max_keys = (size_t)max_len * (size_t)J->blk;
  double *m = (double *)malloc(sizeof(double) * (size_t)J->blk);
  double *L = (double *)malloc(sizeof(double) * (size_t)J->blk);
  double *srow = (double *)malloc(sizeof(double) * max_keys);
  if (!m || !L || !srow) {
    J->status = OSK_ENOMEM;
  } else {
    const int n_units = J->hq * J->n_sel;
    for (int u = W->tid; u < n_units; u += J->nthreads) one_unit(J, u / J->n_sel, u % J->n_sel, m, L, srow);
  }
  free(m);
  free(L);
  free(srow);
  return NULL;
}

/*
 * oracle_attn_fwd_osk — ordered skipping forward, one sequence of T tokens.
 *   q [T][hq][d], k, v [T][hkv][d] float64 (host)
 *   row_ptr [n_qblk+1], col_idx [nnz] int32: the ordered block list (blk x blk)
 *   tau >= 0, min_visit >= 1: the stopping rule above
 *   qblocks [n_sel] int32: the query blocks to compute (NULL: all, n_sel = n_qblk)
 *   out [rows][hq][d], lse [rows][hq]: rows of the selected blocks in order
 *   visited [hq][n_sel] int32: entries visited per (head, selected block)
 *   ratio [hq][nnz] or NULL: the test value max_i (n-e) d_i/L_i after each visited entry
 *     (entries after the stop are left as they were)
 * Returns 0, or a negative code.
 */
int oracle_attn_fwd_osk(const double *q, const double *k, const double *v, int64_t T, int hq,
                        int hkv, int d, int causal, double scale, const int32_t *row_ptr,
                        const int32_t *col_idx, int n_qblk, int blk, double tau, int min_visit,
                        const int32_t *qblocks, int n_sel, double *out, double *lse,
                        int32_t *visited, double *ratio, int nthreads) {
  if (!q || !k || !v || !row_ptr || !col_idx || !out || !lse || !visited || T < 1 || hq < 1 ||
      hkv < 1 || d < 1 || hq % hkv != 0 || blk < 1 || n_qblk != (T + blk - 1) / blk ||
      min_visit < 1 || !(tau >= 0.0))
    return OSK_EINVAL;
  int32_t *all = NULL;
  if (!qblocks) {
    all = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_qblk);
    if (!all) return OSK_ENOMEM;
    for (int i = 0; i < n_qblk; ++i) all[i] = i;
    qblocks = all;
    n_sel = n_qblk;
  }
  int64_t *row_off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_sel > 0 ? n_sel : 1));
  if (!row_off) {
    free(all);
    return OSK_ENOMEM;
  }
  int64_t acc = 0;
  for (int s = 0; s < n_sel; ++s) {
    if (qblocks[s] < 0 || qblocks[s] >= n_qblk) {
      free(all);
      free(row_off);
      return OSK_EINVAL;
    }
    row_off[s] = acc;
    const int64_t r0 = (int64_t)qblocks[s] * blk;
    acc += (r0 + blk < T ? r0 + blk : T) - r0;
  }
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads < 1) nthreads = 1;
  ojob_t J;
  memset(&J, 0, sizeof(J));
  J.q = q; J.k = k; J.v = v; J.T = T; J.hq = hq; J.hkv = hkv; J.d = d; J.causal = causal;
  J.scale = scale; J.row_ptr = row_ptr; J.col_idx = col_idx; J.n_qblk = n_qblk; J.blk = blk;
  J.tau = tau; J.min_visit = min_visit; J.qblocks = qblocks; J.n_sel = n_sel;
  J.row_off = row_off; J.out = out; J.lse = lse; J.visited = visited; J.ratio = ratio;
  J.nthreads = nthreads;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  oworker_t *ws = (oworker_t *)malloc(sizeof(oworker_t) * (size_t)nthreads);
  if (!th || !ws) {
    free(th); free(ws); free(all); free(row_off);
    return OSK_ENOMEM;
  }
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    ws[t].job = &J;
    ws[t].tid = t;
    if (pthread_create(&th[t], NULL, oworker, &ws[t]) != 0) break;
    ++started;
  }
  for (int t = started; t < nthreads; ++t) oworker(&ws[t]);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  free(th);
  free(ws);
  free(all);
  free(row_off);
  return J.status;
}
