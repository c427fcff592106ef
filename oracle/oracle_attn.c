/*
 * oracle_attn.c — plain fp64 CPU oracle for softmax attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU path.
 *
 * What it computes (the plain definition, one query row at a time)
 * ------------------------------------------------------------------
 * For packed sequence b (tokens cu[b] .. cu[b+1]-1, length L), query head h,
 * query position i (0 <= i < L), with g = Hq/Hkv and kv head c = floor(h/g):
 *
 *   A(i)  = { j : 0 <= j < L, (!causal || j <= i),
 *                 (no list || floor(j/blk) is listed for query block floor(i/blk)),
 *                 (no mask || bit floor(j/blk) of the mask row of query block
 *                             floor(i/blk), for sequence b and kv head c, is 1) }
 *   s_j   = scale * sum_d q[i,h,d] * k[j,c,d]          for j in A(i)
 *   m     = max_{j in A(i)} s_j
 *   LSE_i = m + ln( sum_{j in A(i)} exp(s_j - m) )      (natural log)
 *   P_j   = exp(s_j - LSE_i)
 *   O_i   = sum_{j in A(i)} P_j * v[j,c,:]
 *   A(i) empty  =>  LSE_i = -inf, O_i = 0.
 *
 * Sources on the pages: the AdaSplash-2 explainer (technical summary,
 * section 1 "problem statement") says the fused FlashAttention kernels compute
 * the standard softmax attention by fusing the steps in on-chip memory, and
 * that the softmax normaliser is the closed-form log-sum-exp.  Its section 2
 * (sparsity-aware GPU execution) and lay part ("skip the empty shelves") say
 * blocks that are skipped are never visited and contribute nothing.  The CoSA
 * explainer (lay summary) says the kernel receives an ordered priority list of
 * blocks; the order is a visiting order only, so A(i) is the set of listed
 * blocks.  The AdaSplash-2 explainer (section 2, sparsity-aware execution,
 * "bit-packed block masking") stores which blocks hold non-zero weights as a
 * bit mask, 32 blocks per 32-bit word; a block is visited iff its bit is 1.
 * Here bit (kb mod 32) of word floor(kb/32) of a query block's mask row
 * says whether KV block kb is visible; each (sequence, kv head) may have
 * its own mask.  Causal masking, grouped-query heads, packed variable-length batches
 * and the log-sum-exp output are fixed by the workload definitions, not the
 * pages.
 *
 * The whole score row of each query is materialised (masked keys hold -inf);
 * there is no tiling, no online softmax and no reordering of the sums beyond
 * the plain ascending-j loops written here.  Inputs are float64 (callers pass
 * exact widenings of the bfloat16 values the GPU reads).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { ORACLE_OK = 0, ORACLE_EINVAL = -1, ORACLE_ENOMEM = -2 };

typedef struct {
  const double *q, *k, *v;
  const int32_t *cu;
  int n_seqs, hq, hkv, d, causal;
  double scale;
  const int32_t *row_ptr, *col_idx;
  const uint32_t *mask;       /* bit mask (see oracle_attn_fwd_mask), or NULL */
  int64_t mask_ss, mask_sh;   /* words between the masks of consecutive sequences / kv heads */
  int mask_words;             /* words per query-block row */
  int n_qblk, blk;
  const int64_t *rows;
  int64_t n_rows;
  double *out, *lse, *psum;
  int64_t n_tasks;
  int nthreads;
  int status;
} job_t;

typedef struct {
  job_t *job;
  int tid;
} worker_t;

/* Sequence that holds packed token tok (cu is non-decreasing). */
static int find_seq(const int32_t *cu, int n_seqs, int64_t tok) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if ((int64_t)cu[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

/* One (query row, query head) task: build A(i), the score row, LSE, P and O. */
static int one_row(job_t *J, int64_t r, int h, double *srow, unsigned char *allowed,
                   unsigned char *listed) {
  const int64_t tok = J->rows ? J->rows[r] : r;
  const int b = find_seq(J->cu, J->n_seqs, tok);
  const int64_t base = J->cu[b];
  const int64_t L = (int64_t)J->cu[b + 1] - base;
  const int64_t i = tok - base;
  const int g = J->hq / J->hkv;
  const int c = h / g;
  const int d = J->d;
  const double *qi = J->q + ((size_t)r * J->hq + h) * d;
  double *oi = J->out + ((size_t)r * J->hq + h) * d;

  /* allowed set A(i) */
  if (J->mask) {
    const int64_t n_kvblk = (L + J->blk - 1) / J->blk;
    const int qb = (int)(i / J->blk);
    const uint32_t *row = J->mask + (int64_t)b * J->mask_ss + (int64_t)c * J->mask_sh +
                          (int64_t)qb * J->mask_words;
    for (int64_t cb = 0; cb < n_kvblk; ++cb)
      listed[cb] = (unsigned char)((row[cb / 32] >> (cb % 32)) & 1u);
  } else if (J->row_ptr) {
    const int64_t n_kvblk = (L + J->blk - 1) / J->blk;
    const int qb = (int)(i / J->blk);
    memset(listed, 0, (size_t)n_kvblk);
    for (int32_t e = J->row_ptr[qb]; e < J->row_ptr[qb + 1]; ++e) {
      int32_t cb = J->col_idx[e];
      if (cb >= 0 && cb < n_kvblk) listed[cb] = 1;
    }
  }
  for (int64_t j = 0; j < L; ++j) {
    unsigned char ok = 1;
    if (J->causal && j > i) ok = 0;
    if (ok && (J->row_ptr || J->mask) && !listed[j / J->blk]) ok = 0;
    allowed[j] = ok;
  }

  /* materialised score row: s_j for allowed keys, -inf elsewhere */
  for (int64_t j = 0; j < L; ++j) {
    if (!allowed[j]) { srow[j] = -INFINITY; continue; }
    const double *kj = J->k + ((size_t)(base + j) * J->hkv + c) * d;
    double dot = 0.0;
    for (int e = 0; e < d; ++e) dot += qi[e] * kj[e];
    srow[j] = J->scale * dot;
  }

  double m = -INFINITY;
  for (int64_t j = 0; j < L; ++j)
    if (allowed[j] && srow[j] > m) m = srow[j];

  for (int e = 0; e < d; ++e) oi[e] = 0.0;
  double *lse_out = J->lse + (size_t)r * J->hq + h;
  double *psum_out = J->psum ? J->psum + (size_t)r * J->hq + h : NULL;
  if (m == -INFINITY) { /* empty allowed set */
    *lse_out = -INFINITY;
    if (psum_out) *psum_out = 0.0;
    return ORACLE_OK;
  }

  double l = 0.0;
  for (int64_t j = 0; j < L; ++j)
    if (allowed[j]) l += exp(srow[j] - m);
  const double lse = m + log(l);
  *lse_out = lse;

  double ps = 0.0;
  for (int64_t j = 0; j < L; ++j) {
    if (!allowed[j]) continue;
    const double p = exp(srow[j] - lse);
    ps += p;
    const double *vj = J->v + ((size_t)(base + j) * J->hkv + c) * d;
    for (int e = 0; e < d; ++e) oi[e] += p * vj[e];
  }
  if (psum_out) *psum_out = ps;
  return ORACLE_OK;
}

static int64_t max_len(const int32_t *cu, int n) {
  int64_t m = 0;
  for (int b = 0; b < n; ++b)
    if ((int64_t)cu[b + 1] - cu[b] > m) m = (int64_t)cu[b + 1] - cu[b];
  return m;
}

static void *worker(void *arg) {
  worker_t *W = (worker_t *)arg;
  job_t *J = W->job;
  const int64_t L = max_len(J->cu, J->n_seqs);
  double *srow = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  unsigned char *allowed = (unsigned char *)malloc((size_t)(L > 0 ? L : 1));
  unsigned char *listed = (unsigned char *)malloc((size_t)(L / (J->blk > 0 ? J->blk : 1) + 2));
  if (!srow || !allowed || !listed) {
    J->status = ORACLE_ENOMEM;
  } else {
    /* tasks are (row, head) pairs, dealt out round-robin */
    for (int64_t t = W->tid; t < J->n_tasks; t += J->nthreads) {
      one_row(J, t / J->hq, (int)(t % J->hq), srow, allowed, listed);
    }
  }
  free(srow);
  free(allowed);
  free(listed);
  return NULL;
}

/*
 * oracle_attn_fwd — exact fp64 softmax attention forward over packed sequences.
 *
 *   q        float64 [n_q][hq][d]; n_q = n_rows when rows != NULL (the query
 *            rows for those tokens only), else cu[n_seqs] (every token)
 *   k, v     float64 [cu[n_seqs]][hkv][d]
 *   cu       int32 [n_seqs+1] prefix sums of sequence lengths (host)
 *   causal   0/1;  scale  multiplies q.k
 *   row_ptr, col_idx, n_qblk, blk   block list (CSR over query blocks of blk
 *            rows; col_idx holds KV block ids); NULL row_ptr = no list.
 *            Requires n_seqs == 1.
 *   rows     int64 packed token ids to compute (NULL = all tokens)
 *   out      float64 [n_q][hq][d];  lse float64 [n_q][hq];  psum (optional)
 *            float64 [n_q][hq] = sum_j P_j for the invariant check
 *   nthreads worker threads (<= 0: online CPU count)
 * Returns 0, or a negative code on bad arguments / allocation failure.
 */
static int run(const double *q, const double *k, const double *v, const int32_t *cu,
               int n_seqs, int hq, int hkv, int d, int causal, double scale,
               const int32_t *row_ptr, const int32_t *col_idx, const uint32_t *mask,
               int64_t mask_ss, int64_t mask_sh, int mask_words, int n_qblk, int blk,
               const int64_t *rows, int64_t n_rows, double *out, double *lse, double *psum,
               int nthreads) {
  if (!q || !k || !v || !cu || !out || !lse || n_seqs < 1 || hq < 1 || hkv < 1 || d < 1)
    return ORACLE_EINVAL;
  if (row_ptr && mask) return ORACLE_EINVAL;
  if (mask) {
    if (blk < 1 || mask_words < 1 || mask_ss < 0 || mask_sh < 0) return ORACLE_EINVAL;
    for (int b = 0; b < n_seqs; ++b) {
      const int64_t len = (int64_t)cu[b + 1] - cu[b];
      const int64_t nb = (len + blk - 1) / blk;
      if (nb > n_qblk || nb > 32 * (int64_t)mask_words) return ORACLE_EINVAL;
    }
  }
  if (hq % hkv != 0) return ORACLE_EINVAL;
  if (row_ptr && (n_seqs != 1 || blk < 1 || !col_idx)) return ORACLE_EINVAL;
  const int64_t T = cu[n_seqs];
  for (int b = 0; b < n_seqs; ++b)
    if (cu[b + 1] < cu[b]) return ORACLE_EINVAL;
  if (row_ptr) {
    const int64_t need = (T + blk - 1) / blk;
    if (n_qblk < need) return ORACLE_EINVAL;
  }
  const int64_t n_q = rows ? n_rows : T;
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= T) return ORACLE_EINVAL;

  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads < 1) nthreads = 1;

  job_t J;
  memset(&J, 0, sizeof(J));
  J.q = q; J.k = k; J.v = v; J.cu = cu; J.n_seqs = n_seqs; J.hq = hq; J.hkv = hkv; J.d = d;
  J.causal = causal; J.scale = scale; J.row_ptr = row_ptr; J.col_idx = col_idx;
  J.mask = mask; J.mask_ss = mask_ss; J.mask_sh = mask_sh; J.mask_words = mask_words;
  J.n_qblk = n_qblk; J.blk = (row_ptr || mask) ? blk : 1; J.rows = rows; J.n_rows = n_rows;
  J.out = out; J.lse = lse; J.psum = psum; J.n_tasks = n_q * hq; J.nthreads = nthreads;

  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  worker_t *ws = (worker_t *)malloc(sizeof(worker_t) * (size_t)nthreads);
  if (!th || !ws) { free(th); free(ws); return ORACLE_ENOMEM; }
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    ws[t].job = &J;
    ws[t].tid = t;
    if (pthread_create(&th[t], NULL, worker, &ws[t]) != 0) break;
    ++started;
  }
  if (started < nthreads) { /* run the remaining shares on this thread */
    for (int t = started; t < nthreads; ++t) worker(&ws[t]);
  }
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  free(th);
  free(ws);
  return J.status;
}

int oracle_attn_fwd(const double *q, const double *k, const double *v, const int32_t *cu,
                    int n_seqs, int hq, int hkv, int d, int causal, double scale,
                    const int32_t *row_ptr, const int32_t *col_idx, int n_qblk, int blk,
                    const int64_t *rows, int64_t n_rows, double *out, double *lse,
                    double *psum, int nthreads) {
  return run(q, k, v, cu, n_seqs, hq, hkv, d, causal, scale, row_ptr, col_idx, NULL, 0, 0, 0,
             n_qblk, blk, rows, n_rows, out, lse, psum, nthreads);
}

/*
 * oracle_attn_fwd_mask — as oracle_attn_fwd, with a bit-packed block mask in
 * place of the list.  The mask row of query block qb for sequence b and kv
 * head c starts at  mask + b*mask_ss + c*mask_sh + qb*mask_words  (host
 * uint32 words; strides may be 0 to share a mask); bit (kb mod 32) of word
 * floor(kb/32) set means KV block kb is visible.  Blocks of blk positions;
 * every sequence needs ceil(L/blk) <= n_qblk rows and <= 32*mask_words bits.
 * Any number of sequences.
 */
int oracle_attn_fwd_mask(const double *q, const double *k, const double *v, const int32_t *cu,
                         int n_seqs, int hq, int hkv, int d, int causal, double scale,
                         const uint32_t *mask, int64_t mask_ss, int64_t mask_sh, int mask_words,
                         int n_qblk, int blk, const int64_t *rows, int64_t n_rows, double *out,
                         double *lse, double *psum, int nthreads) {
  if (!mask) return ORACLE_EINVAL;
  return run(q, k, v, cu, n_seqs, hq, hkv, d, causal, scale, NULL, NULL, mask, mask_ss, mask_sh,
             mask_words, n_qblk, blk, rows, n_rows, out, lse, psum, nthreads);
}

/* Number of worker threads the oracle uses for nthreads <= 0. */
int oracle_default_threads(void) {
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n < 1 ? 1 : (int)n;
}
