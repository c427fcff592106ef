/*
 * attn_fwd.h — C ABI of the fused softmax-attention forward library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation
 * -------------
 * For every sequence b, query head h and query position i, with g = Hq/Hkv
 * query heads per key/value head and kv head c = floor(h / g):
 *
 *   A(i)  = { j : 0 <= j < L_b, (causal == 0 || j <= i),
 *                 (no block list || floor(j/128) is listed for floor(i/128)),
 *                 (no block mask || the mask bit of block floor(j/128) is set
 *                                   in the row of floor(i/128)) }
 *   O[b,i,h,:] = sum_{j in A(i)} softmax_j(scale * q.k_j) * v[b,j,c,:]
 *   lse[b,h,i] = ln sum_{j in A(i)} exp(scale * q.k_j)      (natural log)
 *   A(i) empty:  O = 0, lse = -inf.
 *
 * This is the softmax attention that FlashAttention-style kernels compute
 * without materialising the score matrix: the AdaSplash-2 explainer
 * (technical summary, section 1) describes those kernels as fusing the
 * softmax attention steps in on-chip memory, with the closed-form
 * log-sum-exp normaliser.  The optional block list is the ordered priority
 * list of KV blocks that the CoSA explainer (lay summary) has a proxy hand to
 * an ordered-skipping kernel; unlisted blocks are never loaded, as the
 * AdaSplash-2 explainer (section 2, sparsity-aware execution) does for
 * empty blocks.  The list order is only a visiting order.
 *
 * Conventions
 * -----------
 * - All tensor and index pointers are DEVICE pointers owned by the caller.
 *   The library allocates nothing, keeps no state between calls, and is
 *   safe to call from several host threads at once.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream).  The library never reads device memory on the host and never
 *   synchronises.  Errors inside a kernel surface at the caller's next
 *   synchronisation.
 * - q, k, v, out are bfloat16; lse is float32; scale is float32;
 *   accumulation is float32 and O is rounded to nearest even.
 * - head_dim is contiguous (stride 1); all strides are in ELEMENTS.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A bfloat16 tensor of logical shape [batch, seqlen, heads, head_dim].
 * Fixed-length batches: element (b, s, h, d) lives at
 *     data + b*stride_batch + s*stride_seq + h*stride_head + d.
 * Packed variable-length batches (cu_seqlens != NULL): batch = number of
 * sequences, seqlen = an upper bound on every sequence length (the
 * max_seqlen), stride_batch is ignored, and token t of the packed [T, H, D]
 * tensor lives at data + t*stride_seq + h*stride_head + d. */
typedef struct attn_tensor {
  void *data;
  int32_t batch, seqlen, heads, head_dim;
  int64_t stride_batch, stride_seq, stride_head;
} attn_tensor_t;

/* Ordered per-query-block list of KV blocks (CSR).
 * row_ptr: device int32 [num_q_blocks + 1], non-decreasing, row_ptr[0] = 0.
 * col_idx: device int32 [row_ptr[num_q_blocks]], the KV block ids of query
 *          block r in visiting order at col_idx[row_ptr[r] .. row_ptr[r+1]).
 * Ids outside [0, ceil(seqlen/block_k)) are skipped.  Each id may appear at
 * most once per row (a repeated id is a caller error: it is visited twice).
 * Under causal masking, ids above the query block contribute nothing. */
typedef struct attn_block_list {
  const int32_t *row_ptr;
  const int32_t *col_idx;
  int32_t block_q, block_k; /* both must be 128 */
  int32_t num_q_blocks;     /* must equal ceil(seqlen / 128) */
} attn_block_list_t;

/* Bit-packed block mask (one per sequence and KV head).
 * The AdaSplash-2 explainer (section 2, sparsity-aware GPU execution) keeps
 * which blocks of the attention matrix to visit as a bit mask, 32 blocks per
 * 32-bit word, and walks only the set bits (find-first-set / popcount).
 * Here bit (kb % 32) of word kb / 32 of row qb says whether KV block kb
 * (keys 128*kb .. 128*kb+127) is visible to query block qb (queries
 * 128*qb .. 128*qb+127).  The row of query block qb for sequence b and KV
 * head c starts at
 *     bits + b*stride_seq + c*stride_head + qb*words_per_row
 * (strides in 32-bit words; 0 shares one mask across sequences or heads).
 * bits: device uint32, owned by the caller.  Set bits of blocks at or beyond
 * a sequence's end, or above the query block under causal masking,
 * contribute nothing.  Blocks are visited in ascending order. */
typedef struct attn_block_mask {
  const uint32_t *bits;
  int32_t block_q, block_k; /* both must be 128 */
  int32_t num_q_blocks;     /* rows per mask, >= ceil(seqlen / 128) */
  int32_t words_per_row;    /* >= ceil(ceil(seqlen / 128) / 32) */
  int64_t stride_seq;       /* words between the masks of consecutive sequences */
  int64_t stride_head;      /* words between the masks of consecutive KV heads */
} attn_block_mask_t;

enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1, /* arguments contradict each other or are null */
  ATTN_ERR_UNSUPPORTED = -2, /* valid, but not implemented by this library   */
  ATTN_ERR_LAUNCH = -3,      /* the HIP kernel launch itself failed          */
  ATTN_ERR_TOO_LARGE = -4    /* the problem exceeds a fixed-size static buffer */
};

/*
 * attn_fwd — fused attention forward.
 *
 *   q          [B, S, Hq, D]  (or packed [T, Hq, D] with cu_seqlens)
 *   k, v       [B, S, Hkv, D] (or packed [T, Hkv, D]); Hq % Hkv == 0,
 *              k and v have equal heads; q/k/v/out share batch, seqlen
 *              and head_dim
 *   cu_seqlens device int32 [B + 1] prefix sums of packed sequence lengths,
 *              or NULL for fixed-length batches
 *   causal     0 or 1 (key j visible to query i iff j <= i, positions counted
 *              from the start of each sequence)
 *   scale      multiplies q.k; finite and > 0
 *   block_list NULL for dense attention, else see attn_block_list_t
 *              (requires B == 1 and cu_seqlens == NULL)
 *   out        [B, S, Hq, D] bfloat16 (or packed [T, Hq, D]), written only
 *              at valid positions
 *   lse        NULL, or float32 [B, Hq, S] contiguous (packed: [Hq, T] with
 *              T = cu_seqlens[B]); natural log, includes scale
 *   stream     hipStream_t to enqueue on
 *
 * Returns ATTN_OK, or:
 *   ATTN_ERR_INVALID_ARG  null descriptor or data pointer, negative sizes,
 *                         Hq % Hkv != 0, mismatched batch/seqlen/head_dim,
 *                         k/v head mismatch, out heads != Hq, causal not 0/1,
 *                         non-finite scale, bad block-list descriptor
 *   ATTN_ERR_UNSUPPORTED  head_dim not in {64, 128, 256}; scale <= 0; data
 *                         pointer or any stride*2 not a multiple of 16 bytes;
 *                         a k or v stride_seq outside [0, 2^24) elements;
 *                         block sizes other than 128; a block list combined
 *                         with cu_seqlens or batch > 1; a launch grid beyond
 *                         2^31 - 1 workgroups
 *   ATTN_ERR_LAUNCH       the kernel launch failed
 * An empty problem (batch == 0 or seqlen == 0) returns ATTN_OK and launches
 * nothing.
 */
int attn_fwd(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
             const int32_t *cu_seqlens, int causal, float scale,
             const attn_block_list_t *block_list, attn_tensor_t *out, float *lse, void *stream);

/* The argument checks of attn_fwd alone: pure host code, no HIP call, no
 * device access.  Returns what attn_fwd would return before launching. */
int attn_fwd_validate(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
                      const int32_t *cu_seqlens, int causal, float scale,
                      const attn_block_list_t *block_list, const attn_tensor_t *out);

/*
 * attn_fwd_mask — fused attention forward with a bit-packed block mask in
 * place of the block list: A(i) keeps key j only when the mask of the
 * query's sequence and KV head has the bit of block floor(j/128) set in the
 * row of query block floor(i/128).  Every other argument is as for attn_fwd;
 * unlike the block list, the mask works with any batch size and with packed
 * sequences (cu_seqlens).
 *
 * Returns what attn_fwd returns for the shared arguments, or:
 *   ATTN_ERR_INVALID_ARG  mask == NULL, bits == NULL for a non-empty problem,
 *                         negative strides, num_q_blocks < ceil(seqlen/128),
 *                         words_per_row < max(1, ceil(ceil(seqlen/128)/32))
 *   ATTN_ERR_UNSUPPORTED  block sizes other than 128
 */
int attn_fwd_mask(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
                  const int32_t *cu_seqlens, int causal, float scale,
                  const attn_block_mask_t *mask, attn_tensor_t *out, float *lse, void *stream);

/* The argument checks of attn_fwd_mask alone (host code only). */
int attn_fwd_mask_validate(const attn_tensor_t *q, const attn_tensor_t *k,
                           const attn_tensor_t *v, const int32_t *cu_seqlens, int causal,
                           float scale, const attn_block_mask_t *mask,
                           const attn_tensor_t *out);

/*
 * attn_fwd_osk — block-list forward with ordered skipping.
 *
 * The CoSA explainer (lay summary) has the kernel read a query block's KV
 * blocks in the proxy's priority order, gather a cumulative score from the
 * most important ones first, and then skip later blocks it no longer needs;
 * the page states no rule for when to stop.  The rule here: walk the n
 * entries of query block qb's list in order; for each row i of the block let
 * L_i be its softmax mass (sum of exp(scale q_i.k_j) over the keys visited so
 * far) and d_i the part the newest entry e added.  After entry e, if
 * e >= min_visit and (n - e) * d_i <= tau * L_i for every row of the block
 * (for the query head at hand), the walk stops; otherwise it goes on to the
 * end of the list.  If the list ranks blocks by their mass, (n - e) * d_i
 * bounds the mass a row would still gain, so tau bounds the fraction left
 * out.  The result is exact softmax attention (as attn_fwd with the list)
 * over the visited prefix of each (query head, query block); it is an
 * approximation of attn_fwd with the whole list.  The sums are formed in
 * fp32 as the kernel meets them, so a walk whose test value lands within
 * rounding of tau may stop one entry earlier or later than an exact
 * evaluation would.
 *
 *   block_list  required (same rules as for attn_fwd: batch 1, no cu_seqlens)
 *   tau         finite, >= 0 (0: stop only where the rest can add nothing)
 *   min_visit   >= 1: entries always visited before the test applies
 *   visited     NULL, or device int32 [Hq, num_q_blocks]: entries visited per
 *               (query head, query block), written by the call
 * Other arguments and returns as for attn_fwd; additionally
 * ATTN_ERR_INVALID_ARG for a NULL list, a negative or non-finite tau, or
 * min_visit < 1.
 */
int attn_fwd_osk(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
                 int causal, float scale, const attn_block_list_t *block_list, float tau,
                 int min_visit, attn_tensor_t *out, float *lse, int32_t *visited, void *stream);

/* The argument checks of attn_fwd_osk alone (host code only). */
int attn_fwd_osk_validate(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
                          int causal, float scale, const attn_block_list_t *block_list, float tau,
                          int min_visit, const attn_tensor_t *out);

/*
 * attn_entmax_fwd — alpha-entmax attention forward.
 *
 * The AdaSplash-2 explainer (technical summary sections 1-2) replaces softmax
 * by alpha-entmax: for each query row, with scores z_j = scale * q.k_j over
 * the allowed keys (all keys of the sequence, or j <= i under causal
 * masking),
 *     p_j = [(alpha - 1) z_j - tau]_+ ^ (1 / (alpha - 1)),   sum_j p_j = 1,
 *     O = sum_j p_j v_j,
 * so most weights are exactly zero.  tau has no closed form: in one pass
 * that also finds the row max m, the kernel bins the scores of the window
 * [m - 1/(alpha-1), m] into a histogram (32 bins of width 1/(31 (alpha-1))
 * on a fixed grid) whose root is a lower bound of tau within 1/31 of it, then
 * takes steps of a hybrid root finder (Halley for alpha <= 1.5, Newton for
 * alpha <= 2, a secant through the bracket ends above) with a bisection
 * fallback -- until every row of a 128-row tile has |sum p - 1| <= 4e-6, has
 * taken a last Halley step from |sum p - 1| <= 0.1 or Newton step from
 * 2e-3, has taken a sparsemax (alpha = 2) Newton step that no key crosses
 * (exact), has (alpha > 2) at most 8 keys above the histogram bound and
 * solved the mass equation on them exactly, or n_iter steps are done --
 * and finally visits only the 128 x 128
 * blocks that can hold a non-zero weight.  O is divided by sum p at the
 * final tau.
 *
 *   q [B, S, Hq, D], k, v [B, S, Hkv, D] bf16 (fixed-length batches)
 *   alpha        in [1.05, 3] (above 3 the weights rise too steeply from the
 *                support edge for fp32 scores to reproduce exact weights)
 *   n_iter       at most this many refinement steps after the histogram start, 1..32
 *   out          [B, S, Hq, D] bf16
 *   tau          NULL, or float32 [B, Hq, S]: the final threshold per row
 *   block_mask   NULL, or uint32 [B, Hq, ceil(S/128), mask_words]: bit kb % 32
 *                of word kb / 32 of query block qb's row is set when block kb
 *                was visited (a superset of the blocks with a non-zero weight)
 *   mask_words   words per mask row, >= ceil(ceil(S/128) / 32) (with a mask)
 *   tau_init     NULL, or float32 [B, Hq, S]: the histogram lower bound
 * Returns what attn_fwd returns for q, k, v, out (no cu_seqlens, no list), or
 * ATTN_ERR_INVALID_ARG for alpha <= 1 or not finite, n_iter outside 1..32, or
 * too few mask words; ATTN_ERR_UNSUPPORTED for alpha outside [1.05, 3] or
 * more than 16384 blocks of 128 per sequence.
 */
int attn_entmax_fwd(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
                    int causal, float scale, float alpha, int n_iter, attn_tensor_t *out,
                    float *tau, uint32_t *block_mask, int mask_words, float *tau_init,
                    void *stream);

/* The argument checks of attn_entmax_fwd alone (host code only); mask_words
 * is 0 when no mask is written. */
int attn_entmax_fwd_validate(const attn_tensor_t *q, const attn_tensor_t *k,
                             const attn_tensor_t *v, int causal, float scale, float alpha,
                             int n_iter, const attn_tensor_t *out, int mask_words);

/* Static description of a status code (never NULL). */
const char *attn_status_str(int status);

/* Library ABI version: major*10000 + minor*100 + patch. */
int attn_version(void);

/* sha256[:16] (hex) of the compile flags and sources the library was built
 * from, fixed at build time; lets a caller detect a library built from other
 * sources than the headers and kernels beside it. */
const char *attn_source_sha(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
