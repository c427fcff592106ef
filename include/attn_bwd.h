/*
 * attn_bwd.h — C ABI of the softmax-attention backward pass (gradients of
 * the forward in attn_fwd.h) for AMD Instinct MI355X (gfx950).
 *
 * The operation
 * -------------
 * With the forward's allowed set A(i), P_ij = exp(scale*q_i.k_j - lse_i) for
 * j in A(i) (0 otherwise), and dO the gradient of a scalar loss with respect
 * to O, the library computes
 *
 *   D_i    = sum_d dO[i,d] * O[i,d]                 (= sum_j P_ij dP_ij)
 *   dP_ij  = dO_i . v_j
 *   dS_ij  = P_ij * (dP_ij - D_i)
 *   dQ_i   = scale * sum_j dS_ij k_j
 *   dK_j   = scale * sum_{h in the group of j's kv head} sum_i dS_ij q_i
 *   dV_j   = sum_{h in the group} sum_i P_ij dO_i
 *
 * the chain rule of the forward, recomputing P from the saved natural-log
 * LSE rather than storing it.  The AdaSplash-2 explainer (section 2,
 * sparsity-aware execution) names a backward pass that visits only the
 * non-zero blocks of a bit-packed block mask, and (section 4) reports that
 * pass as the one that gains most from skipping; with a mask, only the 128 x
 * 128 blocks whose bit is set are loaded here, in both directions.
 *
 * Conventions
 * -----------
 * As for attn_fwd (attn_fwd.h): device pointers owned by the caller, bf16
 * tensors with contiguous head_dim and strides in elements, fp32
 * accumulation, asynchronous on `stream`, no host synchronisation, and the
 * library allocates nothing: the caller passes a device workspace of at least
 * attn_bwd_workspace_size(q) bytes (its contents on entry do not matter; the
 * call overwrites it).  dq, dk, dv are written in bf16 (round to nearest
 * even) at every valid position, zero where no query sees the key (dk, dv)
 * or the query sees no key (dq).  Calls that share a workspace must not
 * overlap.
 */
#ifndef ATTN_BWD_H
#define ATTN_BWD_H

#include <stddef.h>
#include <stdint.h>

#include "attn_fwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of workspace attn_bwd needs for query descriptor q: two float32
 * arrays of q->heads * q->batch * q->seqlen entries (the per-row D and the
 * base-2 LSE).  0 for an empty problem or a NULL descriptor. */
size_t attn_bwd_workspace_size(const attn_tensor_t *q);

/*
 * attn_bwd — gradients of fused attention.
 *
 *   q, out, dout  [B, S, Hq, D]  (or packed [T, Hq, D] with cu_seqlens)
 *   k, v          [B, S, Hkv, D] (or packed [T, Hkv, D])
 *   lse           float32 [B, Hq, S] (packed: [Hq, T]), the natural-log LSE
 *                 attn_fwd returned for these q, k, v (a row of -inf, a row
 *                 that sees no key, gets dq = 0)
 *   cu_seqlens, causal, scale   as for attn_fwd
 *   mask          NULL (dense or causal), or a bit-packed block mask as for
 *                 attn_fwd_mask; the same mask the forward used
 *   dq            [B, S, Hq, D];  dk, dv [B, S, Hkv, D] (packed: [T, H, D])
 *   workspace     device memory of workspace_bytes >= attn_bwd_workspace_size(q)
 *   stream        hipStream_t to enqueue on
 *
 * Returns ATTN_OK, or:
 *   ATTN_ERR_INVALID_ARG  what attn_fwd rejects for q, k, v, out (plus dout
 *                         and dq like out, dk and dv like k); lse == NULL or
 *                         workspace == NULL or workspace_bytes too small for
 *                         a non-empty problem; a bad mask descriptor
 *   ATTN_ERR_UNSUPPORTED  what attn_fwd does not support (head_dim 64, 128
 *                         and 256 are supported); a q or dout stride_seq
 *                         outside [0, 2^24) elements (like k and v); with a
 *                         mask, more than 16384 blocks of 128 per sequence
 *   ATTN_ERR_LAUNCH       a kernel launch failed
 * An empty problem returns ATTN_OK and launches nothing.
 */
int attn_bwd(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
             const attn_tensor_t *out, const attn_tensor_t *dout, const float *lse,
             const int32_t *cu_seqlens, int causal, float scale, const attn_block_mask_t *mask,
             attn_tensor_t *dq, attn_tensor_t *dk, attn_tensor_t *dv, void *workspace,
             size_t workspace_bytes, void *stream);

/*
 * attn_bwd_noalloc — attn_bwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation and arguments without the
 * workspace, which lives instead in a static device array of
 * ATTN_BWD_SCRATCH_BYTES inside the library (one per GPU, held until the
 * process ends).  The call allocates nothing.  The problem must fit it:
 * attn_bwd_workspace_size(q) <= ATTN_BWD_SCRATCH_BYTES (8 bytes per query
 * row and head: e.g. 32 heads x 131072 rows), else ATTN_ERR_TOO_LARGE.  The
 * scratch of the current device (hipGetDevice) is used, so `stream` must
 * belong to that device.  Every call on one GPU shares its scratch and each
 * call overwrites what it needs before reading it, so nothing carries over
 * between calls; calls that overlap on one GPU (other streams, other host
 * threads) race on it and must be serialised by the caller.
 * Returns what attn_bwd returns (the workspace checks aside), or
 * ATTN_ERR_TOO_LARGE, or ATTN_ERR_LAUNCH if the scratch's device address
 * cannot be obtained.
 */
#define ATTN_BWD_SCRATCH_BYTES (32u << 20)
int attn_bwd_noalloc(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
                     const attn_tensor_t *out, const attn_tensor_t *dout, const float *lse,
                     const int32_t *cu_seqlens, int causal, float scale,
                     const attn_block_mask_t *mask, attn_tensor_t *dq, attn_tensor_t *dk,
                     attn_tensor_t *dv, void *stream);

/*
 * attn_block_list_to_mask — the bit-packed block mask of a block list's set,
 * for the backward of a forward that took the list.  The backward navigates
 * bit masks (the AdaSplash-2 explainer, section 2); the ordered list of the
 * CoSA explainer's proxy (attn_fwd.h) is a visiting order over a block set,
 * and the gradients depend on the set only, so a list's backward is the
 * backward with the mask of its set.  Row qb of the output has bit kb % 32
 * of word kb / 32 set exactly when kb is listed for query block qb and
 * 0 <= kb < n_kv_blocks (ids outside that range are skipped, as the forward
 * skips them); every other bit of words 0 .. mask_words-1 is cleared.
 *
 *   list         device row_ptr [num_q_blocks + 1] (non-decreasing, from
 *                row_ptr[0] >= 0) and col_idx [row_ptr[num_q_blocks]], block
 *                sizes 128 (the kernel trusts the contents, which live on the
 *                device)
 *   n_kv_blocks  key blocks per row, 0 .. 16384
 *   mask         device uint32 [num_q_blocks, mask_words], written in full
 *   mask_words   words per row, ceil(n_kv_blocks / 32) .. 512
 * The result, as one sequence's mask shared by every KV head, is what
 * attn_bwd's `mask` takes (num_q_blocks = ceil(S / 128), stride_seq =
 * stride_head = 0, row_stride = mask_words).
 * Returns ATTN_OK (nothing is launched for num_q_blocks == 0),
 * ATTN_ERR_INVALID_ARG for a NULL list, pointer or mask, negative counts or
 * too few or too many words, ATTN_ERR_UNSUPPORTED for block sizes other than
 * 128 or more than 16384 key blocks, ATTN_ERR_LAUNCH if the launch fails.
 */
int attn_block_list_to_mask(const attn_block_list_t *list, int n_kv_blocks, uint32_t *mask,
                            int mask_words, void *stream);

/* The argument checks of attn_bwd alone: host code only, no HIP call. */
int attn_bwd_validate(const attn_tensor_t *q, const attn_tensor_t *k, const attn_tensor_t *v,
                      const attn_tensor_t *out, const attn_tensor_t *dout, const float *lse,
                      const int32_t *cu_seqlens, int causal, float scale,
                      const attn_block_mask_t *mask, const attn_tensor_t *dq,
                      const attn_tensor_t *dk, const attn_tensor_t *dv, const void *workspace,
                      size_t workspace_bytes);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BWD_H */
