"""Pins for the fp64 oracle: results fixed by mathematics rather than by the oracle itself.

Each ``pin_*`` takes an implementation ``impl(q, k, v, cu, causal, scale,
row_ptr=None, col_idx=None, block=128) -> (O, LSE)`` over packed float64
tensors (q [T,Hq,D], k/v [T,Hkv,D]) and raises AssertionError when the
implementation disagrees with the closed form, invariant, brute force or
library special case the pin states.  The oracle must pass every pin; each
deliberately broken implementation at the bottom of this file (a plausible
mistake planted in a numpy copy, on the CPU) must fail at least one.

What is pinned, and by what:
* whole formula           brute force with a differently written textbook
                          formula (no max subtraction, math.fsum), and
                          torch's scaled_dot_product_attention in float64
* normaliser / LSE        Q = 0 gives O = mean of the allowed V and
                          LSE = ln |A(i)| (closed form)
* mask and list membership  Q = 0 with one-hot V counts |A(i) ∩ block|;
                          causal leak needle; list LSE count formula
* max tracking / overflow key-shift invariance with |scores| in the thousands
* linearity, permutation, GQA = repeated MHA, packed = per-sequence,
  full list = dense, list order irrelevant, power-of-two scale, empty set.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def oracle_impl(q, k, v, cu, causal, scale, row_ptr=None, col_idx=None, block=128):
    return oracle.attn_fwd(q, k, v, cu, causal, scale, row_ptr, col_idx, block, nthreads=4)


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def causal_list_rows(rows):
    """CSR from a python list of per-query-block KV block lists."""
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col = np.array([c for r in rows for c in r], dtype=np.int32)
    return row_ptr, col


def allowed_set(i, L, causal, listed_blocks, block):
    out = []
    for j in range(L):
        if causal and j > i:
            continue
        if listed_blocks is not None and (j // block) not in listed_blocks:
            continue
        out.append(j)
    return out


def listed_for(row_ptr, col_idx, qb):
    return set(int(c) for c in col_idx[row_ptr[qb]:row_ptr[qb + 1]])


# ----------------------------------------------------------------------------
# Textbook brute force: no max subtraction, exact summation with math.fsum.
# ----------------------------------------------------------------------------
def textbook(q, k, v, cu, causal, scale, row_ptr=None, col_idx=None, block=128):
    T, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    O = np.zeros((T, hq, d))
    LSE = np.zeros((T, hq))
    for b in range(len(cu) - 1):
        s0, L = int(cu[b]), int(cu[b + 1] - cu[b])
        for i in range(L):
            lb = None if row_ptr is None else listed_for(row_ptr, col_idx, i // block)
            A = allowed_set(i, L, causal, lb, block)
            for h in range(hq):
                kv = h // g
                if not A:
                    LSE[s0 + i, h] = -math.inf
                    continue
                w = [math.exp(scale * math.fsum(q[s0 + i, h, e] * k[s0 + j, kv, e] for e in range(d)))
                     for j in A]
                Z = math.fsum(w)
                LSE[s0 + i, h] = math.log(Z)
                for e in range(d):
                    O[s0 + i, h, e] = math.fsum(wj * v[s0 + j, kv, e] for wj, j in zip(w, A)) / Z
    return O, LSE


TINY_CASES = [
    # name, lengths, hq, hkv, d, causal, list rows (block 4) or None
    ("dense", [16], 2, 2, 8, False, None),
    ("causal", [16], 2, 2, 8, True, None),
    ("gqa_causal", [13], 4, 2, 5, True, None),
    ("varlen", [5, 11, 1, 7], 2, 1, 4, True, None),
    ("varlen_noncausal", [3, 9], 3, 3, 4, False, None),
    ("list", [16], 2, 1, 6, True, [[0], [1, 0], [2], [3, 1]]),
    ("list_noncausal", [16], 2, 2, 3, False, [[2, 0], [3], [0, 1, 2, 3], [1]]),
]


def tiny_inputs(seed, lengths, hq, hkv, d):
    T = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return rnd(seed, T, hq, d), rnd(seed + 1, T, hkv, d), rnd(seed + 2, T, hkv, d), cu


def pin_bruteforce(impl):
    for n, (name, lengths, hq, hkv, d, causal, lrows) in enumerate(TINY_CASES):
        q, k, v, cu = tiny_inputs(100 + 10 * n, lengths, hq, hkv, d)
        rp, ci = (None, None) if lrows is None else causal_list_rows(lrows)
        scale = 0.37
        O, L = impl(q, k, v, cu, causal, scale, rp, ci, 4)
        Ot, Lt = textbook(q, k, v, cu, causal, scale, rp, ci, 4)
        np.testing.assert_allclose(O, Ot, rtol=0, atol=1e-12, err_msg=name)
        np.testing.assert_allclose(L, Lt, rtol=0, atol=1e-12, err_msg=name)


def pin_sdpa(impl):
    """torch SDPA (float64, CPU, explicit boolean mask, K/V repeated per group)."""
    for n, (name, lengths, hq, hkv, d, causal, lrows) in enumerate(TINY_CASES):
        q, k, v, cu = tiny_inputs(200 + 10 * n, lengths, hq, hkv, d)
        rp, ci = (None, None) if lrows is None else causal_list_rows(lrows)
        scale = 0.29
        O, L = impl(q, k, v, cu, causal, scale, rp, ci, 4)
        g = hq // hkv
        for b in range(len(cu) - 1):
            s0, Lb = int(cu[b]), int(cu[b + 1] - cu[b])
            mask = np.zeros((Lb, Lb), dtype=bool)
            for i in range(Lb):
                lb = None if rp is None else listed_for(rp, ci, i // 4)
                for j in allowed_set(i, Lb, causal, lb, 4):
                    mask[i, j] = True
            rows_ok = mask.any(axis=1)
            tq = torch.from_numpy(q[s0:s0 + Lb]).permute(1, 0, 2)
            tk = torch.from_numpy(k[s0:s0 + Lb]).permute(1, 0, 2).repeat_interleave(g, dim=0)
            tv = torch.from_numpy(v[s0:s0 + Lb]).permute(1, 0, 2).repeat_interleave(g, dim=0)
            tm = torch.from_numpy(mask)
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=scale)
            sc = (tq @ tk.transpose(1, 2).contiguous()) * scale
            sc = sc.masked_fill(~tm, float("-inf"))
            lref = torch.logsumexp(sc, dim=-1)
            ok = torch.from_numpy(rows_ok)
            np.testing.assert_allclose(O[s0:s0 + Lb][rows_ok], ref.permute(1, 0, 2)[ok].numpy(),
                                       rtol=0, atol=1e-12, err_msg=name)
            np.testing.assert_allclose(L[s0:s0 + Lb][rows_ok], lref.permute(1, 0)[ok].numpy(),
                                       rtol=0, atol=1e-12, err_msg=name)


def pin_zero_q(impl):
    """Q = 0: O_i = mean of V over A(i), LSE_i = ln |A(i)|."""
    # dense causal: prefix means, LSE = ln(i+1)
    T, hq, d = 40, 2, 6
    v = rnd(7, T, 1, d)
    k = rnd(8, T, 1, d)
    O, L = impl(np.zeros((T, hq, d)), k, v, np.array([0, T], np.int32), True, 0.5)
    pref = np.cumsum(v[:, 0, :], axis=0) / np.arange(1, T + 1)[:, None]
    for h in range(hq):
        np.testing.assert_allclose(O[:, h], pref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(L[:, h], np.log(np.arange(1, T + 1)), rtol=0, atol=1e-13)
    # non-causal: full mean, LSE = ln T
    O, L = impl(np.zeros((T, hq, d)), k, v, np.array([0, T], np.int32), False, 0.5)
    np.testing.assert_allclose(O, np.broadcast_to(v[:, 0].mean(0), (T, hq, d)), rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, np.full((T, hq), math.log(T)), rtol=0, atol=1e-13)
    # block list at 128-row blocks: LSE_i = ln(128 * #off-diagonal listed + (i mod 128) + 1)
    S, blk = 640, 128
    rows = [[0], [1, 0], [2], [3, 0, 1], [4, 2, 0]]
    rp, ci = causal_list_rows(rows)
    kk, vv = rnd(9, S, 1, 4), rnd(10, S, 1, 4)
    O, L = impl(np.zeros((S, 1, 4)), kk, vv, np.array([0, S], np.int32), True, 0.1, rp, ci, blk)
    for i in range(S):
        qb = i // blk
        off = len([c for c in rows[qb] if c != qb])
        np.testing.assert_allclose(L[i, 0], math.log(blk * off + (i % blk) + 1), rtol=0, atol=1e-12)
        A = [j for c in rows[qb] for j in range(c * blk, min((c + 1) * blk, i + 1))]
        np.testing.assert_allclose(O[i, 0], vv[A, 0].mean(0), rtol=0, atol=1e-12)


def pin_one_hot_membership(impl):
    """Q = 0 and V[:, 0] = 1 on block c: O_i[0] = |A(i) ∩ block c| / |A(i)|."""
    S, blk = 768, 128
    rows = [[0], [0, 1], [2, 0], [3], [4, 1, 3], [5, 2, 0, 4]]
    rp, ci = causal_list_rows(rows)
    k = rnd(11, S, 1, 4)
    for c in range(6):
        v = np.zeros((S, 1, 4))
        v[c * blk:(c + 1) * blk, 0, 0] = 1.0
        O, _ = impl(np.zeros((S, 1, 4)), k, v, np.array([0, S], np.int32), True, 0.3, rp, ci, blk)
        for i in range(S):
            qb = i // blk
            A = [j for b in rows[qb] for j in range(b * blk, min((b + 1) * blk, i + 1))]
            inside = sum(1 for j in A if j // blk == c)
            assert abs(O[i, 0, 0] - inside / len(A)) <= 1e-13, (c, i, O[i, 0, 0], inside, len(A))


def pin_row0_single_key(impl):
    q, k, v = rnd(20, 9, 2, 5), rnd(21, 9, 2, 5), rnd(22, 9, 2, 5)
    O, L = impl(q, k, v, np.array([0, 9], np.int32), True, 0.7)
    np.testing.assert_allclose(O[0], v[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(L[0], 0.7 * np.einsum("hd,hd->h", q[0], k[0]), rtol=0, atol=1e-14)
    # S = 1, non-causal
    O, L = impl(q[:1], k[:1], v[:1], np.array([0, 1], np.int32), False, 0.7)
    np.testing.assert_allclose(O[0], v[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(L[0], 0.7 * np.einsum("hd,hd->h", q[0], k[0]), rtol=0, atol=1e-14)


def pin_shift_invariance(impl):
    """K' = K + u: O unchanged, LSE' = LSE + scale * q.u (|scores| reach several thousand)."""
    T, hq, d = 48, 2, 16
    q, k, v = rnd(30, T, hq, d), rnd(31, T, 1, d), rnd(32, T, 1, d)
    u = np.full(d, 2000.0)
    for causal in (False, True):
        O, L = impl(q, k, v, np.array([0, T], np.int32), causal, 0.25)
        O2, L2 = impl(q, k + u, v, np.array([0, T], np.int32), causal, 0.25)
        assert np.all(np.isfinite(O2)) and np.all(np.isfinite(L2))
        np.testing.assert_allclose(O2, O, rtol=0, atol=1e-9)
        np.testing.assert_allclose(L2, L + 0.25 * (q @ u), rtol=1e-12, atol=1e-9)


def pin_linearity(impl):
    T, hq, d = 30, 2, 4
    q, k = rnd(40, T, hq, d), rnd(41, T, 2, d)
    v1, v2 = rnd(42, T, 2, d), rnd(43, T, 2, d)
    cu = np.array([0, 12, T], np.int32)
    O1, _ = impl(q, k, v1, cu, True, 0.6)
    O2, _ = impl(q, k, v2, cu, True, 0.6)
    O12, _ = impl(q, k, v1 + v2, cu, True, 0.6)
    np.testing.assert_allclose(O12, O1 + O2, rtol=0, atol=1e-12)
    c = np.array([1.5, -2.0, 0.25, 3.0])
    Oc, _ = impl(q, k, np.broadcast_to(c, (T, 2, d)).copy(), cu, True, 0.6)
    np.testing.assert_allclose(Oc, np.broadcast_to(c, (T, hq, d)), rtol=0, atol=1e-13)


def pin_permutation(impl):
    T, hq, d = 25, 2, 6
    q, k, v = rnd(50, T, hq, d), rnd(51, T, 2, d), rnd(52, T, 2, d)
    perm = np.random.default_rng(53).permutation(T)
    O, L = impl(q, k, v, np.array([0, T], np.int32), False, 0.4)
    Op, Lp = impl(q, k[perm], v[perm], np.array([0, T], np.int32), False, 0.4)
    np.testing.assert_allclose(Op, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lp, L, rtol=0, atol=1e-12)


def pin_gqa_repeat(impl):
    """Query head h reads KV head floor(h / g): GQA equals MHA with K/V repeated per group."""
    T, hq, hkv, d = 20, 8, 2, 4
    q, k, v = rnd(60, T, hq, d), rnd(61, T, hkv, d), rnd(62, T, hkv, d)
    cu = np.array([0, 7, T], np.int32)
    O, L = impl(q, k, v, cu, True, 0.5)
    g = hq // hkv
    Om, Lm = impl(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), cu, True, 0.5)
    np.testing.assert_allclose(O, Om, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, Lm, rtol=0, atol=1e-13)


def pin_varlen_split(impl):
    lengths = [6, 1, 13, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v = rnd(70, T, 2, 4), rnd(71, T, 1, 4), rnd(72, T, 1, 4)
    for causal in (False, True):
        O, L = impl(q, k, v, cu, causal, 0.8)
        for b in range(len(lengths)):
            s, e = int(cu[b]), int(cu[b + 1])
            Ob, Lb = impl(q[s:e], k[s:e], v[s:e], np.array([0, e - s], np.int32), causal, 0.8)
            np.testing.assert_allclose(O[s:e], Ob, rtol=0, atol=1e-13)
            np.testing.assert_allclose(L[s:e], Lb, rtol=0, atol=1e-13)


def pin_list_vs_dense(impl):
    """A full causal list equals dense causal; list order does not change the result."""
    S, blk = 20, 4
    q, k, v = rnd(80, S, 2, 3), rnd(81, S, 1, 3), rnd(82, S, 1, 3)
    cu = np.array([0, S], np.int32)
    Od, Ld = impl(q, k, v, cu, True, 0.9)
    rows = [list(range(i + 1)) for i in range(5)]
    rp, ci = causal_list_rows(rows)
    Ol, Ll = impl(q, k, v, cu, True, 0.9, rp, ci, blk)
    np.testing.assert_allclose(Ol, Od, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Ll, Ld, rtol=0, atol=1e-13)
    rev = [r[::-1] for r in rows]
    rp2, ci2 = causal_list_rows(rev)
    Or, Lr = impl(q, k, v, cu, True, 0.9, rp2, ci2, blk)
    np.testing.assert_allclose(Or, Ol, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Lr, Ll, rtol=0, atol=1e-13)


def pin_scale_pow2(impl):
    """scale = 1/8 is a power of two: scale*(q.k) and (q/8).k agree exactly."""
    T = 16
    q, k, v = rnd(90, T, 1, 64), rnd(91, T, 1, 64), rnd(92, T, 1, 64)
    cu = np.array([0, T], np.int32)
    O1, L1 = impl(q, k, v, cu, True, 0.125)
    O2, L2 = impl(q / 8.0, k, v, cu, True, 1.0)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-15)


def pin_empty_set(impl):
    """A query block whose list names no visible block gets O = 0 and LSE = -inf."""
    S, blk = 12, 4
    q, k, v = rnd(95, S, 1, 3), rnd(96, S, 1, 3), rnd(97, S, 1, 3)
    rp, ci = causal_list_rows([[0], [2], [1, 2]])  # block 1 lists only a future block
    O, L = impl(q, k, v, np.array([0, S], np.int32), True, 0.5, rp, ci, blk)
    assert np.all(L[4:8] == -np.inf) and np.all(O[4:8] == 0.0)
    assert np.all(np.isfinite(L[:4])) and np.all(np.isfinite(L[8:]))


def pin_causal_needle(impl):
    """Keys after row i aligned with q_i and carrying large V must not move O_i."""
    T, d = 32, 8
    q, k, v = rnd(98, T, 1, d), rnd(99, T, 1, d), rnd(100, T, 1, d)
    cu = np.array([0, T], np.int32)
    for i in (0, 5, 17, 30):
        k2, v2 = k.copy(), v.copy()
        k2[i + 1:, 0] = 30.0 * q[i, 0] / np.linalg.norm(q[i, 0])
        v2[i + 1:, 0] = 10.0
        O, L = impl(q, k, v, cu, True, 0.5)
        O2, L2 = impl(q, k2, v2, cu, True, 0.5)
        np.testing.assert_allclose(O2[i], O[i], rtol=0, atol=1e-13)
        np.testing.assert_allclose(L2[i], L[i], rtol=0, atol=1e-13)


PINS = [pin_bruteforce, pin_sdpa, pin_zero_q, pin_one_hot_membership, pin_row0_single_key,
        pin_shift_invariance, pin_linearity, pin_permutation, pin_gqa_repeat, pin_varlen_split,
        pin_list_vs_dense, pin_scale_pow2, pin_empty_set, pin_causal_needle]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_passes_pin(pin):
    pin(oracle_impl)


def test_oracle_probabilities_sum_to_one():
    """Sum_j P_ij = 1 for every row with a non-empty allowed set (fp64, 1e-12)."""
    lengths = [37, 100, 5]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v = rnd(110, T, 4, 16) * 3, rnd(111, T, 2, 16), rnd(112, T, 2, 16)
    for causal in (False, True):
        _, _, ps = oracle.attn_fwd(q, k, v, cu, causal, 0.5, with_psum=True)
        np.testing.assert_allclose(ps, 1.0, rtol=0, atol=1e-12)


def test_oracle_rows_subset_matches_full():
    """Computing only sampled rows gives the same numbers as the full run."""
    S = 300
    q, k, v = rnd(120, S, 4, 8), rnd(121, S, 2, 8), rnd(122, S, 2, 8)
    rows = np.array([0, 1, 127, 128, 200, 299])
    cu = np.array([0, S], np.int32)
    Of, Lf = oracle.attn_fwd(q, k, v, cu, True, 0.3)
    Os, Ls = oracle.attn_fwd(q[rows], k, v, cu, True, 0.3, rows=rows)
    np.testing.assert_array_equal(Os, Of[rows])
    np.testing.assert_array_equal(Ls, Lf[rows])


def test_oracle_rejects_bad_arguments():
    q = np.zeros((4, 3, 2))
    k = np.zeros((4, 2, 2))
    with pytest.raises(RuntimeError):  # Hq not a multiple of Hkv
        oracle.attn_fwd(q, k, k, np.array([0, 4], np.int32), False, 1.0)
    with pytest.raises(RuntimeError):  # list with two sequences
        oracle.attn_fwd(np.zeros((4, 2, 2)), k, k, np.array([0, 2, 4], np.int32), True, 1.0,
                        np.array([0, 1], np.int32), np.array([0], np.int32), 4)


# ----------------------------------------------------------------------------
# Planted mistakes: a numpy copy of the definition with one bug each.  Every
# mutant must be caught by at least one pin (evidence the pins have power).
# ----------------------------------------------------------------------------
def mutant(bug):
    def impl(q, k, v, cu, causal, scale, row_ptr=None, col_idx=None, block=128):
        T, hq, d = q.shape
        hkv = k.shape[1]
        g = hq // hkv
        O = np.zeros((T, hq, d))
        LSE = np.full((T, hq), -np.inf)
        segs = [(0, T)] if bug == "varlen_leak" else [(int(cu[b]), int(cu[b + 1])) for b in range(len(cu) - 1)]
        for s0, e0 in segs:
            L = e0 - s0
            for h in range(hq):
                kv = (h % hkv) if bug == "gqa_mod" else h // g
                kv_v = (kv + 1) % hkv if bug == "v_head" else kv
                sc_scale = scale * scale if bug == "scale_twice" else scale
                s = sc_scale * q[s0:e0, h] @ k[s0:e0, kv].T
                ii = np.arange(L)[:, None]
                jj = np.arange(L)[None, :]
                allowed = np.ones((L, L), bool)
                if causal:
                    allowed &= (jj < ii) if bug == "causal_strict" else (jj <= ii + (1 if bug == "causal_plus1" else 0))
                if row_ptr is not None and bug != "list_ignored":
                    blk_of_j = (jj - 1) // block if bug == "list_block_off" else jj // block
                    lm = np.zeros((L, L), bool)
                    for i in range(L):
                        listed = listed_for(row_ptr, col_idx, i // block)
                        lm[i] = np.isin(blk_of_j[0], list(listed))
                    allowed &= lm
                if bug == "drop_last_key":
                    allowed[:, L - 1] = False
                s = np.where(allowed, s, -np.inf)
                for i in range(L):
                    if not allowed[i].any():
                        continue
                    if bug == "no_max_sub":
                        w = np.exp(s[i])
                        Z = w.sum()
                        lse = np.log(Z)
                    else:
                        m = s[i].max()
                        w = np.exp(s[i] - m)
                        Z = w.sum()
                        lse = m + np.log(Z)
                    if bug == "lse_log2":
                        lse = lse / math.log(2)
                    p = w if bug == "no_normalise" else w / Z
                    O[s0 + i, h] = p @ v[s0:e0, kv_v]
                    LSE[s0 + i, h] = lse
        return O, LSE
    return impl


MUTANTS = ["causal_strict", "causal_plus1", "gqa_mod", "v_head", "scale_twice", "list_ignored",
           "list_block_off", "drop_last_key", "no_max_sub", "lse_log2", "no_normalise",
           "varlen_leak"]


def test_clean_numpy_copy_passes_pins():
    """The numpy copy without a planted bug passes every pin (so the mutants differ by one bug only)."""
    impl = mutant(None)
    for pin in PINS:
        pin(impl)


@pytest.mark.parametrize("bug", MUTANTS)
def test_pins_catch_planted_mistake(bug):
    impl = mutant(bug)
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(impl)
            except AssertionError:
                caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {bug!r}"
