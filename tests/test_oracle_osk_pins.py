"""Pins for the ordered-skipping oracle (``oracle.attn_fwd_osk``).

Each ``pin_*`` takes ``impl(q, k, v, causal, scale, row_ptr, col_idx, tau,
min_visit, block) -> (O, LSE, visited)`` over one sequence (q [T,Hq,D], k/v
[T,Hkv,D]; O and LSE for every row, visited [Hq, n_qblk]) and raises
AssertionError when it disagrees with what the pin fixes:

* tau = 0 never stops early on lists whose every entry adds mass: the result
  is the exact block-list attention of ``oracle.attn_fwd`` (itself pinned).
* a tau no ratio can exceed stops right after min_visit entries: the result
  is ``oracle.attn_fwd`` on the list cut after min_visit entries.
* a brute force written differently (whole score matrix, cumulative masses as
  running sums of exp(s) without a reference maximum, math.fsum) gives the
  same visited counts and outputs for several tau.
* visited counts never grow when tau grows.
* a block whose keys outscore every other key by ~50, listed first, is
  followed by exactly one more entry (the first entry is all the mass seen so
  far, so the test can only pass at the second), and O is the softmax over
  that block alone to within exp(-40).
* the last entry of a list always passes (nothing remains), so a list whose
  entries all carry equal mass is cut only at its end.
A numpy copy of the rule with one planted mistake each (stop one entry late
or early, ratio taken before adding the entry, min_visit ignored, any row
instead of every row, causal mask ignored in the mass, the remaining-entry
count dropped) fails at least one pin.
"""
import math

import numpy as np
import pytest

import oracle


def oracle_impl(q, k, v, causal, scale, row_ptr, col_idx, tau, min_visit, block):
    o, l, vis, _ = oracle.attn_fwd_osk(q, k, v, causal, scale, row_ptr, col_idx, tau, min_visit,
                                       block=block, nthreads=4)
    return o, l, vis


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def random_list(seed, n_qblk, causal, max_len=None):
    """Ordered lists: every row holds a random subset of its visible blocks in random order,
    always including block 0 and (causal) the diagonal, so every listed entry adds mass."""
    rng = np.random.default_rng(seed)
    rp, ci = [0], []
    for i in range(n_qblk):
        vis = list(range(i + 1)) if causal else list(range(n_qblk))
        take = [b for b in vis if b in (0, i) or rng.random() < 0.6]
        rng.shuffle(take)
        if max_len:
            take = take[:max_len]
        ci += take
        rp.append(len(ci))
    return np.array(rp, np.int32), np.array(ci, np.int32)


def cut_list(row_ptr, col_idx, n_keep):
    rp, ci = [0], []
    for r in range(len(row_ptr) - 1):
        ent = list(col_idx[row_ptr[r]:row_ptr[r + 1]])[:n_keep[r]]
        ci += ent
        rp.append(len(ci))
    return np.array(rp, np.int32), np.array(ci, np.int32)


CASES = [(1, 37, 2, 1, 4, True, 4), (2, 40, 2, 2, 3, False, 5), (3, 29, 4, 2, 4, True, 3)]


def case(seed, T, hq, hkv, d, causal, block):
    q, k, v = rnd(seed, T, hq, d), rnd(seed + 10, T, hkv, d), rnd(seed + 20, T, hkv, d)
    n_qblk = -(-T // block)
    rp, ci = random_list(seed + 30, n_qblk, causal)
    return q, k, v, causal, 0.6, rp, ci, block


def pin_tau_zero_is_exact_list(impl):
    for c in CASES:
        q, k, v, causal, scale, rp, ci, block = case(*c)
        o, l, vis = impl(q, k, v, causal, scale, rp, ci, 0.0, 1, block)
        assert np.array_equal(vis, np.broadcast_to(np.diff(rp), vis.shape)), c
        o_ref, l_ref = oracle.attn_fwd(q, k, v, np.array([0, len(q)], np.int32), causal, scale, rp, ci, block)
        assert np.abs(o - o_ref).max() < 1e-12 and np.abs(l - l_ref).max() < 1e-12, c


def pin_huge_tau_stops_at_min_visit(impl):
    for c in CASES:
        q, k, v, causal, scale, rp, ci, block = case(*c)
        for mv in (1, 2):
            o, l, vis = impl(q, k, v, causal, scale, rp, ci, 1e30, mv, block)
            want = np.minimum(np.diff(rp), mv)
            assert np.array_equal(vis, np.broadcast_to(want, vis.shape)), (c, mv)
            rp2, ci2 = cut_list(rp, ci, want)
            o_ref, l_ref = oracle.attn_fwd(q, k, v, np.array([0, len(q)], np.int32), causal, scale, rp2, ci2, block)
            assert np.abs(o - o_ref).max() < 1e-12 and np.abs(l - l_ref).max() < 1e-12, (c, mv)


def brute(q, k, v, causal, scale, rp, ci, tau, min_visit, block):
    """Whole score matrix per head, cumulative masses as plain running sums of exp(s)."""
    T, hq, d = q.shape
    hkv = k.shape[1]
    n_qblk = len(rp) - 1
    O = np.zeros((T, hq, d))
    LSE = np.full((T, hq), -np.inf)
    vis = np.zeros((hq, n_qblk), np.int32)
    for h in range(hq):
        c = h // (hq // hkv)
        s = scale * q[:, h] @ k[:, c].T
        for qb in range(n_qblk):
            rows = range(qb * block, min(T, (qb + 1) * block))
            ents = list(ci[rp[qb]:rp[qb + 1]])
            cum = {i: 0.0 for i in rows}
            n_vis = len(ents)
            for e, kb in enumerate(ents):
                ok = True
                left = len(ents) - (e + 1)
                for i in rows:
                    keys = [j for j in range(kb * block, min(T, (kb + 1) * block)) if not causal or j <= i]
                    add = math.fsum(math.exp(s[i, j]) for j in keys)
                    cum[i] += add
                    if left * add > tau * cum[i]:
                        ok = False
                if e + 1 >= min_visit and ok:
                    n_vis = e + 1
                    break
            vis[h, qb] = n_vis
            for i in rows:
                keys = sorted({j for kb in ents[:n_vis] for j in range(kb * block, min(T, (kb + 1) * block))
                               if not causal or j <= i})
                if not keys:
                    continue
                w = np.array([math.exp(s[i, j]) for j in keys])
                Z = math.fsum(w)
                O[i, h] = (w / Z) @ v[keys, c]
                LSE[i, h] = math.log(Z)
    return O, LSE, vis


def pin_brute_force(impl):
    for c in CASES:
        q, k, v, causal, scale, rp, ci, block = case(*c)
        for tau in (0.05, 0.3, 1.1, 2.7):  # away from the exact ratios (n - 1) of a first entry
            for mv in (1, 2):
                o, l, vis = impl(q, k, v, causal, scale, rp, ci, tau, mv, block)
                o_b, l_b, vis_b = brute(q, k, v, causal, scale, rp, ci, tau, mv, block)
                assert np.array_equal(vis, vis_b), (c, tau, mv)
                fin = np.isfinite(l_b)
                assert np.abs(o - o_b).max() < 1e-10 and np.abs(l[fin] - l_b[fin]).max() < 1e-10, (c, tau, mv)


def pin_monotone_in_tau(impl):
    for c in CASES:
        q, k, v, causal, scale, rp, ci, block = case(*c)
        prev = None
        for tau in (0.0, 0.03, 0.2, 1.0, 3.0, 10.0):
            _, _, vis = impl(q, k, v, causal, scale, rp, ci, tau, 1, block)
            if prev is not None:
                assert np.all(vis <= prev), (c, tau)
            prev = vis


def pin_dominant_block(impl):
    T, d, block = 24, 4, 4
    rng = np.random.default_rng(7)
    q = rng.standard_normal((T, 1, d)) * 0.1
    q[:, 0, 0] = 5.0
    k = rng.standard_normal((T, 1, d)) * 0.1
    k[8:12, 0, 0] = 10.0             # block 2 outscores every other key by ~50
    v = rng.standard_normal((T, 1, d))
    n_qblk = T // block
    rp = np.arange(n_qblk + 1, dtype=np.int32) * 3
    ci = np.array([b for _ in range(n_qblk) for b in (2, 0, 5)], np.int32)
    o, l, vis = impl(q, k, v, False, 1.0, rp, ci, 1e-12, 1, block)
    assert np.all(vis == 2)
    s = q[:, 0] @ k[8:12, 0].T
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    assert np.abs(o[:, 0] - p @ v[8:12, 0]).max() < 1e-12


def pin_equal_mass_runs_to_the_end(impl):
    """Keys of equal score everywhere: every entry adds the same mass, so
    (n - e) d / L = (n - e) / e stays above tau = 0.5 until the last entry."""
    T, d, block = 32, 4, 4
    q = np.zeros((T, 2, d))
    k = np.zeros((T, 1, d))
    v = np.random.default_rng(8).standard_normal((T, 1, d))
    n_qblk = T // block
    rp = np.arange(n_qblk + 1, dtype=np.int32) * n_qblk
    ci = np.array([b for _ in range(n_qblk) for b in np.random.default_rng(9).permutation(n_qblk)], np.int32)
    _, _, vis = impl(q, k, v, False, 1.0, rp, ci, 0.5, 1, block)
    # (n - e) / e <= 0.5  <=>  e >= 2n/3
    want = int(np.ceil(2 * n_qblk / 3))
    assert np.all(vis == want), vis


PINS = [pin_tau_zero_is_exact_list, pin_huge_tau_stops_at_min_visit, pin_brute_force, pin_monotone_in_tau,
        pin_dominant_block, pin_equal_mass_runs_to_the_end]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_osk_passes(pin):
    pin(oracle_impl)


def test_oracle_osk_selected_blocks_and_ratio_trace():
    """Computing a subset of query blocks gives the same rows; the reported ratios
    are above tau before the stop and at most tau at it."""
    q, k, v, causal, scale, rp, ci, block = case(*CASES[0])
    o, l, vis, ratio = oracle.attn_fwd_osk(q, k, v, causal, scale, rp, ci, 0.2, 2, block=block)
    sel = np.array([1, 4, 6], np.int32)
    o2, l2, vis2, _ = oracle.attn_fwd_osk(q, k, v, causal, scale, rp, ci, 0.2, 2, qblocks=sel, block=block)
    rows = np.concatenate([np.arange(b * block, min(len(q), (b + 1) * block)) for b in sel])
    assert np.array_equal(o2, o[rows]) and np.array_equal(vis2, vis[:, sel])
    for h in range(vis.shape[0]):
        for qb in range(len(rp) - 1):
            r = ratio[h, rp[qb]:rp[qb] + vis[h, qb]]
            n = rp[qb + 1] - rp[qb]
            if vis[h, qb] < n:
                assert r[-1] <= 0.2
            assert np.all(r[1:-1] > 0.2) if vis[h, qb] > 2 else True


def test_oracle_osk_rejects_bad_arguments():
    q, k, v, causal, scale, rp, ci, block = case(*CASES[0])
    with pytest.raises(RuntimeError):
        oracle.attn_fwd_osk(q, k, v, causal, scale, rp, ci, 0.1, 0, block=block)   # min_visit < 1
    with pytest.raises(RuntimeError):
        oracle.attn_fwd_osk(q, k, v, causal, scale, rp, ci, -1.0, 1, block=block)  # tau < 0


# ----------------------------------------------------------------------------
# Planted mistakes
# ----------------------------------------------------------------------------
def mutant(bug):
    def impl(q, k, v, causal, scale, rp, ci, tau, min_visit, block):
        T, hq, d = q.shape
        hkv = k.shape[1]
        n_qblk = len(rp) - 1
        O = np.zeros((T, hq, d))
        LSE = np.full((T, hq), -np.inf)
        vis = np.zeros((hq, n_qblk), np.int32)
        for h in range(hq):
            c = h // (hq // hkv)
            s = scale * q[:, h] @ k[:, c].T
            for qb in range(n_qblk):
                r0, r1 = qb * block, min(T, (qb + 1) * block)
                ents = list(ci[rp[qb]:rp[qb + 1]])
                cum = np.zeros(r1 - r0)
                n_vis = len(ents)
                for e, kb in enumerate(ents):
                    left = 1 if bug == "no_remaining_count" else len(ents) - (e + 1)
                    jj = np.arange(kb * block, min(T, (kb + 1) * block))
                    ii = np.arange(r0, r1)[:, None]
                    allowed = np.ones((r1 - r0, len(jj)), bool)
                    if causal and bug != "mass_no_causal":
                        allowed = jj[None, :] <= ii
                    add = np.where(allowed, np.exp(s[r0:r1][:, jj]), 0.0).sum(1)
                    before = cum.copy()
                    cum = cum + add
                    base = before if bug == "ratio_before_add" else cum
                    sat = left * add <= tau * base
                    ok = sat.any() if bug == "any_row" else sat.all()
                    if (bug == "min_visit_ignored" or e + 1 >= min_visit) and ok:
                        n_vis = e + 1 + (1 if bug == "stop_late" else 0) - (1 if bug == "stop_early" else 0)
                        n_vis = max(0, min(n_vis, len(ents)))
                        break
                vis[h, qb] = n_vis
                for i in range(r0, r1):
                    keys = np.array(sorted({j for kb in ents[:n_vis] for j in range(kb * block, min(T, (kb + 1) * block))
                                            if not causal or j <= i}), dtype=np.int64)
                    if len(keys) == 0:
                        continue
                    w = np.exp(s[i, keys] - s[i, keys].max())
                    O[i, h] = (w / w.sum()) @ v[keys, c]
                    LSE[i, h] = s[i, keys].max() + np.log(w.sum())
        return O, LSE, vis
    return impl


OSK_MUTANTS = ["stop_late", "stop_early", "ratio_before_add", "min_visit_ignored", "any_row", "mass_no_causal",
               "no_remaining_count"]


def test_clean_numpy_copy_passes_osk_pins():
    impl = mutant(None)
    for pin in PINS:
        pin(impl)


@pytest.mark.parametrize("bug", OSK_MUTANTS)
def test_osk_pins_catch_planted_mistake(bug):
    impl = mutant(bug)
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(impl)
            except AssertionError:
                caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {bug!r}"
