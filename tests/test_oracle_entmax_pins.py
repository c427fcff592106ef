"""Pins for the alpha-entmax oracle (``oracle.entmax_fwd``).

Each ``pin_*`` takes ``impl(q, k, v, cu, causal, scale, alpha) -> (O, tau)``
over packed float64 tensors and raises AssertionError when it disagrees with
what mathematics fixes:

* alpha = 2 (sparsemax): tau from the sorting closed form (scores sorted
  descending, support size k = the largest k with 1 + k z_(k) > sum_{j<=k}
  z_(j), tau = (sum_{j<=k} z_(j) - 1) / k).
* any alpha: tau is the root scipy's brentq finds for sum_j [(alpha-1) z_j -
  tau]_+^(1/(alpha-1)) = 1 (a library root finder on the definition).
* alpha -> 1: O tends to softmax attention (torch SDPA in float64).
* invariants: sum p = 1 is implied by O of a constant V being that constant;
  adding one vector to every key shifts every score of a row equally, leaving
  O unchanged and moving tau by (alpha-1) times the shift; GQA equals MHA with
  repeated K/V; packed equals per-sequence.
* the histogram bound: tau* - 1/(B-1) <= tau_h <= tau* for B bins of width
  W/(B-1), W = 1/(alpha-1).
* the block mask: bit set exactly where some row of the query block gives
  some key of the key block a positive weight (from the brentq taus).
Planted mistakes in a numpy copy (exponent 1/alpha, (alpha-1) factor
dropped, weights not clipped at zero, causal limit off by one, a
too-short bisection) each fail a pin.
"""
import numpy as np
import pytest
import torch
from scipy.optimize import brentq

import oracle


def oracle_impl(q, k, v, cu, causal, scale, alpha):
    o, t, _ = oracle.entmax_fwd(q, k, v, cu, causal, scale, alpha, nthreads=4)
    return o, t


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def scores(q, k, cu, causal, scale):
    """Per (sequence, head, row): the allowed scores (list of arrays)."""
    T, hq, _ = q.shape
    g = hq // k.shape[1]
    out = {}
    for b in range(len(cu) - 1):
        s0, e0 = int(cu[b]), int(cu[b + 1])
        for h in range(hq):
            z = scale * q[s0:e0, h] @ k[s0:e0, h // g].T
            for i in range(e0 - s0):
                out[(s0 + i, h)] = z[i, :i + 1] if causal else z[i]
    return out


def tau_brentq(z, alpha):
    e = 1.0 / (alpha - 1.0)
    f = lambda t: np.sum(np.clip((alpha - 1.0) * z - t, 0.0, None) ** e) - 1.0
    m = z.max()
    lo, hi = (alpha - 1.0) * m - 1.0, (alpha - 1.0) * m
    if f(lo) <= 0.0:   # the largest score alone already has weight 1
        return lo
    return brentq(f, lo, hi, xtol=1e-15, rtol=1e-15, maxiter=500)


CASES = [(1, [0, 30], 2, 1, 8, False), (2, [0, 17, 40], 4, 2, 8, True), (3, [0, 1, 33], 2, 2, 16, True)]


def case(seed, cu, hq, hkv, d, causal):
    cu = np.array(cu, np.int32)
    T = int(cu[-1])
    return rnd(seed, T, hq, d), rnd(seed + 1, T, hkv, d), rnd(seed + 2, T, hkv, d), cu, causal


def pin_sparsemax_closed_form(impl):
    for c in CASES:
        q, k, v, cu, causal = case(*c)
        _, tau = impl(q, k, v, cu, causal, 0.7, 2.0)
        for (t, h), z in scores(q, k, cu, causal, 0.7).items():
            zs = np.sort(z)[::-1]
            cs = np.cumsum(zs)
            kk = np.arange(1, len(zs) + 1)
            ks = kk[1 + kk * zs > cs].max()
            want = (cs[ks - 1] - 1.0) / ks
            assert abs(tau[t, h] - want) < 1e-12, (c, t, h)


def pin_brentq_root(impl):
    for alpha in (1.25, 1.5, 1.8, 3.0):
        for c in CASES[:2]:
            q, k, v, cu, causal = case(*c)
            o, tau = impl(q, k, v, cu, causal, 0.9, alpha)
            g = q.shape[1] // k.shape[1]
            for (t, h), z in scores(q, k, cu, causal, 0.9).items():
                tb = tau_brentq(z, alpha)
                assert abs(tau[t, h] - tb) < 1e-10, (alpha, c, t, h)
                p = np.clip((alpha - 1.0) * z - tb, 0.0, None) ** (1.0 / (alpha - 1.0))
                b = int(np.searchsorted(cu, t, side="right")) - 1
                s0 = int(cu[b])
                want = p @ v[s0:s0 + len(z), h // g]
                assert np.abs(o[t, h] - want).max() < 1e-9, (alpha, c, t, h)


def pin_alpha_to_one_is_softmax(impl):
    q, k, v, cu, causal = case(*CASES[0])
    o, _ = impl(q, k, v, cu, causal, 0.5, 1.0 + 1e-4)
    qt = torch.tensor(q).permute(1, 0, 2)[None]
    kt = torch.tensor(np.repeat(k, q.shape[1] // k.shape[1], axis=1)).permute(1, 0, 2)[None]
    vt = torch.tensor(np.repeat(v, q.shape[1] // k.shape[1], axis=1)).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.5)[0].permute(1, 0, 2).numpy()
    assert np.abs(o - ref).max() < 2e-3


def pin_constant_v_and_shift(impl):
    for alpha in (1.5, 2.0, 2.5):
        q, k, v, cu, causal = case(*CASES[1])
        vc = np.broadcast_to(np.array([1.5, -2.0, 0.25, 3.0, 0, 1, 2, -1]), v.shape).copy()
        o, tau = impl(q, k, vc, cu, causal, 0.8, alpha)
        assert np.abs(o - vc[0, 0]).max() < 1e-12, alpha
        w = rnd(9, 8)                        # one vector added to every key of every head
        o1, tau1 = impl(q, k, v, cu, causal, 0.8, alpha)
        o2, tau2 = impl(q, k + w, v, cu, causal, 0.8, alpha)
        shift = (alpha - 1.0) * 0.8 * np.einsum("thd,d->th", q, w)
        assert np.abs(o1 - o2).max() < 1e-9 and np.abs(tau2 - tau1 - shift).max() < 1e-9, alpha


def pin_gqa_and_packing(impl):
    q, k, v, cu, causal = case(4, [0, 21, 21, 50], 6, 2, 8, True)
    o, tau = impl(q, k, v, cu, causal, 0.6, 1.6)
    o2, tau2 = impl(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), cu, causal, 0.6, 1.6)
    assert np.abs(o - o2).max() < 1e-13 and np.abs(tau - tau2).max() < 1e-13
    for b in range(3):
        s0, e0 = int(cu[b]), int(cu[b + 1])
        if e0 == s0:
            continue
        ob, tb = impl(q[s0:e0], k[s0:e0], v[s0:e0], np.array([0, e0 - s0], np.int32), causal, 0.6, 1.6)
        assert np.abs(o[s0:e0] - ob).max() < 1e-13 and np.abs(tau[s0:e0] - tb).max() < 1e-13


PINS = [pin_sparsemax_closed_form, pin_brentq_root, pin_alpha_to_one_is_softmax, pin_constant_v_and_shift,
        pin_gqa_and_packing]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_entmax_passes(pin):
    pin(oracle_impl)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 3.0])
@pytest.mark.parametrize("bins", [4, 16, 64])
def test_histogram_bound(alpha, bins):
    q, k, v, cu, causal = case(*CASES[1])
    _, tau, tau_h = oracle.entmax_fwd(q, k, v, cu, causal, 1.3, alpha, bins=bins)
    assert np.all(tau_h <= tau + 1e-12)
    assert np.all(tau_h >= tau - 1.0 / (bins - 1) - 1e-12)


def test_block_mask_marks_positive_weights():
    q, k, v, cu, causal = case(5, [0, 37, 60], 2, 1, 8, True)
    block, alpha = 4, 1.5
    _, tau, _, mask = oracle.entmax_fwd(q, k, v, cu, causal, 1.7, alpha, with_mask=True, block=block)
    n_qblk, words = mask.shape[2], mask.shape[3]
    want = np.zeros_like(mask)
    for (t, h), z in scores(q, k, cu, causal, 1.7).items():
        b = int(np.searchsorted(cu, t, side="right")) - 1
        i = t - int(cu[b])
        tb = tau_brentq(z, alpha)
        for j in np.nonzero((alpha - 1.0) * z - tb > 1e-12)[0]:
            want[b, h, i // block, (j // block) // 32] |= np.uint32(1 << ((j // block) % 32))
    assert np.array_equal(mask, want)
    assert mask.any() and not np.all(mask == mask.max())


def test_rejects_bad_arguments():
    q, k, v, cu, causal = case(*CASES[0])
    with pytest.raises(RuntimeError):
        oracle.entmax_fwd(q, k, v, cu, causal, 1.0, 1.0)   # alpha must exceed 1
    with pytest.raises(RuntimeError):
        oracle.entmax_fwd(q, k, v, cu, causal, 1.0, 1.5, bins=0)


# ----------------------------------------------------------------------------
# Planted mistakes
# ----------------------------------------------------------------------------
def mutant(bug):
    def impl(q, k, v, cu, causal, scale, alpha):
        T, hq, d = q.shape
        g = hq // k.shape[1]
        O = np.zeros((T, hq, d))
        tau = np.zeros((T, hq))
        a1 = 1.0 if bug == "no_alpha_factor" else alpha - 1.0
        e = 1.0 / alpha if bug == "exponent_1_over_alpha" else 1.0 / (alpha - 1.0)
        for b in range(len(cu) - 1):
            s0, e0 = int(cu[b]), int(cu[b + 1])
            for h in range(hq):
                zz = scale * q[s0:e0, h] @ k[s0:e0, h // g].T
                for i in range(e0 - s0):
                    n = i + 1 + (1 if bug == "causal_plus1" and i + 1 < e0 - s0 else 0) if causal else e0 - s0
                    z = zz[i, :n]

                    def mass(t):
                        u = a1 * z - t
                        if bug != "no_clip":
                            u = np.clip(u, 0.0, None)
                        with np.errstate(invalid="ignore"):
                            return np.nansum(np.abs(u) ** e * np.sign(u) if bug == "no_clip" else u ** e)
                    lo, hi = a1 * z.max() - 1.0, a1 * z.max()
                    for _ in range(20 if bug == "short_bisection" else 64):
                        mid = 0.5 * (lo + hi)
                        if mass(mid) >= 1.0:
                            lo = mid
                        else:
                            hi = mid
                    t = 0.5 * (lo + hi)
                    u = a1 * z - t
                    p = np.clip(u, 0.0, None) ** e if bug != "no_clip" else np.abs(u) ** e * np.sign(u)
                    O[s0 + i, h] = p @ v[s0:s0 + n, h // g] / p.sum()
                    tau[s0 + i, h] = t
        return O, tau
    return impl


ENTMAX_MUTANTS = ["exponent_1_over_alpha", "no_alpha_factor", "no_clip", "causal_plus1", "short_bisection"]


def test_clean_numpy_copy_passes_entmax_pins():
    impl = mutant(None)
    for pin in PINS:
        pin(impl)


@pytest.mark.parametrize("bug", ENTMAX_MUTANTS)
def test_entmax_pins_catch_planted_mistake(bug):
    impl = mutant(bug)
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(impl)
            except (AssertionError, ValueError):
                caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {bug!r}"
