"""Pins for the fp64 backward oracle: gradients fixed by mathematics, not by the oracle.

Each ``pin_*`` takes an implementation ``impl(q, k, v, dout, cu, causal,
scale, block_mask=None, block=128) -> (dq, dk, dv)`` over packed float64
tensors (q, dout [T,Hq,D]; k, v [T,Hkv,D]) and raises AssertionError when it
disagrees with what the pin states.  The oracle passes every pin; each numpy
copy at the bottom with one planted mistake (on the CPU) fails at least one.

What is pinned, and by what:
* every gradient        central finite differences of the forward oracle
                        (itself pinned by test_oracle_pins.py), with and
                        without causal masking, GQA, packing and a block mask
* every gradient        torch autograd through a plain float64 CPU attention
                        written here (a library special case)
* softmax Jacobian      constant V gives dQ = dK = 0; a one-key sequence
                        gives dQ = dK = 0 and dV = sum of its group's dO
* invariants            sum_j dK_j = 0; sum_j dV_j = sum of dO over rows with
                        a non-empty allowed set; sum_i q_i.dQ_i =
                        sum_j k_j.dK_j = scale * dLoss/dscale (finite
                        difference in the scale)
* structure             GQA = repeated MHA with dK, dV summed over the group;
                        packed = per-sequence; linear in dout; full mask = no mask
"""
import numpy as np
import pytest
import torch

import oracle


def oracle_impl(q, k, v, dout, cu, causal, scale, block_mask=None, block=128):
    return oracle.attn_bwd(q, k, v, dout, cu, causal, scale, block_mask, block, nthreads=4)


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def fwd_loss(q, k, v, dout, cu, causal, scale, block_mask=None, block=128):
    o, _ = oracle.attn_fwd(q, k, v, cu, causal, scale, block=block, nthreads=1,
                           block_mask=block_mask)
    return float((o * dout).sum())


def pack_mask(vis):
    """bool [n_seqs, hkv, nqb, nkb] -> uint32 [n_seqs, hkv, nqb, words]."""
    ns, hkv, nqb, nkb = vis.shape
    words = max(1, (nkb + 31) // 32)
    m = np.zeros((ns, hkv, nqb, words), np.uint32)
    for idx in np.ndindex(vis.shape):
        if vis[idx]:
            m[idx[:3] + (idx[3] // 32,)] |= np.uint32(1 << (idx[3] % 32))
    return m


# small problems: (seed, cu, hq, hkv, d, causal, masked, block)
SMALL = [
    (1, [0, 5], 1, 1, 3, False, False, 128),
    (2, [0, 3, 7], 2, 1, 4, True, False, 128),
    (3, [0, 6, 6, 11], 4, 2, 3, True, False, 128),
    (4, [0, 8, 13], 2, 2, 2, False, True, 2),
    (5, [0, 9], 2, 1, 3, True, True, 3),
]


def small_case(seed, cu, hq, hkv, d, causal, masked, block):
    cu = np.array(cu, np.int32)
    T = int(cu[-1])
    q, k, v = rnd(seed, T, hq, d), rnd(seed + 100, T, hkv, d), rnd(seed + 200, T, hkv, d)
    g = rnd(seed + 300, T, hq, d)
    m = None
    if masked:
        nb = -(-int(np.diff(cu).max()) // block)
        vis = np.random.default_rng(seed + 400).random((len(cu) - 1, hkv, nb, nb)) < 0.6
        m = pack_mask(vis)
    return q, k, v, g, cu, causal, 0.7, m, block


def pin_finite_differences(impl):
    h = 1e-6
    for case in SMALL:
        q, k, v, g, cu, causal, scale, m, block = small_case(*case)
        grads = impl(q, k, v, g, cu, causal, scale, m, block)
        for which, x in enumerate((q, k, v)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                args = [q, k, v]
                xp = x.copy()
                xp[idx] += h
                args[which] = xp
                lp = fwd_loss(*args, g, cu, causal, scale, m, block)
                xm = x.copy()
                xm[idx] -= h
                args[which] = xm
                lm = fwd_loss(*args, g, cu, causal, scale, m, block)
                fd[idx] = (lp - lm) / (2 * h)
            err = np.abs(fd - grads[which]).max()
            assert err < 1e-7, (case, "qkv"[which], err)


def torch_grads(q, k, v, g, cu, causal, scale, vis=None, block=128):
    """float64 autograd through the plain formula, one (sequence, head) at a time."""
    qt, kt, vt = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    hq, hkv = q.shape[1], k.shape[1]
    loss = torch.zeros((), dtype=torch.float64)
    for b in range(len(cu) - 1):
        s0, e0 = int(cu[b]), int(cu[b + 1])
        L = e0 - s0
        if L == 0:
            continue
        for h in range(hq):
            c = h // (hq // hkv)
            s = scale * qt[s0:e0, h] @ kt[s0:e0, c].T
            allowed = torch.ones(L, L, dtype=torch.bool)
            if causal:
                allowed &= torch.tril(torch.ones(L, L, dtype=torch.bool))
            if vis is not None:
                ii = torch.arange(L) // block
                allowed &= torch.tensor(vis[b, c])[ii][:, ii]
            rows = allowed.any(1)
            s = s.masked_fill(~allowed, float("-inf"))[rows]
            p = torch.softmax(s, dim=1)
            o = p @ vt[s0:e0, c]
            loss = loss + (o * torch.tensor(g[s0:e0, h][rows.numpy()])).sum()
    loss.backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def pin_torch_autograd(impl):
    cases = [(11, [0, 40], 4, 2, 8, True, None), (12, [0, 17, 17, 50], 2, 1, 8, False, None),
             (13, [0, 23, 48], 4, 1, 4, True, 8), (14, [0, 30], 2, 2, 4, False, 8)]
    for seed, cu, hq, hkv, d, causal, block in cases:
        cu = np.array(cu, np.int32)
        T = int(cu[-1])
        q, k, v = rnd(seed, T, hq, d), rnd(seed + 1, T, hkv, d), rnd(seed + 2, T, hkv, d)
        g = rnd(seed + 3, T, hq, d)
        vis = m = None
        if block is not None:
            nb = -(-int(np.diff(cu).max()) // block)
            vis = np.random.default_rng(seed + 4).random((len(cu) - 1, hkv, nb, nb)) < 0.5
            m = pack_mask(vis)
        ref = torch_grads(q, k, v, g, cu, causal, 0.45, vis, block or 128)
        got = impl(q, k, v, g, cu, causal, 0.45, m, block or 128)
        for name, a, b in zip("qkv", got, ref):
            assert np.abs(a - b).max() < 1e-11, (seed, name, np.abs(a - b).max())


def pin_constant_v(impl):
    cu = np.array([0, 9, 20], np.int32)
    q, k = rnd(21, 20, 4, 6), rnd(22, 20, 2, 6)
    v = np.broadcast_to(rnd(23, 1, 2, 6), (20, 2, 6)).copy()
    g = rnd(24, 20, 4, 6)
    for causal in (False, True):
        dq, dk, _ = impl(q, k, v, g, cu, causal, 0.9)
        assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12, causal


def pin_one_key_sequence(impl):
    cu = np.array([0, 1, 2, 3], np.int32)
    q, k, v = rnd(31, 3, 4, 5), rnd(32, 3, 2, 5), rnd(33, 3, 2, 5)
    g = rnd(34, 3, 4, 5)
    dq, dk, dv = impl(q, k, v, g, cu, False, 1.3)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    want = g.reshape(3, 2, 2, 5).sum(axis=2)  # heads 0,1 -> kv 0; heads 2,3 -> kv 1
    assert np.abs(dv - want).max() < 1e-14


def pin_sums(impl):
    """sum_j dK_j = 0 and sum_j dV_j = sum of dout over non-empty rows, per (sequence, kv head)."""
    cu = np.array([0, 33, 33, 70], np.int32)
    q, k, v = rnd(41, 70, 4, 8), rnd(42, 70, 2, 8), rnd(43, 70, 2, 8)
    g = rnd(44, 70, 4, 8)
    vis = np.random.default_rng(45).random((3, 2, 5, 5)) < 0.5
    vis[:, :, 0, :] = False  # query block 0 sees nothing: its rows are empty
    m = pack_mask(vis)
    for causal, mask in ((False, None), (True, None), (True, m), (False, m)):
        _, dk, dv = impl(q, k, v, g, cu, causal, 0.6, mask, 8)
        for b in range(3):
            s0, e0 = int(cu[b]), int(cu[b + 1])
            for c in range(2):
                assert np.abs(dk[s0:e0, c].sum(0)).max() < 1e-12, (b, c, causal)
                gsum = np.zeros(8)
                for i in range(e0 - s0):
                    seen = np.arange(i + 1 if causal else e0 - s0)
                    if mask is not None:
                        seen = seen[vis[b, c, i // 8, seen // 8]]
                    if len(seen):
                        gsum += g[s0 + i, 2 * c] + g[s0 + i, 2 * c + 1]
                assert np.abs(dv[s0:e0, c].sum(0) - gsum).max() < 1e-12, (b, c, causal)


def pin_scale_derivative(impl):
    """sum_i q_i.dQ_i = sum_j k_j.dK_j = scale * dLoss/dscale."""
    cu = np.array([0, 12, 30], np.int32)
    q, k, v = rnd(51, 30, 2, 4), rnd(52, 30, 1, 4), rnd(53, 30, 1, 4)
    g = rnd(54, 30, 2, 4)
    for causal in (False, True):
        scale = 0.8
        dq, dk, _ = impl(q, k, v, g, cu, causal, scale)
        a = float((q * dq).sum())
        b = float((k * dk).sum())
        h = 1e-6
        fd = (fwd_loss(q, k, v, g, cu, causal, scale + h) - fwd_loss(q, k, v, g, cu, causal, scale - h)) / (2 * h)
        assert abs(a - b) < 1e-12 and abs(a - scale * fd) < 1e-7, (causal, a, b, scale * fd)


def pin_gqa_is_repeated_mha(impl):
    cu = np.array([0, 25], np.int32)
    q, k, v = rnd(61, 25, 6, 4), rnd(62, 25, 2, 4), rnd(63, 25, 2, 4)
    g = rnd(64, 25, 6, 4)
    dq, dk, dv = impl(q, k, v, g, cu, True, 0.5)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    dq2, dk2, dv2 = impl(q, kr, vr, g, cu, True, 0.5)
    assert np.abs(dq - dq2).max() < 1e-13
    assert np.abs(dk - dk2.reshape(25, 2, 3, 4).sum(2)).max() < 1e-13
    assert np.abs(dv - dv2.reshape(25, 2, 3, 4).sum(2)).max() < 1e-13


def pin_packed_is_per_sequence(impl):
    cu = np.array([0, 7, 7, 19, 30], np.int32)
    q, k, v = rnd(71, 30, 2, 4), rnd(72, 30, 2, 4), rnd(73, 30, 2, 4)
    g = rnd(74, 30, 2, 4)
    for causal in (False, True):
        got = impl(q, k, v, g, cu, causal, 0.5)
        for b in range(4):
            s0, e0 = int(cu[b]), int(cu[b + 1])
            if e0 == s0:
                continue
            one = impl(q[s0:e0], k[s0:e0], v[s0:e0], g[s0:e0], np.array([0, e0 - s0], np.int32), causal, 0.5)
            for a, r in zip(got, one):
                assert np.abs(a[s0:e0] - r).max() < 1e-13, (b, causal)


def pin_linear_in_dout(impl):
    cu = np.array([0, 21], np.int32)
    q, k, v = rnd(81, 21, 2, 4), rnd(82, 21, 1, 4), rnd(83, 21, 1, 4)
    g1, g2 = rnd(84, 21, 2, 4), rnd(85, 21, 2, 4)
    r1 = impl(q, k, v, g1, cu, True, 0.5)
    r2 = impl(q, k, v, g2, cu, True, 0.5)
    r3 = impl(q, k, v, 2.0 * g1 - 3.0 * g2, cu, True, 0.5)
    for a, b, c in zip(r1, r2, r3):
        assert np.abs(2.0 * a - 3.0 * b - c).max() < 1e-12


def pin_full_mask_is_dense(impl):
    cu = np.array([0, 20, 37], np.int32)
    q, k, v = rnd(91, 37, 2, 4), rnd(92, 37, 2, 4), rnd(93, 37, 2, 4)
    g = rnd(94, 37, 2, 4)
    full = pack_mask(np.ones((2, 2, 5, 5), bool))
    for causal in (False, True):
        a = impl(q, k, v, g, cu, causal, 0.5)
        b = impl(q, k, v, g, cu, causal, 0.5, full, 4)
        for x, y in zip(a, b):
            assert np.abs(x - y).max() < 1e-14


PINS = [pin_finite_differences, pin_torch_autograd, pin_constant_v, pin_one_key_sequence, pin_sums,
        pin_scale_derivative, pin_gqa_is_repeated_mha, pin_packed_is_per_sequence,
        pin_linear_in_dout, pin_full_mask_is_dense]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_bwd_passes(pin):
    pin(oracle_impl)


def test_oracle_bwd_rejects_bad_arguments():
    q = np.zeros((4, 3, 2))
    k = np.zeros((4, 2, 2))
    with pytest.raises(RuntimeError):  # Hq not a multiple of Hkv
        oracle.attn_bwd(q, k, k, q, np.array([0, 4], np.int32), False, 1.0)
    with pytest.raises(ValueError):  # dout shape differs from q
        oracle.attn_bwd(np.zeros((4, 2, 2)), k, k, np.zeros((4, 2, 3)), np.array([0, 4], np.int32), False, 1.0)


# ----------------------------------------------------------------------------
# Planted mistakes: a numpy copy of the gradient formulas with one bug each.
# ----------------------------------------------------------------------------
def mutant(bug):
    def impl(q, k, v, dout, cu, causal, scale, block_mask=None, block=128):
        T, hq, d = q.shape
        hkv = k.shape[1]
        grp = hq // hkv
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        segs = [(0, T)] if bug == "varlen_leak" else [(int(cu[b]), int(cu[b + 1])) for b in range(len(cu) - 1)]
        for b, (s0, e0) in enumerate(segs):
            L = e0 - s0
            if L == 0:
                continue
            for h in range(hq):
                c = (h % hkv) if bug == "gqa_mod" else h // grp
                s = scale * q[s0:e0, h] @ k[s0:e0, c].T
                ii = np.arange(L)[:, None]
                jj = np.arange(L)[None, :]
                allowed = np.ones((L, L), bool)
                if causal:
                    allowed &= (jj < ii) if bug == "causal_strict" else (jj <= ii)
                if block_mask is not None and bug != "mask_ignored":
                    mb = block_mask[b if block_mask.shape[0] > 1 else 0, c if block_mask.shape[1] > 1 else 0]
                    qb, kb = ii // block, jj // block
                    allowed &= ((mb[qb, kb // 32] >> (kb % 32).astype(np.uint32)) & 1).astype(bool)
                rows = allowed.any(1)
                sm = np.where(allowed, s if bug != "p_unscaled" else s / scale, -np.inf)
                sm[~rows] = 0.0
                p = np.exp(sm - sm.max(1, keepdims=True))
                p /= p.sum(1, keepdims=True)
                p[~rows] = 0.0
                go = dout[s0:e0, h]
                vv = v[s0:e0, c]
                dp = go @ vv.T
                D = (p * dp).sum(1, keepdims=True)
                if bug == "no_D":
                    D = 0.0 * D
                ds = p * (dp - D) if bug != "ds_sign" else p * (D - dp)
                dq[s0:e0, h] += (1.0 if bug == "dq_no_scale" else scale) * ds @ (vv if bug == "dq_uses_v" else k[s0:e0, c])
                dk[s0:e0, c] += scale * (ds if bug != "dk_untransposed" else ds.T).T @ q[s0:e0, h]
                dv[s0:e0, c] += (p if bug != "dv_untransposed" else p.T).T @ go
        return dq, dk, dv
    return impl


BWD_MUTANTS = ["varlen_leak", "gqa_mod", "causal_strict", "mask_ignored", "p_unscaled", "no_D",
               "ds_sign", "dq_no_scale", "dq_uses_v", "dk_untransposed", "dv_untransposed"]


def test_clean_numpy_copy_passes_bwd_pins():
    impl = mutant(None)
    for pin in PINS:
        pin(impl)


@pytest.mark.parametrize("bug", BWD_MUTANTS)
def test_bwd_pins_catch_planted_mistake(bug):
    impl = mutant(bug)
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(impl)
            except (AssertionError, ValueError, IndexError):
                caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {bug!r}"
