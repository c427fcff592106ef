"""Pins for the oracle's bit-packed block-mask mode (one mask per sequence and
KV head, 32 blocks per 32-bit word; the bit-packed block masks of the
AdaSplash-2 explainer, section 2).

Each ``pin_*`` takes ``impl(q, k, v, cu, causal, scale, mask, block) -> (O, LSE)``
(packed float64 tensors; mask uint32 [n_seqs|1, Hkv|1, n_qblk, words]) and
raises AssertionError on disagreement with what mathematics fixes:
* membership   Q = 0 gives LSE = ln |A(i)| with |A(i)| counted here from the
               mask bits (decoded with numpy's unpackbits, not the oracle's
               shifts); one-hot V gives |A(i) ∩ block| / |A(i)|
* formula      brute force in plain Python (math.fsum, no max subtraction)
* encodings    a mask built from a block list equals the list (oracle list
               path, itself pinned in test_oracle_pins.py)
* selection    per-sequence masks in a packed batch equal per-sequence runs;
               per-head masks equal running each KV head on its own
Planted mistakes in a numpy copy (bottom) must each fail at least one pin.
"""
import math

import numpy as np
import pytest

import attn_workloads as W
import oracle


def oracle_impl(q, k, v, cu, causal, scale, mask, block):
    return oracle.attn_fwd(q, k, v, cu, causal, scale, block=block, nthreads=4, block_mask=mask)


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def decode(mask):
    """bool [..., n_qblk, 32*words] from the packed words (independent of the oracle)."""
    return np.unpackbits(np.ascontiguousarray(mask, dtype=np.uint32).view(np.uint8), axis=-1,
                         bitorder="little").astype(bool)


def random_mask(seed, n_sets_s, n_sets_h, n_qblk, n_kblk, p=0.5, diag=True):
    rng = np.random.default_rng(seed)
    vis = rng.random((n_sets_s, n_sets_h, n_qblk, n_kblk)) < p
    if diag:
        for qb in range(min(n_qblk, n_kblk)):
            vis[..., qb, qb] = True
    return W.pack_block_mask(vis)


def allowed(i, L, causal, vis_row, block):
    return [j for j in range(L) if (not causal or j <= i) and vis_row[j // block]]


# ---------------------------------------------------------------------------- pins
def pin_mask_q0_counts(impl):
    """Per-sequence and per-head masks, Q = 0: LSE_i = ln |A(i)|."""
    block, hq, hkv, d = 8, 4, 2, 4
    lengths = [37, 20]
    cu = np.array([0, 37, 57], np.int32)
    n_qblk = 5
    mask = random_mask(1, 2, hkv, n_qblk, n_qblk)
    vis = decode(mask)
    q = np.zeros((57, hq, d))
    k = rnd(2, 57, hkv, d)
    v = rnd(3, 57, hkv, d)
    for causal in (False, True):
        O, LSE = impl(q, k, v, cu, causal, 0.5, mask, block)
        for b, L in enumerate(lengths):
            for h in range(hq):
                c = h // (hq // hkv)
                for i in range(L):
                    A = allowed(i, L, causal, vis[b, c, i // block], block)
                    t = cu[b] + i
                    if not A:
                        assert LSE[t, h] == -np.inf and np.all(O[t, h] == 0)
                        continue
                    assert abs(LSE[t, h] - math.log(len(A))) <= 1e-12
                    mean = v[cu[b] + np.array(A), c].mean(axis=0)
                    assert np.abs(O[t, h] - mean).max() <= 1e-12


def pin_mask_one_hot(impl):
    """Q = 0 and V[:, c, 0] = 1 on one block: O_i[0] = |A(i) ∩ block| / |A(i)| per head."""
    block, hq, hkv, d, L = 8, 2, 2, 2, 40
    cu = np.array([0, L], np.int32)
    mask = random_mask(4, 1, hkv, 5, 5, p=0.4)
    vis = decode(mask)
    q = np.zeros((L, hq, d))
    k = rnd(5, L, hkv, d)
    for target in range(5):
        v = np.zeros((L, hkv, d))
        v[target * block:(target + 1) * block, :, 0] = 1.0
        O, _ = impl(q, k, v, cu, True, 1.0, mask, block)
        for h in range(hq):
            for i in range(L):
                A = allowed(i, L, True, vis[0, h, i // block], block)
                inside = sum(1 for j in A if j // block == target)
                expect = inside / len(A) if A else 0.0
                assert abs(O[i, h, 0] - expect) <= 1e-12, (target, h, i)


def pin_mask_brute_force(impl):
    """Textbook formula in plain Python: no max subtraction, math.fsum."""
    block, hq, hkv, d, L = 4, 2, 1, 3, 13
    cu = np.array([0, L], np.int32)
    mask = random_mask(6, 1, 1, 4, 4, p=0.6)
    vis = decode(mask)
    q, k, v = rnd(7, L, hq, d), rnd(8, L, hkv, d), rnd(9, L, hkv, d)
    scale = 0.7
    for causal in (False, True):
        O, LSE = impl(q, k, v, cu, causal, scale, mask, block)
        for h in range(hq):
            for i in range(L):
                A = allowed(i, L, causal, vis[0, 0, i // block], block)
                w = [math.exp(scale * math.fsum(q[i, h, e] * k[j, 0, e] for e in range(d))) for j in A]
                Z = math.fsum(w)
                assert abs(LSE[i, h] - math.log(Z)) <= 1e-12
                for e in range(d):
                    o = math.fsum(wj * v[j, 0, e] for wj, j in zip(w, A)) / Z
                    assert abs(O[i, h, e] - o) <= 1e-12


def pin_mask_equals_list(impl):
    """The bit-packed form of a block list gives the list's result."""
    block, hq, hkv, d, L = 8, 2, 2, 4, 48
    cu = np.array([0, L], np.int32)
    rows = [[0], [1, 0], [2], [3, 1], [0, 4, 2], [5, 3, 0]]
    row_ptr = np.zeros(len(rows) + 1, np.int32)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col_idx = np.array([c for r in rows for c in r], np.int32)
    mask = W.pack_block_mask(W.list_visibility(row_ptr, col_idx, 6)[None, None])
    q, k, v = rnd(10, L, hq, d), rnd(11, L, hkv, d), rnd(12, L, hkv, d)
    for causal in (False, True):
        O1, L1 = impl(q, k, v, cu, causal, 0.4, mask, block)
        O2, L2 = oracle.attn_fwd(q, k, v, cu, causal, 0.4, row_ptr, col_idx, block, nthreads=2)
        assert np.abs(O1 - O2).max() <= 1e-12 and np.abs(L1 - L2).max() <= 1e-12


def pin_mask_selection(impl):
    """Packed run with per-sequence masks = separate runs; per-head masks = one run per KV head."""
    block, hq, hkv, d = 8, 4, 2, 4
    cu = np.array([0, 30, 47], np.int32)
    mask = random_mask(13, 2, hkv, 4, 4, p=0.5)
    q, k, v = rnd(14, 47, hq, d), rnd(15, 47, hkv, d), rnd(16, 47, hkv, d)
    O, LSE = impl(q, k, v, cu, True, 0.6, mask, block)
    g = hq // hkv
    for b in range(2):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        for c in range(hkv):
            hs = slice(c * g, (c + 1) * g)
            Ob, Lb = impl(q[s0:s1, hs], k[s0:s1, c:c + 1], v[s0:s1, c:c + 1],
                          np.array([0, s1 - s0], np.int32), True, 0.6, mask[b:b + 1, c:c + 1], block)
            assert np.abs(O[s0:s1, hs] - Ob).max() <= 1e-12
            assert np.abs(LSE[s0:s1, hs] - Lb).max() <= 1e-12


PINS = [pin_mask_q0_counts, pin_mask_one_hot, pin_mask_brute_force, pin_mask_equals_list,
        pin_mask_selection]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_passes_mask_pin(pin):
    pin(oracle_impl)


def test_oracle_rejects_bad_mask_arguments():
    q = np.zeros((20, 2, 2))
    k = np.zeros((20, 1, 2))
    cu = np.array([0, 20], np.int32)
    with pytest.raises(RuntimeError):  # too few rows for ceil(20/8) = 3 query blocks
        oracle.attn_fwd(q, k, k, cu, True, 1.0, block=8, block_mask=np.zeros((1, 1, 2, 1), np.uint32))
    with pytest.raises(ValueError):  # a list and a mask together
        oracle.attn_fwd(q, k, k, cu, True, 1.0, np.array([0, 1, 1, 1], np.int32), np.array([0], np.int32), 8,
                        block_mask=np.zeros((1, 1, 3, 1), np.uint32))


def test_pack_block_mask_bit_order():
    vis = np.zeros((1, 1, 2, 40), bool)
    vis[0, 0, 0, [0, 31, 32, 39]] = True
    vis[0, 0, 1, 5] = True
    m = W.pack_block_mask(vis)
    assert m.shape == (1, 1, 2, 2)
    assert m[0, 0, 0, 0] == (1 | (1 << 31)) and m[0, 0, 0, 1] == (1 | (1 << 7))
    assert m[0, 0, 1, 0] == (1 << 5) and m[0, 0, 1, 1] == 0


# ---------------------------------------------------------------------------- planted mistakes
def mutant(bug):
    def impl(q, k, v, cu, causal, scale, mask, block):
        T, hq, d = q.shape
        hkv = k.shape[1]
        g = hq // hkv
        O = np.zeros((T, hq, d))
        LSE = np.full((T, hq), -np.inf)
        for b in range(len(cu) - 1):
            s0, e0 = int(cu[b]), int(cu[b + 1])
            L = e0 - s0
            for h in range(hq):
                c = h // g
                ms = 0 if (mask.shape[0] == 1 or bug == "seq_shared") else b
                mh = 0 if (mask.shape[1] == 1 or bug == "head_shared") else (h % mask.shape[1] if bug == "head_from_q" else c)
                words = mask[ms, mh]
                s = scale * q[s0:e0, h] @ k[s0:e0, c].T
                for i in range(L):
                    qb = i // block
                    if bug == "qblock_off":
                        qb = max(qb - 1, 0)
                    ok = np.zeros(L, bool)
                    for j in range(L):
                        kb = j // block
                        bit = 31 - kb % 32 if bug == "bit_reversed" else kb % 32
                        vis = (int(words[qb, kb // 32]) >> bit) & 1
                        if bug == "mask_ignored":
                            vis = 1
                        ok[j] = bool(vis) and (not causal or j <= i)
                    if not ok.any():
                        continue
                    si = np.where(ok, s[i], -np.inf)
                    m = si.max()
                    w = np.exp(si - m)
                    Z = w.sum()
                    O[s0 + i, h] = (w / Z) @ v[s0:e0, c]
                    LSE[s0 + i, h] = m + np.log(Z)
        return O, LSE
    return impl


MASK_MUTANTS = ["seq_shared", "head_shared", "head_from_q", "qblock_off", "bit_reversed", "mask_ignored"]


def test_clean_mask_copy_passes_pins():
    for pin in PINS:
        pin(mutant(None))


@pytest.mark.parametrize("bug", MASK_MUTANTS)
def test_mask_pins_catch_planted_mistake(bug):
    impl = mutant(bug)
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(impl)
            except AssertionError:
                caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {bug!r}"
