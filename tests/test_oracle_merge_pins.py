"""Pin of the oracle's LSE through the exact merge of key-disjoint partial results.

When the keys of every row are split into disjoint parts (as a multi-device
split of the sequence would do) and attention is computed over each part
alone, the full result follows exactly from the parts:

    LSE = ln sum_r exp(LSE_r),    O = sum_r exp(LSE_r - LSE) O_r

(a part with no visible key has LSE_r = -inf and adds nothing).  This holds
only if LSE is the natural-log log-sum-exp of the scaled scores over exactly
the visible keys, so it pins the oracle's LSE (base, scale, allowed set) and
its block-mask handling against its own unmasked result.  A base-2 LSE, or
a merge that ignores the LSE weights, fails it.
"""
import numpy as np
import pytest

import oracle


def pack_mask(vis):
    """bool [n_qblk, n_kblk] -> uint32 [1, 1, n_qblk, words] (bit kb % 32 of word kb // 32)."""
    n_qblk, n_kblk = vis.shape
    words = (n_kblk + 31) // 32
    m = np.zeros((1, 1, n_qblk, words), np.uint32)
    for kb in range(n_kblk):
        m[0, 0, :, kb // 32] |= vis[:, kb].astype(np.uint32) << np.uint32(kb % 32)
    return m


def merge(os_, ls_, base=np.e, weighted=True):
    ls = np.stack(ls_) / np.log(base)  # natural-log LSEs read in another base when base != e
    lse = np.logaddexp.reduce(ls, axis=0)
    with np.errstate(invalid="ignore"):
        w = np.where(np.isneginf(ls), 0.0, np.exp(ls - lse[None]))
    if not weighted:
        w = np.where(np.isneginf(ls), 0.0, 1.0) / np.maximum(1, (~np.isneginf(ls)).sum(0))[None]
    return np.einsum("rth,rthd->thd", w, np.stack(os_)), lse


CASES = [
    # cu_seqlens, hq, hkv, d, causal, block, parts
    ([0, 45], 4, 2, 8, True, 4, 3),
    ([0, 23, 61], 2, 1, 16, True, 4, 2),
    ([0, 37], 2, 2, 8, False, 8, 4),
]


def parts_of(case_i, n_kblk, parts):
    """Disjoint part of every KV block: a seeded shuffle dealt round-robin."""
    rng = np.random.default_rng(100 + case_i)
    order = rng.permutation(n_kblk)
    owner = np.empty(n_kblk, np.int64)
    owner[order] = np.arange(n_kblk) % parts
    return owner


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_lse_merge_of_key_parts_is_exact(ci):
    cu, hq, hkv, d, causal, block, parts = CASES[ci]
    cu = np.array(cu, np.int32)
    t = int(cu[-1])
    rng = np.random.default_rng(7 + ci)
    q, k, v = (rng.standard_normal((t, h, d)) for h in (hq, hkv, hkv))
    scale = 0.7
    o_full, l_full = oracle.attn_fwd(q, k, v, cu, causal, scale, nthreads=2)
    max_len = int(np.max(np.diff(cu)))
    n_blk = (max_len + block - 1) // block
    owner = parts_of(ci, n_blk, parts)
    os_, ls_ = [], []
    for r in range(parts):
        vis = np.broadcast_to(owner[None, :] == r, (n_blk, n_blk))
        o_r, l_r = oracle.attn_fwd(q, k, v, cu, causal, scale, block=block, block_mask=pack_mask(vis), nthreads=2)
        os_.append(o_r)
        ls_.append(l_r)
    # under causal masking some row of some part sees no key at all (the
    # part's blocks all lie after it): the -inf case is exercised
    if causal:
        assert any(np.isneginf(l).any() for l in ls_)
    o_m, l_m = merge(os_, ls_)
    assert np.abs(l_m - l_full).max() < 1e-12
    assert np.abs(o_m - o_full).max() < 1e-12
    # the pin is sensitive: a base-2 reading of the LSE or an unweighted merge fails
    o_b2, l_b2 = merge(os_, ls_, base=2.0)
    assert np.abs(o_b2 - o_full).max() > 1e-3 or np.abs(l_b2 - l_full).max() > 1e-3
    o_uw, _ = merge(os_, ls_, weighted=False)
    assert np.abs(o_uw - o_full).max() > 1e-3
