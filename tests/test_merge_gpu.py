"""The kernel on one device's share of a split problem (GPU).

* Keys split into disjoint parts (as a split of the sequence over devices
  would do): the kernel's per-part O and LSE, merged on the host with
  LSE = ln sum_r exp(LSE_r), O = sum_r exp(LSE_r - LSE) O_r, match the fp64
  oracle of the whole problem within the usual tolerances, including rows
  that see no key of some part (LSE_r = -inf, O_r = 0).
* Heads split over devices: the 128K block-sparse workload at one device's
  share when its 8 KV heads go to 8 devices (query heads 0-3 and KV head 0 of
  the same tensors, the same block list), checked on the sampled rows.
"""
import sys

import numpy as np
import pytest

import attn_workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def pack_mask(vis):
    n_qblk, n_kblk = vis.shape
    words = (n_kblk + 31) // 32
    m = np.zeros((1, 1, n_qblk, words), np.uint32)
    for kb in range(n_kblk):
        m[0, 0, :, kb // 32] |= vis[:, kb].astype(np.uint32) << np.uint32(kb % 32)
    return m


@pytest.mark.parametrize("causal", [True, False])
def test_lse_merge_of_kernel_key_parts(causal):
    w = W.make_dense("merge", 41, 1, 1100, 8, 2, 128, causal)
    n_blk = (w.seqlen + 127) // 128
    parts = 3
    owner = np.random.default_rng(5).permutation(n_blk) % parts
    note(f"merge causal={causal}: S={w.seqlen}, {parts} key parts over {n_blk} blocks")
    os_, ls_ = [], []
    for r in range(parts):
        w.block_mask = pack_mask(np.broadcast_to(owner[None, :] == r, (n_blk, n_blk)))
        o, l = P.run_gpu(w)
        os_.append(o)
        ls_.append(l)
    w.block_mask = None
    if causal:
        assert any(np.isneginf(l).any() for l in ls_)
    ls = np.stack(ls_)
    lse = np.logaddexp.reduce(ls, axis=0)
    wts = np.where(np.isneginf(ls), 0.0, np.exp(ls - lse[None]))
    o_m = np.einsum("rth,rthd->thd", wts, np.stack(os_))
    import oracle
    o_ref, l_ref = oracle.run_workload(w)
    stats = P.compare(o_m, lse, o_ref, l_ref, f"merge causal={causal}")
    note(f"  {stats}")


def test_sparse_head_share_sampled():
    full = W.make("sparse")
    w = W.Workload(name="sparse_share", seed=full.seed, batch=1, seqlen=full.seqlen, hq=4, hkv=1, d=full.d,
                   causal=True, scale=full.scale,
                   q=np.ascontiguousarray(full.q[:, :, 0:4]), k=np.ascontiguousarray(full.k[:, :, 0:1]),
                   v=np.ascontiguousarray(full.v[:, :, 0:1]), row_ptr=full.row_ptr, col_idx=full.col_idx,
                   sample_rows=full.sample_rows)
    del full
    note(f"sparse head share S={w.seqlen} Hq={w.hq} Hkv={w.hkv}: {len(w.sample_rows)} sampled rows")
    stats = P.check_workload(w, rows=w.sample_rows)
    note(f"  {stats}")
