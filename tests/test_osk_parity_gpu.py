"""GPU parity of ordered skipping (attn_fwd_osk) against the fp64 oracle.

The stop of each (query head, query block) is an integer decided by floating
point: the GPU forms the test in fp32, the oracle in fp64.  So the GPU's
visited counts are checked to be valid stops of the rule (within a relative
band around tau, against the oracle's fp64 test values), and the GPU output
is compared with the oracle's exact attention over the prefix the GPU
visited.  GPU-side pins: tau = 0 visits whole lists and equals the static
block-list kernel bitwise; a huge tau visits min_visit entries and equals
the static kernel on the cut list bitwise.
"""
import numpy as np
import pytest

import attn_workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu


def small(seed=31, s=6144, mu=6.0, budget=0.5, hq=4, hkv=2, d=128):
    return W.make_osk("osk_small", seed, s, hq, hkv, d, budget=budget, mu=mu)


# head configurations: pairs of query heads of one GQA group per workgroup
# (the pipelined loop, head_dim 64 and 128), an odd group and head_dim 256
# (one query head per workgroup, the plain loop)
SHAPES = [("pair_d128", 4, 2, 128, 6144), ("pair_d64", 4, 2, 64, 6144),
          ("single_g3_d128", 3, 1, 128, 4096), ("single_d256", 2, 1, 256, 3072)]


def static_list(w, row_ptr=None, col_idx=None):
    import torch
    import attention_forward_flashattention_amd as attn

    q, k, v, _, sp = P.to_device(w)
    if row_ptr is not None:
        sp = {"block_list": (torch.from_numpy(row_ptr).cuda(), torch.from_numpy(col_idx).cuda())}
    out, lse = attn.attn_fwd(q, k, v, causal=True, scale=w.scale, **sp)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().reshape(w.seqlen, w.hq, w.d), lse.cpu().numpy()[0].T


def _stops_and_prefix(w, tau, min_visit):
    o, l, vis = P.run_gpu_osk(w, tau, min_visit)
    n_qblk = len(w.row_ptr) - 1
    qbs = np.arange(n_qblk)
    ratio = P.osk_trace(w, qbs)
    P.check_visited(w, vis, ratio, tau, min_visit, qbs)
    lens = np.diff(w.row_ptr)
    skip = 1 - vis.sum() / (lens.sum() * w.hq)
    rows = P.sample_tokens(w, per_seq=160, seed=3)
    o_ref, l_ref = P.oracle_prefix_rows(w, vis, rows)
    stats = P.compare(o[rows], l[rows], o_ref, l_ref, f"osk tau={tau}")
    print(f"  skipped {skip:.3f} of the listed entries; {stats}", flush=True)


@pytest.mark.parametrize("tau,min_visit", [(1e-3, 2), (1e-2, 2), (5e-2, 3), (3e-1, 2)])
def test_osk_valid_stops_and_prefix_parity(tau, min_visit):
    print(f"osk small tau={tau} min_visit={min_visit}", flush=True)
    _stops_and_prefix(small(), tau, min_visit)


@pytest.mark.parametrize("shape", SHAPES[1:], ids=[c[0] for c in SHAPES[1:]])
def test_osk_shapes_valid_stops_and_prefix_parity(shape):
    name, hq, hkv, d, s = shape
    print(f"osk {name} tau=1e-2", flush=True)
    _stops_and_prefix(small(seed=35, s=s, hq=hq, hkv=hkv, d=d), 1e-2, 2)


@pytest.mark.parametrize("shape", SHAPES, ids=[c[0] for c in SHAPES])
def test_osk_tau_zero_is_the_static_list(shape):
    name, hq, hkv, d, s = shape
    print(f"osk {name} tau=0", flush=True)
    w = small(seed=32, s=s, hq=hq, hkv=hkv, d=d)
    o, l, vis = P.run_gpu_osk(w, 0.0, 1)
    assert np.array_equal(vis, np.broadcast_to(np.diff(w.row_ptr), vis.shape))
    o_s, l_s = static_list(w)
    assert np.array_equal(o, o_s) and np.array_equal(l, l_s)


@pytest.mark.parametrize("shape", SHAPES, ids=[c[0] for c in SHAPES])
def test_osk_huge_tau_is_the_cut_list(shape):
    name, hq, hkv, d, s = shape
    print(f"osk {name} huge tau", flush=True)
    w = small(seed=33, s=s, hq=hq, hkv=hkv, d=d)
    mv = 3
    o, l, vis = P.run_gpu_osk(w, 1e30, mv)
    want = np.minimum(np.diff(w.row_ptr), mv)
    assert np.array_equal(vis, np.broadcast_to(want, vis.shape))
    rp = np.zeros_like(w.row_ptr)
    ci = []
    for qb in range(len(w.row_ptr) - 1):
        ci.extend(w.col_idx[w.row_ptr[qb]:w.row_ptr[qb] + want[qb]])
        rp[qb + 1] = len(ci)
    o_s, l_s = static_list(w, rp, np.array(ci, np.int32))
    assert np.array_equal(o, o_s) and np.array_equal(l, l_s)


def test_osk_visited_monotone_in_tau():
    w = small(seed=34)
    prev = None
    for tau in (0.0, 1e-3, 1e-2, 1e-1, 1.0):
        _, _, vis = P.run_gpu_osk(w, tau, 2)
        if prev is not None:
            assert np.all(vis <= prev), tau
        prev = vis


def test_osk_full_size_sampled():
    """The 128K planted-relevance workload at tau = 1e-2: sampled query blocks'
    stops are valid and sampled rows match the oracle on the visited prefix."""
    w = W.make("sparse_osk")
    tau, mv = 1e-2, 2
    print("osk full size", flush=True)
    o, l, vis = P.run_gpu_osk(w, tau, mv)
    n_qblk = len(w.row_ptr) - 1
    qbs = np.array([0, 1, 2, 100, 511, n_qblk - 1], np.int32)
    ratio = P.osk_trace(w, qbs)
    P.check_visited(w, vis, ratio, tau, mv, qbs)
    lens = np.diff(w.row_ptr)
    print(f"  skipped {1 - vis.sum() / (lens.sum() * w.hq):.3f} of the listed entries", flush=True)
    rows = np.array(sorted(set(int(r) for r in w.sample_rows[:64]) | {0, 127, 128, w.seqlen - 1}), np.int64)
    o_ref, l_ref = P.oracle_prefix_rows(w, vis, rows)
    print(f"  {P.compare(o[rows], l[rows], o_ref, l_ref, 'osk full')}", flush=True)
