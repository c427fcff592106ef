"""GPU parity of the attention backward (dq, dk, dv) against the fp64 oracle.

Each case runs the GPU forward, then the GPU backward through the C ABI
(attn_bwd via the binding), on seeded bf16 inputs and a seeded bf16 dO, and
compares every gradient element with ``oracle.attn_bwd`` on the same inputs
(rel-RMS and max-relative bounds of tests/_parity.py).
"""
import numpy as np
import pytest

import attn_workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu


def check(w, layout="bshd"):
    do = W.make_dout(w)
    print(f"bwd case {w.name}", flush=True)
    got = P.run_gpu_bwd(w, do, layout)
    ref = P.oracle_bwd(w, do)
    stats = P.compare_grads(got, ref, w.name)
    print(f"  {stats}", flush=True)
    return got, ref


DENSE = [
    # name, seed, B, S, Hq, Hkv, D, causal
    ("b_tiny", 41, 1, 128, 2, 2, 64, False),
    ("b_causal_ragged", 42, 2, 300, 4, 4, 128, True),
    ("b_noncausal_ragged", 43, 2, 200, 2, 2, 128, False),
    ("b_gqa", 44, 1, 257, 8, 2, 128, True),
    ("b_d64_causal", 45, 2, 389, 4, 1, 64, True),
    ("b_short", 46, 3, 17, 2, 1, 128, True),
    ("b_d256_causal_ragged", 58, 2, 300, 4, 2, 256, True),
    ("b_d256_noncausal", 59, 1, 257, 2, 1, 256, False),
    ("b_d256_gqa_short", 60, 2, 45, 8, 2, 256, True),
]


@pytest.mark.parametrize("case", DENSE, ids=[c[0] for c in DENSE])
def test_bwd_dense(case):
    name, seed, b, s, hq, hkv, d, causal = case
    check(W.make_dense(name, seed, b, s, hq, hkv, d, causal))


def test_bwd_strided_layout():
    check(W.make_dense("b_bhsd", 47, 2, 190, 4, 2, 128, True), layout="bhsd")


VARLEN = [
    ("bv_mixed_causal", 48, [1, 127, 128, 129, 300, 64], 4, 2, 128, True),
    ("bv_mixed_dense", 49, [200, 0, 65, 256], 2, 2, 64, False),
    ("bv_gqa_d64", 50, [513, 31, 128], 8, 2, 64, True),
    ("bv_gqa_d256", 61, [400, 1, 129, 260], 4, 2, 256, True),
]


@pytest.mark.parametrize("case", VARLEN, ids=[c[0] for c in VARLEN])
def test_bwd_varlen(case):
    name, seed, lens, hq, hkv, d, causal = case
    check(W.make_varlen(name, seed, lens, hq, hkv, d, causal))


def masked(name, seed, b, s, hq, hkv, d, causal, per_seq, per_head, density, lens=None):
    """Dense or packed workload with a random block mask."""
    if lens is None:
        w = W.make_dense(name, seed, b, s, hq, hkv, d, causal)
    else:
        w = W.make_varlen(name, seed, lens, hq, hkv, d, causal)
        b, s = len(lens), int(max(lens))
    n_blk = -(-s // 128)
    rng = np.random.default_rng(seed + 1000)
    vis = rng.random((b if per_seq else 1, hkv if per_head else 1, n_blk, n_blk)) < density
    w.block_mask = W.pack_block_mask(vis)
    return w


MASKED = [
    ("bm_causal_heads", 51, 2, 700, 4, 2, 128, True, True, True, 0.5, None),
    ("bm_dense_shared", 52, 1, 600, 2, 2, 64, False, False, False, 0.4, None),
    ("bm_varlen", 53, 0, 0, 4, 2, 128, True, True, True, 0.6, [300, 513, 129]),
    ("bm_sparse", 54, 1, 1100, 2, 1, 128, False, False, False, 0.15, None),
    ("bm_d256_causal_heads", 62, 2, 520, 4, 2, 256, True, True, True, 0.5, None),
    ("bm_d256_varlen", 63, 0, 0, 2, 1, 256, False, True, False, 0.6, [300, 140]),
]


@pytest.mark.parametrize("case", MASKED, ids=[c[0] for c in MASKED])
def test_bwd_block_mask(case):
    check(masked(*case))


def test_bwd_mask_empty_rows_and_columns():
    """Query blocks that see no key block get dq = 0; key blocks no query sees get dk = dv = 0."""
    w = W.make_dense("bm_empty", 55, 1, 512, 2, 2, 128, False)
    vis = np.ones((1, 1, 4, 4), bool)
    vis[0, 0, 1, :] = False   # query block 1 sees nothing
    vis[0, 0, :, 2] = False   # key block 2 is seen by nobody
    w.block_mask = W.pack_block_mask(vis)
    got, _ = check(w)
    dq, dk, dv = got
    assert np.all(dq[128:256] == 0)
    assert np.all(dk[256:384] == 0) and np.all(dv[256:384] == 0)


@pytest.mark.parametrize("d", [128, 256])
def test_bwd_deterministic(d):
    w = W.make_dense("b_det", 56, 2, 333, 4, 2, d, True)
    runs = P.run_gpu_bwd(w, W.make_dout(w), repeat=2)
    for a, b in zip(runs[0], runs[1]):
        assert np.array_equal(a, b)


def test_bwd_full_mask_equals_causal():
    w = W.make_dense("b_full", 57, 1, 500, 2, 2, 128, True)
    do = W.make_dout(w)
    plain = P.run_gpu_bwd(w, do)
    w.block_mask = W.pack_block_mask(np.ones((1, 1, 4, 4), bool))
    full = P.run_gpu_bwd(w, do)
    for a, b in zip(plain, full):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["mha", "gqa"])
def test_bwd_full_size_sampled_units(name):
    """Full-size workloads (the forward's configurations) through the GPU
    backward; the oracle recomputes two (sequence, KV head) units exactly, one
    query head per thread (dk and dv summed over the group's heads)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from attn_workloads import bf16_bits_to_f32

    w = W.make(name)
    do = W.make_dout(w)
    print(f"bwd full {name}", flush=True)
    dq, dk, dv = P.run_gpu_bwd(w, do)
    g = w.hq // w.hkv
    f = lambda a: bf16_bits_to_f32(a).astype(np.float64)
    S = w.seqlen
    cu = np.array([0, S], np.int32)
    units = [(0, 1), (w.batch - 1, w.hkv - 1)]

    def one_head(b, h):
        c = h // g
        return oracle.attn_bwd(f(w.q[b, :, h:h + 1]), f(w.k[b, :, c:c + 1]), f(w.v[b, :, c:c + 1]),
                               f(do[b, :, h:h + 1]), cu, w.causal, w.scale, nthreads=1)

    jobs = [(b, c * g + j) for b, c in units for j in range(g)]
    with ThreadPoolExecutor(max_workers=min(16, len(jobs))) as ex:
        parts = list(ex.map(lambda bh: one_head(*bh), jobs))
    for b, c in units:
        mine = [parts[i] for i, (bb, h) in enumerate(jobs) if bb == b and h // g == c]
        ref = (np.concatenate([m[0] for m in mine], axis=1), sum(m[1] for m in mine), sum(m[2] for m in mine))
        rows = slice(b * S, (b + 1) * S)
        got = (dq[rows, c * g:(c + 1) * g], dk[rows, c:c + 1], dv[rows, c:c + 1])
        print(f"  unit b={b} kv={c}: {P.compare_grads(got, ref, name)}", flush=True)


# ---------------------------------------------------------------------------
# The backward of a forward that took a block list (the mask of the list's set)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed,s", [(60, 700), (61, 128), (62, 129), (63, 1100)])
def test_block_list_to_mask_matches_host(seed, s):
    """attn_block_list_to_mask against the host's packing of the list's set (bit-exact):
    random order, ids above the diagonal and outside the sequence, repeated ids,
    an empty row."""
    import torch
    import attention_forward_flashattention_amd as attn
    from tests.test_parity_gpu import random_list

    n = (s + 127) // 128
    row_ptr, col_idx = random_list(seed, n, n, p=0.5, empty_row=1 if n > 1 else None)
    if len(col_idx):                      # a repeated id in the first row
        col_idx = np.insert(col_idx, row_ptr[1], col_idx[0]).astype(np.int32)
        row_ptr = row_ptr.copy()
        row_ptr[1:] += 1
    dev = torch.device("cuda:0")
    bl = (torch.from_numpy(row_ptr).to(dev), torch.from_numpy(col_idx.astype(np.int32)).to(dev))
    got = attn.block_list_to_mask(bl, s).cpu().numpy().view(np.uint32).reshape(n, -1)
    want = W.pack_block_mask(W.list_visibility(row_ptr, col_idx, n))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_bwd_block_list(d):
    """Forward with a block list, backward with the same list: equal bit for bit to the
    backward with the mask of the list's set, and within the gradient bounds of the
    oracle's backward on that set."""
    import torch
    import attention_forward_flashattention_amd as attn
    from tests.test_parity_gpu import random_list

    s = 650
    w = W.make_dense(f"b_list_d{d}", 64, 1, s, 4, 2, d, True)
    n = (s + 127) // 128
    w.row_ptr, w.col_idx = random_list(65, n, n, p=0.5, empty_row=2)
    print(f"bwd block list d={d}", flush=True)
    do_bits = W.make_dout(w)
    q, k, v, _, sp = P.to_device(w)
    do = P.bf16_tensor(do_bits, q.device)
    out, lse = attn.attn_fwd(q, k, v, causal=True, scale=w.scale, **sp)
    g_list = attn.attn_bwd(q, k, v, out, do, lse, causal=True, scale=w.scale, block_list=sp["block_list"])
    vis = W.list_visibility(w.row_ptr, w.col_idx, n)
    mask = torch.from_numpy(W.pack_block_mask(vis[None, None]).view(np.int32)).to(q.device)
    g_mask = attn.attn_bwd(q, k, v, out, do, lse, causal=True, scale=w.scale, block_mask=mask)
    torch.cuda.synchronize()
    for a, b in zip(g_list, g_mask):
        assert torch.equal(a, b)
    got = tuple(x.float().cpu().numpy().astype(np.float64).reshape(s, x.shape[-2], d) for x in g_list)
    w.row_ptr = w.col_idx = None
    w.block_mask = W.pack_block_mask(vis[None, None])
    ref = P.oracle_bwd(w, do_bits)
    print(f"  {P.compare_grads(got, ref, w.name)}", flush=True)
