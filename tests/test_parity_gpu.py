"""GPU parity: the HIP library against the fp64 oracle on the same seeded inputs.

Tolerances (bf16 I/O, fp32 accumulation): O max abs <= 2e-2, O mean abs
<= 2e-3, LSE max abs <= 1e-3, plus a relative RMS bound on O of 1e-2.
Small problems and the dense causal MHA and GQA workloads are compared on
every output; the packed variable-length workloads on every row of one query
head per KV head plus every head of sampled rows; the 128K block-sparse
workload on its 256 sampled rows (all heads), which the oracle computes one by
one.  Structural properties (GQA = repeated MHA, packed = per-sequence, list
= dense, run-to-run determinism) are checked bitwise where the kernel's
arithmetic is the same.
"""
import math
import sys

import numpy as np
import pytest

import attn_workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu

_cache = {}


def workload(name):
    if name not in _cache:
        _cache.clear()  # keep at most one large workload resident
        _cache[name] = W.make(name)
    return _cache[name]


def note(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- small cases, every output
SMALL = [
    # name, lengths (None = fixed B x S), B, S, hq, hkv, d, causal
    ("d64_dense_ragged", None, 2, 300, 4, 2, 64, False),
    ("d64_causal_ragged", None, 2, 300, 4, 2, 64, True),
    ("d128_dense_ragged", None, 1, 333, 4, 1, 128, False),
    ("d128_causal_ragged", None, 2, 390, 8, 2, 128, True),
    ("d256_causal_ragged", None, 1, 260, 2, 2, 256, True),
    ("d256_dense", None, 1, 256, 2, 1, 256, False),
    ("single_row", None, 1, 1, 2, 1, 128, True),
    ("seq_65", None, 3, 65, 2, 2, 64, True),
    ("varlen_d64", [1, 130, 64, 257, 0, 513], 0, 0, 4, 2, 64, True),
    ("varlen_d128", [200, 7, 384, 129], 0, 0, 8, 2, 128, True),
    ("varlen_d256_noncausal", [100, 300, 1], 0, 0, 4, 4, 256, False),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_full(case):
    name, lengths, b, s, hq, hkv, d, causal = case
    note(f"small case {name}")
    if lengths is None:
        w = W.make_dense(name, 11, b, s, hq, hkv, d, causal)
    else:
        w = W.make_varlen(name, 12, lengths, hq, hkv, d, causal)
    P.check_workload(w)


def test_tiny_workload():
    note("tiny workload B1 H2 S128 D64 non-causal")
    P.check_workload(W.make("tiny"))


def test_bhsd_layout_matches():
    """Strided [B,H,S,D] memory order gives the same bits as [B,S,H,D]."""
    w = W.make_dense("layout", 13, 2, 320, 4, 2, 128, True)
    o1, l1 = P.run_gpu(w, "bshd")
    o2, l2 = P.run_gpu(w, "bhsd")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------- full-size workloads, every output
@pytest.mark.parametrize("name", ["mha", "gqa"])
def test_workload_full(name):
    """Every row of every head of the dense causal workloads against the oracle."""
    w = workload(name)
    note(f"workload {name}: all {w.tokens} rows x {w.hq} heads")
    stats = P.check_workload(w)
    note(f"  {stats}")


@pytest.mark.parametrize("name", ["varlen_d64", "varlen_d128", "varlen_d256"])
def test_varlen_workload(name):
    """Packed variable-length workloads: every row of one query head per KV head
    (c*g + c mod g: every tile, wave and XCD slot of the schedule, and every head
    position within a GQA group), plus every head of sampled rows (tile edges and
    sequence ends of every sequence and random rows)."""
    w = workload(name)
    o, l = P.run_gpu(w)
    heads = P.one_head_per_kv_head(w)
    note(f"workload {name}: all {w.tokens} rows of heads {heads}")
    o_ref, l_ref = P.oracle_heads(w, heads)
    stats = P.compare(o[:, heads], l[:, heads], o_ref, l_ref, f"{name} heads {heads}")
    note(f"  {stats}")
    import oracle
    rows = P.sample_tokens(w, per_seq=48, seed=1)
    note(f"workload {name}: {len(rows)} sampled rows x {w.hq} heads")
    o_ref, l_ref = oracle.run_workload(w, rows=rows, nthreads=P.oracle_threads())
    stats = P.compare(o[rows], l[rows], o_ref, l_ref, f"{name} sampled rows")
    note(f"  {stats}")


def test_sparse_sampled():
    w = workload("sparse")
    note(f"sparse workload S={w.seqlen}: {len(w.sample_rows)} sampled rows x {w.hq} heads")
    stats = P.check_workload(w, rows=w.sample_rows)
    note(f"  {stats}")


# ---------------------------------------------------------------- pins repeated on the GPU
def test_zero_q_counts_dense_causal():
    """Q = 0: LSE_i = ln(i+1) and O_i = prefix mean of V (checked against the oracle)."""
    w = W.make_dense("zq", 14, 1, 1000, 2, 1, 128, True)
    w.q[:] = 0
    o, l = P.run_gpu(w)
    np.testing.assert_allclose(l[:, 0], np.log(np.arange(1, 1001)), rtol=0, atol=1e-5)
    vf = W.bf16_bits_to_f32(w.v[0, :, 0]).astype(np.float64)
    pref = np.cumsum(vf, axis=0) / np.arange(1, 1001)[:, None]
    assert np.abs(o[:, 0] - pref).max() <= 1e-2


def sparse_small(s=4096, seed=15, hq=4, hkv=1, d=128):
    g = W.streams(seed)
    nq = s // 128
    rp, ci = W.build_block_list(nq, g["block_scores"].random(size=(nq, nq)), 0.10)
    w = W.make_dense("sp", seed, 1, s, hq, hkv, d, True)
    w.row_ptr, w.col_idx = rp, ci
    return w


def test_zero_q_counts_block_list():
    """Q = 0 under a block list: LSE_i = ln(128 * #off-diagonal listed + (i mod 128) + 1)."""
    w = sparse_small()
    w.q[:] = 0
    _, l = P.run_gpu(w)
    rp, ci = w.row_ptr, w.col_idx
    for i in range(0, w.seqlen, 7):
        qb = i // 128
        off = int(np.sum(ci[rp[qb]:rp[qb + 1]] != qb))
        assert abs(l[i, 0] - math.log(128 * off + (i % 128) + 1)) <= 1e-5, i


def test_one_hot_membership_block_list():
    """Q = 0, V[:,0] = 1 on block c: O_i[0] = |A(i) ∩ c| / |A(i)|, exactly 0 iff c is not visible."""
    w = sparse_small(s=2048, hkv=1, hq=2)
    w.q[:] = 0
    rp, ci = w.row_ptr, w.col_idx
    for c in (0, 3, 9, 15):
        w.v[:] = 0
        w.v[0, c * 128:(c + 1) * 128, 0, 0] = W.f32_to_bf16_bits(np.ones(1, np.float32))[0]
        o, _ = P.run_gpu(w)
        for i in range(w.seqlen):
            qb = i // 128
            blocks = ci[rp[qb]:rp[qb + 1]]
            n_all = sum(min(128, i + 1 - b * 128) for b in blocks if b * 128 <= i)
            inside = min(128, i + 1 - c * 128) if (c in blocks and c * 128 <= i) else 0
            expect = inside / n_all
            got = o[i, 0, 0]
            if inside == 0:
                assert got == 0.0, (c, i, got)
            else:
                assert abs(got - expect) <= expect * 2 ** -8, (c, i, got, expect)


def test_gqa_equals_repeated_mha_bitwise():
    w = W.make_dense("g", 16, 2, 400, 8, 2, 128, True)
    o, l = P.run_gpu(w)
    wm = W.make_dense("m", 16, 2, 400, 8, 2, 128, True)
    wm.hkv = 8
    wm.k = np.repeat(w.k, 4, axis=2)
    wm.v = np.repeat(w.v, 4, axis=2)
    om, lm = P.run_gpu(wm)
    assert np.array_equal(o, om) and np.array_equal(l, lm)


def test_packed_equals_per_sequence_bitwise():
    lengths = [300, 1, 129, 640]
    w = W.make_varlen("v", 17, lengths, 4, 2, 64, True)
    o, l = P.run_gpu(w)
    cu = w.cu_seqlens
    for b, n in enumerate(lengths):
        s, e = int(cu[b]), int(cu[b + 1])
        wb = W.Workload("vb", 0, 1, n, 4, 2, 64, True, w.scale, w.q[s:e][None], w.k[s:e][None], w.v[s:e][None])
        ob, lb = P.run_gpu(wb)
        assert np.array_equal(o[s:e], ob) and np.array_equal(l[s:e], lb), b


def test_full_list_equals_dense():
    w = W.make_dense("fl", 18, 1, 1000, 4, 2, 128, True)
    od, ld = P.run_gpu(w)
    n_q = (1000 + 127) // 128
    w.row_ptr, w.col_idx = W.full_causal_list(n_q)
    ol, ll = P.run_gpu(w)
    assert np.array_equal(od, ol) and np.array_equal(ld, ll)  # same visiting order: same bits
    w.row_ptr, w.col_idx = W.full_causal_list(n_q, shuffle_seed=3)
    os_, ls = P.run_gpu(w)
    P.compare(os_, ls, od, ld, "shuffled list")


def random_list(seed, n_qblk, n_kblk, p=0.4, bad_ids=True, empty_row=None):
    """A block list in random order per query block: the diagonal and a random share of
    the others (some above the diagonal), plus ids outside the sequence that must be
    skipped; one row may be left empty."""
    rng = np.random.default_rng(seed)
    rows = []
    for qb in range(n_qblk):
        ids = [b for b in range(n_kblk) if b == qb or rng.random() < p]
        if bad_ids and qb % 3 == 1:
            ids += [-1, n_kblk + 2]
        rng.shuffle(ids)
        rows.append([] if qb == empty_row else ids)
    row_ptr = np.zeros(n_qblk + 1, np.int32)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    return row_ptr, np.array([c for r in rows for c in r] or [0], np.int32)[:row_ptr[-1]]


LIST_CASES = [
    # name, S, hq, hkv, d, causal (paired kernels for even groups; g = 1 and 3 use the 4-wave kernel)
    ("list_d64_causal", 700, 4, 2, 64, True),
    ("list_d64_noncausal", 700, 4, 2, 64, False),
    ("list_d128_causal", 900, 8, 2, 128, True),
    ("list_d128_noncausal_g1", 500, 3, 3, 128, False),
    ("list_d128_causal_g3", 600, 6, 2, 128, True),
    ("list_d256_causal", 650, 4, 2, 256, True),
    ("list_d256_noncausal", 400, 2, 1, 256, False),
]


@pytest.mark.parametrize("case", LIST_CASES, ids=[c[0] for c in LIST_CASES])
def test_block_list_small_full(case):
    """Random block lists (any order, ids above the diagonal, ids outside the sequence,
    an empty row, a ragged last block) against the oracle on every output."""
    name, s, hq, hkv, d, causal = case
    note(f"block list case {name}")
    w = W.make_dense(name, 25, 1, s, hq, hkv, d, causal)
    n = (s + 127) // 128
    w.row_ptr, w.col_idx = random_list(26, n, n, empty_row=2)
    o, l = P.run_gpu(w)
    assert np.all(o[256:384] == 0) and np.all(l[256:384] == -np.inf)
    import oracle
    o_ref, l_ref = oracle.run_workload(w, nthreads=P.oracle_threads())
    stats = P.compare(o, l, o_ref, l_ref, name)
    note(f"  {stats}")


def test_empty_allowed_set():
    """A query block that lists only a future block: O = 0 and LSE = -inf."""
    w = W.make_dense("e", 19, 1, 384, 2, 1, 64, True)
    w.row_ptr = np.array([0, 1, 2, 4], np.int32)
    w.col_idx = np.array([0, 2, 2, 1], np.int32)
    o, l = P.run_gpu(w)
    assert np.all(o[128:256] == 0) and np.all(l[128:256] == -np.inf)
    import oracle
    o_ref, l_ref = oracle.run_workload(w)
    P.compare(o, l, o_ref, l_ref, "empty")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_large_scores_shifted_keys(d):
    """Keys shifted by a large constant (scores of several hundred) stay finite and exact
    (each head_dim runs its own loop form)."""
    note(f"shifted keys d={d}")
    w = W.make_dense("sh", 20, 1, 512, 2, 1, d, True)
    kf = W.bf16_bits_to_f32(w.k) + np.float32(24.0)
    w.k = W.f32_to_bf16_bits(kf)
    stats = P.check_workload(w)
    note(f"  {stats}")


# ---------------------------------------------------------------- bit-packed block masks
def random_visibility(seed, n_s, n_h, n_qblk, n_kblk, p=0.5, diag=True):
    rng = np.random.default_rng(seed)
    vis = rng.random((n_s, n_h, n_qblk, n_kblk)) < p
    if diag:
        for qb in range(min(n_qblk, n_kblk)):
            vis[..., qb, qb] = True
    return vis


MASK_CASES = [
    # name, lengths (None = fixed B x S), B, S, hq, hkv, d, causal, mask sets (seq, head)
    ("per_head_causal_d128", None, 2, 700, 4, 2, 128, True, (1, 2)),
    ("per_seq_noncausal_d64", None, 3, 300, 4, 4, 64, False, (3, 1)),
    ("per_seq_head_varlen_d128", [300, 1, 700, 129], 0, 0, 8, 2, 128, True, (4, 2)),
    ("per_head_causal_d256", None, 1, 520, 4, 2, 256, True, (1, 2)),
    ("per_head_causal_d64_paired", None, 2, 700, 4, 2, 64, True, (1, 2)),
    ("per_seq_head_varlen_d64", [640, 3, 200], 0, 0, 8, 2, 64, True, (3, 2)),
    ("two_words_causal_d64", None, 1, 40 * 128 + 17, 2, 2, 64, True, (1, 2)),
    ("shared_noncausal_d128", None, 2, 400, 2, 1, 128, False, (1, 1)),
]


@pytest.mark.parametrize("case", MASK_CASES, ids=[c[0] for c in MASK_CASES])
def test_block_mask_small_full(case):
    name, lengths, b, s, hq, hkv, d, causal, (ns, nh) = case
    note(f"block mask case {name}")
    if lengths is None:
        w = W.make_dense(name, 30, b, s, hq, hkv, d, causal)
    else:
        w = W.make_varlen(name, 31, lengths, hq, hkv, d, causal)
    n_qblk = (w.seqlen + 127) // 128
    w.block_mask = W.pack_block_mask(random_visibility(32, ns, nh, n_qblk, n_qblk, p=0.45))
    stats = P.check_workload(w)
    note(f"  {stats}")


def test_block_mask_empty_rows():
    """A query block whose mask row has no visible block: O = 0 and LSE = -inf there."""
    w = W.make_dense("mask_empty", 33, 1, 384, 2, 1, 64, False)
    vis = random_visibility(34, 1, 1, 3, 3, p=0.6)
    vis[0, 0, 1, :] = False
    w.block_mask = W.pack_block_mask(vis)
    o, l = P.run_gpu(w)
    assert np.all(o[128:256] == 0) and np.all(l[128:256] == -np.inf)
    import oracle
    o_ref, l_ref = oracle.run_workload(w)
    P.compare(o, l, o_ref, l_ref, "mask_empty")


def test_block_mask_zero_q_counts_per_head():
    """Q = 0: LSE_i = ln |A(i)| with the count taken from each KV head's own mask."""
    w = W.make_dense("mask_zq", 35, 1, 1024, 4, 2, 128, True)
    w.q[:] = 0
    vis = random_visibility(36, 1, 2, 8, 8, p=0.5)
    w.block_mask = W.pack_block_mask(vis)
    _, l = P.run_gpu(w)
    for h in range(4):
        c = h // 2
        for i in range(0, 1024, 5):
            qb = i // 128
            n = sum(min(128, i + 1 - kb * 128) for kb in range(qb + 1) if vis[0, c, qb, kb])
            assert abs(l[i, h] - math.log(n)) <= 1e-5, (h, i)


def test_block_mask_of_list_matches_list():
    """The bit-packed form of the block list gives the list's result (visit order differs)."""
    w = sparse_small(s=4096, seed=37)
    ol, ll = P.run_gpu(w)
    vis = W.list_visibility(w.row_ptr, w.col_idx, 32)
    w.row_ptr, w.col_idx = None, None
    w.block_mask = W.pack_block_mask(vis[None, None])
    om, lm = P.run_gpu(w)
    P.compare(om, lm, ol, ll, "mask of list")


def test_full_block_mask_equals_dense_causal():
    w = W.make_dense("mask_full", 38, 1, 1000, 4, 2, 128, True)
    od, ld = P.run_gpu(w)
    n = 8
    w.block_mask = W.pack_block_mask(np.tril(np.ones((n, n), bool))[None, None])
    om, lm = P.run_gpu(w)
    P.compare(om, lm, od, ld, "full mask")


def test_block_mask_workload_sampled():
    """Per-KV-head masks at S = 32768 (256 query blocks, 8 words per row), sampled rows."""
    w = W.make_sparse_mask("mask_32k", 39, 32768, 32, 8, 128, n_sample=128)
    note(f"per-head mask workload S=32768: {len(w.sample_rows)} sampled rows x {w.hq} heads")
    stats = P.check_workload(w, rows=w.sample_rows)
    note(f"  {stats}")


def _chip_wide(n_units, unit_group, n_tiles):
    """Whether a block-list / block-mask launch of the paired kernel takes the chip-wide
    KV-group order: whole GQA groups dealt over the 8 XCDs and at least 8 workgroups per
    CU (the launch's own rule, restated for the test's shapes)."""
    return n_units % (8 * unit_group) == 0 and n_units * n_tiles >= 8 * 256


def test_block_list_chip_wide_order_full():
    """A block list at a size where the workgroups take the chip-wide KV-group order
    (S = 16384, 32 query heads in pairs over 8 KV heads: 16 units x 128 query blocks);
    random visiting order, ids out of range, against the oracle on every output."""
    s, hq, hkv, d = 16384, 32, 8, 64
    n = s // 128
    assert _chip_wide(hq // 2, (hq // hkv) // 2, n)
    note(f"block list, chip-wide order: S={s} hq={hq} hkv={hkv} d={d}")
    w = W.make_dense("list_chip", 40, 1, s, hq, hkv, d, True)
    w.row_ptr, w.col_idx = random_list(41, n, n, p=0.08)
    stats = P.check_workload(w)
    note(f"  {stats}")


def test_block_mask_chip_wide_order_packed_full():
    """Per-sequence, per-KV-head masks over a packed batch at a size where the workgroups
    take the chip-wide KV-group order (7 sequences x 16 units x 24 query blocks), an empty
    and a one-token sequence included, against the oracle on every output."""
    lengths = [2500, 1, 3000, 0, 700, 1900, 128]
    hq, hkv, d = 32, 8, 64
    n_qblk = (max(lengths) + 127) // 128
    assert _chip_wide(len(lengths) * hq // 2, (hq // hkv) // 2, n_qblk)
    note(f"block mask, chip-wide order: lengths={lengths} hq={hq} hkv={hkv} d={d}")
    w = W.make_varlen("mask_chip", 42, lengths, hq, hkv, d, True)
    w.block_mask = W.pack_block_mask(random_visibility(43, len(lengths), hkv, n_qblk, n_qblk, p=0.3))
    stats = P.check_workload(w)
    note(f"  {stats}")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_late_large_score_raises_running_max(d):
    """A key late in the sequence scores far above every earlier key (P would be
    2^22 or more against the running max): the kernel must raise the max and
    rescale O and l mid-row, in each head_dim's loop form.  Q is positive so
    that key 700 wins in every row that sees it."""
    note(f"late large score d={d}")
    w = W.make_dense("late", 22, 1, 1024, 4, 2, d, True)
    qf = np.abs(W.bf16_bits_to_f32(w.q))
    w.q = W.f32_to_bf16_bits(qf)
    kf = W.bf16_bits_to_f32(w.k)
    kf[0, 700] = 4.0
    w.k = W.f32_to_bf16_bits(kf)
    stats = P.check_workload(w)
    note(f"  {stats}")


def test_deterministic():
    w = W.make_dense("det", 21, 2, 700, 8, 2, 128, True)
    t = P.to_device(w)
    o1, l1 = P.run_gpu(w, tensors=t)
    o2, l2 = P.run_gpu(w, tensors=t)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
