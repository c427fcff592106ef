"""Seeded workload generators, block lists and FLOP bookkeeping (CPU only)."""
import hashlib
import math
import os

import numpy as np

import attn_workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_generator_is_reproducible():
    """SHA-256 of the generated bfloat16 bytes is fixed per seed."""
    w = W.make("tiny")
    assert w.q.shape == (1, 128, 2, 64) and w.q.dtype == np.uint16
    assert sha(w.q) == "4751caf8720ba1853a5757218ee3a6e68b90b74703ddb8072c18929966adb58d"
    assert sha(w.k) == "c639193d819c7931c728012fd6b3ac7ada00c3654d59e5dbd283ec35d5baa5f1"
    assert sha(w.v) == "762ebcec81e9cfc2009b745f2f8d2f437e3f184c6312a18c94dc66f263425808"
    w = W.make("mha")
    assert w.q.shape == (4, 2048, 16, 128)
    assert sha(w.q) == "c6a28d38ebc162c0b7d5f86841219562a77b60523b20afce7289e5901ffbef54"
    assert sha(w.k) == "2f4fa53f8ead5d5c08074f245f8f2bf92ab3847e1a93a7bef0ae07172893633e"
    assert sha(w.v) == "63fa5d60182e02001ef3f7bd94073134e488b4e1112ed1f4cebba0a66ca587eb"


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e-3], dtype=np.float32)
    b = W.f32_to_bf16_bits(x)
    back = W.bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2 ** -6 and back[3] == 1.0
    assert back[4] == -2.5
    assert abs(back[5] - 3.0e-3) <= 2 ** -8 * 3.0e-3  # half an ulp: 2^-8 relative
    # round trip of bf16 values is exact
    assert np.array_equal(W.f32_to_bf16_bits(back), b)


def test_inputs_are_standard_normal():
    w = W.make("mha")
    x = W.bf16_bits_to_f32(w.q[0, :512]).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01


def test_varlen_lengths():
    L = W.varlen_lengths(4)
    assert len(L) == 8 and L.min() >= 512 and L.max() <= 16384
    w = W.make_varlen("v", 4, [3, 5, 1], 4, 2, 64)
    assert list(w.cu_seqlens) == [0, 3, 8, 9] and w.q.shape == (9, 4, 64) and w.k.shape == (9, 2, 64)
    # D=64 and D=256 variants reuse the same lengths
    assert list(W.varlen_lengths(4)) == list(L)


def test_block_list_properties():
    """Sink, diagonal and previous block present; no duplicates; causal ids; budget; order."""
    nq = 1024
    g = W.streams(5)
    scores = g["block_scores"].random(size=(nq, nq))
    rp, ci = W.build_block_list(nq, scores)
    assert rp[0] == 0 and np.all(np.diff(rp) >= 1)
    for i in range(nq):
        row = [int(c) for c in ci[rp[i]:rp[i + 1]]]
        assert len(row) == len(set(row))
        assert all(0 <= c <= i for c in row)
        assert row[0] == 0 and i in row and (i == 0 or i - 1 in row)
        expect = min(i + 1, max(len({0, max(i - 1, 0), i}), math.ceil(0.1 * (i + 1) - 1e-9)))
        assert len(row) == expect
        fixed = [c for c in (0, i, i - 1) if c >= 0]
        fixed = list(dict.fromkeys(fixed))
        assert row[:len(fixed)] == fixed
        extra = row[len(fixed):]
        s = [scores[i, c] for c in extra]
        assert s == sorted(s, reverse=True)
        if extra:  # every unselected candidate scores no higher than the last selected one
            rest = [c for c in range(1, i - 1) if c not in row]
            assert all(scores[i, c] <= s[-1] for c in rest)
    # totals for the 128K, 10% budget workload
    assert int(rp[-1]) == 52969 and int(np.diff(rp).max()) == 103


def test_sample_positions():
    g = W.streams(5)
    r = W.sample_positions(g["sample_rows"], 131072, 256)
    assert len(r) == 256 and len(set(r.tolist())) == 256
    assert {0, 127, 128, 131071} <= set(r.tolist())
    assert np.all(np.diff(r) > 0)


def test_pair_counts_golden():
    """Dense pair counts match the numbers printed on the AdaSplash-2 explainer page."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "pair_counts.txt")) if l.strip() and not l.startswith("#")]
    for n, pairs in rows:
        assert W.dense_pairs(int(n), int(n)) == int(pairs)


def test_counted_flops():
    w = W.make("tiny")
    assert W.counted_flops(w) == 4 * 64 * 2 * 128 * 128  # non-causal: full grid
    w = W.make_dense("c", 9, 4, 2048, 16, 16, 8, True)
    assert W.counted_flops(w) == 0.5 * 4 * 8 * 16 * 4 * 2048 * 2048
    # sparse: 128x128 pairs per listed block, half for the diagonal block
    rp = np.array([0, 1, 3], np.int32)
    ci = np.array([0, 1, 0], np.int32)
    w = W.Workload("s", 0, 1, 256, 2, 1, 8, True, 0.1, None, None, None, row_ptr=rp, col_idx=ci)
    assert W.counted_flops(w) == 4 * 8 * 2 * 128 * 128 * (1 + 0.5 + 0.5)


def test_bench_workload_numbers():
    """FLOPs and bytes of the dense causal MHA workload (B=4, H=16, S=2048, D=128)."""
    w = W.make("mha")
    assert W.counted_flops(w) == 68719476736.0
    assert W.algorithmic_bytes(w) == 2 * 4 * 2048 * 128 * (2 * 16 + 2 * 16) + 4 * 4 * 2048 * 16


def test_block_mask_generator():
    """Per-KV-head masks: each head's set follows the list rule with its own scores."""
    w = W.make_sparse_mask("m", 6, 4096, 4, 2, 64)
    assert w.block_mask.shape == (1, 2, 32, 1) and w.block_mask.dtype == np.uint32
    assert sha(w.block_mask) == "8c22e869bce01c3ffe8f3584c97f63e1fdb4757a25c80cad29bba3da46d283f1"
    vis = np.unpackbits(w.block_mask.view(np.uint8), axis=-1, bitorder="little")[..., :32].astype(bool)
    for c in range(2):
        for i in range(32):
            row = vis[0, c, i]
            assert row[0] and row[i] and (i == 0 or row[i - 1])
            assert int(row.sum()) == W.sparse_budget(i)
            assert not row[i + 1:].any()
    assert (vis[0, 0] != vis[0, 1]).any()
    # counted flops: 128x128 pairs per visible off-diagonal block, half for the diagonal, g heads each
    per_head = sum(W.sparse_budget(i) - 0.5 for i in range(32))
    assert W.counted_flops(w) == 4 * 64 * 2 * 128 * 128 * 2 * per_head


def test_osk_generator():
    """Planted-relevance workload: deterministic bytes; each query block's list is its
    own block, then the top ceil(budget * i) earlier blocks by proxy score, highest
    first; keys of a block share one boost along the head's direction, which the
    query rows all see alike (query noise is orthogonal to it)."""
    w = W.make_osk("o", 8, 4096, 4, 2, 64)
    assert sha(w.q) == "605d8d9b73d51d542557d74b5439b3e94216953ee6e9f99d14c0278ae2481bde"
    assert sha(w.k) == "11437e094208718a741a9527f40b86be287a58ca5cb07b5d3d18d2f294392b9f"
    assert sha(w.col_idx) == "8eb6b0fbf3d64e5b8caa7ed17d0a2639ed00b6312ed6c15de4a2b74eef9e28a3"
    g = W.streams(8)["block_scores"]
    a = 4.0 * g.exponential(size=32)
    proxy = a + 0.5 * g.standard_normal(32)
    e = g.standard_normal((2, 64))
    e /= np.linalg.norm(e, axis=1, keepdims=True)
    for i in range(32):
        ents = w.col_idx[w.row_ptr[i]:w.row_ptr[i + 1]]
        assert ents[0] == i and len(ents) == 1 + int(np.ceil(0.25 * i))
        assert np.all(ents[1:] < i) and len(set(ents)) == len(ents)
        assert np.all(np.diff(proxy[ents[1:]]) <= 0)
    q = W.bf16_bits_to_f32(w.q).reshape(4096, 4, 64).astype(np.float64)
    k = W.bf16_bits_to_f32(w.k).reshape(4096, 2, 64).astype(np.float64)
    # every query of head h has component ~mu along e of its KV head (bf16 rounding aside)
    for h in range(4):
        comp = q[:, h] @ e[h // 2]
        assert np.abs(comp - 5.0).max() < 0.1
    # a key's component along e is its block's relevance plus N(0,1) noise
    kcomp = k[:, 0] @ e[0]
    blk_mean = kcomp.reshape(32, 128).mean(1)
    assert np.corrcoef(blk_mean, a)[0, 1] > 0.99
