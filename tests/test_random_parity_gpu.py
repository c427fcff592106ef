"""Seeded random sweep of the forward against the fp64 oracle on every output.

Each case draws its own problem from a seeded generator: the mode (fixed
batch, packed variable-length, block list, bit-packed block mask), head_dim,
the number of KV heads and the GQA group, causal or not, the softmax scale,
the memory order of Q, K and V, and sequence lengths that mix tile edges
(1, 63, 64, 65, 127, 128, 129, ...) with arbitrary values up to about 2100.
Mode and head_dim are assigned round-robin so that every pair is drawn;
the rest is random.  The draw itself is host code and is checked on the CPU
(``test_draw_covers_every_mode_and_head_dim``); the comparison needs the GPU.
"""
import sys

import numpy as np
import pytest

import attn_workloads as W
from tests import _parity as P

MODES = ("fixed", "packed", "list", "mask")
HEAD_DIMS = (64, 128, 256)
N_CASES = 4 * len(MODES) * len(HEAD_DIMS)
EDGES = (1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 383, 384, 385)
MAX_WORK = 2.0e10  # sum over sequences of len^2 * Hq * D, to keep the oracle within seconds


def _length(rng, hi=2100):
    return int(rng.choice(EDGES)) if rng.random() < 0.4 else int(rng.integers(1, hi + 1))


def _random_list(rng, n_qblk):
    """Random order per query block; random share of blocks, ids above the diagonal
    and outside the sequence included; sometimes an empty row."""
    rows = []
    p = rng.uniform(0.2, 0.9)
    for qb in range(n_qblk):
        ids = [b for b in range(n_qblk) if rng.random() < p]
        if rng.random() < 0.2:
            ids += [int(rng.integers(n_qblk, n_qblk + 4)), -1]
        if rng.random() < 0.1:
            ids = []
        rng.shuffle(ids)
        rows.append(ids)
    row_ptr = np.zeros(n_qblk + 1, np.int32)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col = np.array([c for r in rows for c in r] or [0], np.int32)[:row_ptr[-1]]
    return row_ptr, col


def draw(i: int) -> dict:
    """The i-th case: a dict of problem parameters (no tensors)."""
    rng = np.random.default_rng(4242 + 7919 * i)
    mode = MODES[i % len(MODES)]
    d = HEAD_DIMS[(i // len(MODES)) % len(HEAD_DIMS)]
    hkv = int(rng.integers(1, 5))
    g = int(rng.choice([1, 2, 2, 3, 4]))
    hq = hkv * g
    causal = bool(rng.random() < 0.6)
    scale = None if rng.random() < 0.5 else float(np.float32(rng.uniform(0.3, 2.0) / np.sqrt(d)))
    layout = "bhsd" if (mode in ("fixed", "list", "mask") and rng.random() < 0.3) else "bshd"
    packed_mask = mode == "mask" and rng.random() < 0.5
    if mode == "packed" or packed_mask:
        lengths = [_length(rng) for _ in range(int(rng.integers(1, 6)))]
        if rng.random() < 0.3:
            lengths.insert(int(rng.integers(0, len(lengths) + 1)), 0)
        batch, seqlen = len(lengths), max(lengths)
        layout = "bshd"
    else:
        batch = 1 if mode == "list" else int(rng.integers(1, 4))
        seqlen = _length(rng)
        lengths = None
    case = dict(i=i, mode=mode, d=d, hq=hq, hkv=hkv, causal=causal, scale=scale, layout=layout,
                batch=batch, seqlen=seqlen, lengths=lengths, seed=int(rng.integers(1 << 30)))
    # shrink until the oracle's work fits
    while _work(case) > MAX_WORK:
        if case["lengths"] is not None:
            case["lengths"] = [x // 2 for x in case["lengths"]]
            case["seqlen"] = max(case["lengths"])
        else:
            case["seqlen"] = max(1, case["seqlen"] // 2)
    n_qblk = (case["seqlen"] + 127) // 128
    if mode == "list":
        case["list"] = _random_list(rng, n_qblk)
    elif mode == "mask":
        ns = case["batch"] if rng.random() < 0.5 else 1
        nh = hkv if rng.random() < 0.6 else 1
        vis = rng.random((ns, nh, n_qblk, n_qblk)) < rng.uniform(0.2, 0.9)
        case["mask"] = W.pack_block_mask(vis)
    return case


def _work(c) -> float:
    lens = c["lengths"] if c["lengths"] is not None else [c["seqlen"]] * c["batch"]
    return float(sum(x * x for x in lens)) * c["hq"] * c["d"]


def build(c) -> W.Workload:
    name = f"rand{c['i']}_{c['mode']}_d{c['d']}"
    if c["lengths"] is not None:
        w = W.make_varlen(name, c["seed"], c["lengths"], c["hq"], c["hkv"], c["d"], c["causal"], c["scale"])
    else:
        w = W.make_dense(name, c["seed"], c["batch"], c["seqlen"], c["hq"], c["hkv"], c["d"], c["causal"],
                         c["scale"])
    if "list" in c:
        w.row_ptr, w.col_idx = c["list"]
    if "mask" in c:
        w.block_mask = c["mask"]
    return w


def _label(c):
    lens = c["lengths"] if c["lengths"] is not None else f"{c['batch']}x{c['seqlen']}"
    return (f"case {c['i']}: {c['mode']} d={c['d']} hq={c['hq']} hkv={c['hkv']} causal={c['causal']} "
            f"scale={c['scale']} layout={c['layout']} lengths={lens}")


def test_draw_covers_every_mode_and_head_dim():
    """Host check of the sweep itself: every (mode, head_dim) pair is drawn, the draw is
    reproducible, the oracle's work stays bounded, and the structure is varied
    (GQA groups above 1, both causal settings, tile-edge lengths, an empty sequence)."""
    cases = [draw(i) for i in range(N_CASES)]
    assert {(c["mode"], c["d"]) for c in cases} == {(m, d) for m in MODES for d in HEAD_DIMS}
    assert [_label(c) for c in cases] == [_label(draw(i)) for i in range(N_CASES)]
    assert all(_work(c) <= MAX_WORK for c in cases)
    assert {c["causal"] for c in cases} == {True, False}
    assert any(c["hq"] > c["hkv"] for c in cases) and any(c["hq"] == c["hkv"] for c in cases)
    assert any(c["layout"] == "bhsd" for c in cases) and any(c["scale"] is not None for c in cases)
    lens = [x for c in cases for x in (c["lengths"] or [c["seqlen"]])]
    assert 0 in lens and any(x % 128 not in (0,) for x in lens) and any(x > 512 for x in lens)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_full(i):
    c = draw(i)
    print(f"[gpu] random sweep {_label(c)}", file=sys.stderr, flush=True)
    w = build(c)
    stats = P.check_workload(w, layout=c["layout"])
    print(f"[gpu]   {stats}", file=sys.stderr, flush=True)
