"""Seeded random sweep of the backward (dQ, dK, dV) against the fp64 oracle.

Each case draws its own problem: fixed batch or packed variable-length
sequences, with or without a bit-packed block mask (per sequence and/or per
KV head, or shared), head_dim 64 / 128 / 256 (round-robin with the mode, so
every pair is drawn), the KV head count and GQA group, the causal flag, the
softmax scale, the memory order of the tensors, and lengths that mix tile
edges with arbitrary values.  The GPU forward supplies O and the LSE, the
GPU backward the gradients, which are compared element by element with the
oracle's (the gradient bounds of tests/_parity.py).  The draw is host code,
checked on the CPU.
"""
import sys

import numpy as np
import pytest

import attn_workloads as W
from tests import _parity as P

MODES = ("fixed", "packed", "mask", "mask_packed")
HEAD_DIMS = (64, 128, 256)
N_CASES = 4 * len(MODES) * len(HEAD_DIMS)
EDGES = (1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257)
MAX_WORK = 4.0e9   # sum over sequences of len^2 * Hq * D (the backward oracle does ~3x the forward's work)


def _length(rng, hi=900):
    return int(rng.choice(EDGES)) if rng.random() < 0.4 else int(rng.integers(1, hi + 1))


def _work(c) -> float:
    lens = c["lengths"] if c["lengths"] is not None else [c["seqlen"]] * c["batch"]
    return float(sum(x * x for x in lens)) * c["hq"] * c["d"]


def draw(i: int) -> dict:
    rng = np.random.default_rng(9173 + 104729 * i)
    mode = MODES[i % len(MODES)]
    d = HEAD_DIMS[(i // len(MODES)) % len(HEAD_DIMS)]
    hkv = int(rng.integers(1, 4))
    hq = hkv * int(rng.choice([1, 2, 4]))
    causal = bool(rng.random() < 0.6)
    scale = None if rng.random() < 0.5 else float(np.float32(rng.uniform(0.3, 2.0) / np.sqrt(d)))
    packed = mode in ("packed", "mask_packed")
    layout = "bhsd" if (not packed and rng.random() < 0.3) else "bshd"
    if packed:
        lengths = [_length(rng) for _ in range(int(rng.integers(1, 5)))]
        if rng.random() < 0.3:
            lengths.insert(int(rng.integers(0, len(lengths) + 1)), 0)
        batch, seqlen = len(lengths), max(lengths)
    else:
        lengths, batch, seqlen = None, int(rng.integers(1, 3)), _length(rng)
    c = dict(i=i, mode=mode, d=d, hq=hq, hkv=hkv, causal=causal, scale=scale, layout=layout,
             batch=batch, seqlen=seqlen, lengths=lengths, seed=int(rng.integers(1 << 30)))
    while _work(c) > MAX_WORK:
        if c["lengths"] is not None:
            c["lengths"] = [x // 2 for x in c["lengths"]]
            c["seqlen"] = max(c["lengths"])
        else:
            c["seqlen"] = max(1, c["seqlen"] // 2)
    if mode.startswith("mask"):
        n_blk = (c["seqlen"] + 127) // 128
        ns = c["batch"] if rng.random() < 0.5 else 1
        nh = hkv if rng.random() < 0.6 else 1
        c["mask"] = W.pack_block_mask(rng.random((ns, nh, n_blk, n_blk)) < rng.uniform(0.3, 0.9))
    return c


def build(c) -> W.Workload:
    name = f"rbwd{c['i']}_{c['mode']}_d{c['d']}"
    if c["lengths"] is not None:
        w = W.make_varlen(name, c["seed"], c["lengths"], c["hq"], c["hkv"], c["d"], c["causal"], c["scale"])
    else:
        w = W.make_dense(name, c["seed"], c["batch"], c["seqlen"], c["hq"], c["hkv"], c["d"], c["causal"],
                         c["scale"])
    if "mask" in c:
        w.block_mask = c["mask"]
    return w


def _label(c):
    lens = c["lengths"] if c["lengths"] is not None else f"{c['batch']}x{c['seqlen']}"
    return (f"case {c['i']}: {c['mode']} d={c['d']} hq={c['hq']} hkv={c['hkv']} causal={c['causal']} "
            f"scale={c['scale']} layout={c['layout']} lengths={lens}")


def test_draw_covers_every_mode_and_head_dim():
    cases = [draw(i) for i in range(N_CASES)]
    assert {(c["mode"], c["d"]) for c in cases} == {(m, d) for m in MODES for d in HEAD_DIMS}
    assert [_label(c) for c in cases] == [_label(draw(i)) for i in range(N_CASES)]
    assert all(_work(c) <= MAX_WORK for c in cases)
    assert {c["causal"] for c in cases} == {True, False}
    assert any(c["hq"] > c["hkv"] for c in cases)
    assert any(c["layout"] == "bhsd" for c in cases) and any(c["scale"] is not None for c in cases)
    lens = [x for c in cases for x in (c["lengths"] or [c["seqlen"]])]
    assert 0 in lens and any(x % 64 for x in lens)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_bwd_case(i):
    c = draw(i)
    print(f"[gpu] random backward sweep {_label(c)}", file=sys.stderr, flush=True)
    w = build(c)
    do = W.make_dout(w)
    got = P.run_gpu_bwd(w, do, c["layout"])
    ref = P.oracle_bwd(w, do)
    stats = P.compare_grads(got, ref, w.name)
    print(f"[gpu]   {stats}", file=sys.stderr, flush=True)
