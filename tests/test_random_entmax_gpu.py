"""Seeded random sweep of alpha-entmax attention against the fp64 oracle.

Each case draws alpha (1.5 and 2, which have kernels of their own, or a
value uniform in [1.05, 3]), head_dim 64, 128 or 256, the KV head count and GQA
group, the causal flag, the softmax scale, the memory order and a length
that mixes tile edges with arbitrary values; the checks are those of
tests/test_entmax_parity_gpu.py (O at the forward's tolerances, the
threshold's normalisation and, for alpha <= 2, its value, the histogram
bound, and a block mask that holds every block with a non-zero weight).
The draw is host code, checked on the CPU.
"""
import sys

import numpy as np
import pytest

import attn_workloads as W

HEAD_DIMS = (64, 128, 256)
ALPHA_KINDS = ("1.5", "2", "below 2", "above 2")
N_CASES = 3 * len(HEAD_DIMS) * len(ALPHA_KINDS)
EDGES = (1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 383, 384, 385)


def draw(i: int) -> dict:
    rng = np.random.default_rng(5381 + 65537 * i)
    kind = ALPHA_KINDS[i % len(ALPHA_KINDS)]
    d = HEAD_DIMS[(i // len(ALPHA_KINDS)) % len(HEAD_DIMS)]
    alpha = {"1.5": 1.5, "2": 2.0, "below 2": float(rng.uniform(1.05, 2.0)),
             "above 2": float(rng.uniform(2.0, 3.0))}[kind]
    alpha = float(np.float32(alpha))
    hkv = int(rng.integers(1, 4))
    hq = hkv * int(rng.choice([1, 2, 4]))
    s = int(rng.choice(EDGES)) if rng.random() < 0.4 else int(rng.integers(1, 900))
    return dict(i=i, alpha=alpha, d=d, hq=hq, hkv=hkv, batch=int(rng.integers(1, 3)), seqlen=s,
                causal=bool(rng.random() < 0.7),
                scale=None if rng.random() < 0.5 else float(np.float32(rng.uniform(0.5, 2.0) / np.sqrt(d))),
                layout="bhsd" if rng.random() < 0.3 else "bshd", seed=int(rng.integers(1 << 30)))


def _label(c):
    return (f"case {c['i']}: alpha={c['alpha']:.4f} d={c['d']} hq={c['hq']} hkv={c['hkv']} "
            f"{c['batch']}x{c['seqlen']} causal={c['causal']} scale={c['scale']} layout={c['layout']}")


def test_draw_covers_alpha_kinds_and_head_dims():
    cases = [draw(i) for i in range(N_CASES)]
    alphas = [c["alpha"] for c in cases]
    assert 1.5 in alphas and 2.0 in alphas
    assert any(a < 1.5 for a in alphas) and any(1.5 < a < 2 for a in alphas) and any(a > 2 for a in alphas)
    assert all(1.05 <= a <= 3.0 for a in alphas)
    assert {c["d"] for c in cases} == set(HEAD_DIMS)
    assert {c["causal"] for c in cases} == {True, False}
    assert [_label(c) for c in cases] == [_label(draw(i)) for i in range(N_CASES)]


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_entmax_case(i):
    from tests.test_entmax_parity_gpu import check

    c = draw(i)
    print(f"[gpu] random entmax sweep {_label(c)}", file=sys.stderr, flush=True)
    w = W.make_dense(f"rent{i}", c["seed"], c["batch"], c["seqlen"], c["hq"], c["hkv"], c["d"], c["causal"],
                     c["scale"])
    check(w, c["alpha"], 32 if c["alpha"] > 2 else 16, c["layout"])
