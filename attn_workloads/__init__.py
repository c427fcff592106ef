"""Seeded synthetic workloads for fused softmax-attention forward.

This module is shared by the CPU oracle side (tests, the CPU baseline) and the
GPU side (tests, bench).  It holds no attention arithmetic: only random inputs,
sequence lengths, block lists, sampled rows and pair/FLOP bookkeeping.

Where the workloads come from
-----------------------------
The pages describe fused attention-forward kernels measured over many
scenarios ("AdaSplash-2" explainer, technical summary section 1; the
CMU question-guided-agent article, results section) and long-context
block-sparse attention at a 128K context where a proxy hands the kernel an
ordered list of KV blocks to visit ("CoSA" explainer, lay summary).  None of
their scenario sets, request shapes or model activations are available, so the
five synthetic workloads below stand in for them:

* ``tiny``      B=1, H=2, S=128, D=64, non-causal.
* ``mha``       B=4, H=16, S=2048, D=128, causal.
* ``gqa``       B=2, Hq=32, Hkv=8, S=8192, D=128, causal.
* ``varlen``    8 sequences, lengths uniform in [512, 16384], Hq=32, Hkv=8,
                D in {64, 128, 256}, causal, packed via ``cu_seqlens``.
* ``sparse``    B=1, Hq=32, Hkv=8, S=131072, D=128, causal, ordered per
                query-block list of 128x128 KV blocks (sink, diagonal,
                previous block, then top-scoring blocks up to a 10% budget).

Random streams
--------------
``numpy.random.Generator(PCG64(SeedSequence(seed)))`` children are spawned in
the fixed order [q, k, v, lengths, block_scores, sample_rows].  Q/K/V are drawn
as float32 N(0, 1) in logical C order ([B, S, H, D], or [T, H, D] when packed)
and rounded to bfloat16 with round-to-nearest-even; both the GPU path and the
oracle consume exactly those bfloat16 values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

STREAMS = ("q", "k", "v", "lengths", "block_scores", "sample_rows", "dout")
SPARSE_BLOCK = 128


# ---------------------------------------------------------------------------
# bfloat16 helpers (storage only)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def streams(seed: int):
    """The child generators of ``seed`` in the fixed order of ``STREAMS`` (child i depends only
    on the seed and i, so a stream appended to the tuple leaves the others unchanged)."""
    children = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: np.random.Generator(np.random.PCG64(c)) for name, c in zip(STREAMS, children)}


def normal_bf16(gen: np.random.Generator, shape) -> np.ndarray:
    """i.i.d. N(0,1) float32 rounded to bfloat16; returned as uint16 bits."""
    return f32_to_bf16_bits(gen.standard_normal(size=shape, dtype=np.float32))


# ---------------------------------------------------------------------------
# Workload description
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    """One synthetic attention-forward problem.

    Tensors are bfloat16 bit patterns (uint16):
      fixed length: q [B, S, Hq, D], k/v [B, S, Hkv, D]
      packed varlen: q [T, Hq, D], k/v [T, Hkv, D] with ``cu_seqlens`` [n+1]
    """

    name: str
    seed: int
    batch: int
    seqlen: int            # fixed length S, or max sequence length when packed
    hq: int
    hkv: int
    d: int
    causal: bool
    scale: float           # float32 value used by both sides
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cu_seqlens: Optional[np.ndarray] = None      # int32 [batch+1] when packed
    row_ptr: Optional[np.ndarray] = None         # int32 [n_qblk+1] block list (CSR)
    col_idx: Optional[np.ndarray] = None         # int32 [nnz], visiting order
    sample_rows: Optional[np.ndarray] = None     # int64 token positions checked one by one
    block_mask: Optional[np.ndarray] = None      # uint32 [n_seqs|1, Hkv|1, n_qblk, words] bit mask

    @property
    def packed(self) -> bool:
        return self.cu_seqlens is not None

    @property
    def lengths(self) -> np.ndarray:
        if self.packed:
            return np.diff(self.cu_seqlens).astype(np.int64)
        return np.full(self.batch, self.seqlen, dtype=np.int64)

    @property
    def tokens(self) -> int:
        return int(self.lengths.sum())

    def cu_seqlens_or_fixed(self) -> np.ndarray:
        """cu_seqlens for the packed form, or the equivalent prefix sums of a fixed batch."""
        if self.packed:
            return self.cu_seqlens
        return (np.arange(self.batch + 1, dtype=np.int64) * self.seqlen).astype(np.int32)

    def packed_views(self):
        """q, k, v reshaped to packed [T, H, D] (a view for the fixed-length [B, S, H, D] layout)."""
        if self.packed:
            return self.q, self.k, self.v
        t = self.batch * self.seqlen
        return (self.q.reshape(t, self.hq, self.d), self.k.reshape(t, self.hkv, self.d),
                self.v.reshape(t, self.hkv, self.d))


def make_dout(w: "Workload") -> np.ndarray:
    """Seeded upstream gradient dO for the backward pass: i.i.d. N(0,1) in
    bfloat16 with the shape of ``w.q`` (uint16 bits)."""
    return normal_bf16(streams(w.seed)["dout"], w.q.shape)


def default_scale(d: int) -> float:
    """1/sqrt(D) rounded to float32 (the value both sides use)."""
    return float(np.float32(1.0 / math.sqrt(d)))


# ---------------------------------------------------------------------------
# Block list for the long-context sparse workload
# ---------------------------------------------------------------------------
def sparse_budget(i: int, budget: float = 0.10) -> int:
    """Number of listed KV blocks for query block i.

    The fixed set is {0, i-1, i} clipped to [0, i]; the budget is 10% of the
    causally visible KV blocks (i+1 of them), rounded up, never below the fixed
    set and never above i+1.
    """
    fixed = len({0, max(i - 1, 0), i})
    want = math.ceil(round(budget * (i + 1), 9))
    return min(i + 1, max(fixed, want))


def build_block_list(n_qblk: int, block_scores: np.ndarray, budget: float = 0.10):
    """Ordered per-query-block KV block list (CSR: row_ptr, col_idx).

    Visiting order for query block i: the sink block 0, the diagonal block i,
    the previous block i-1, then blocks from {1..i-2} by descending seeded
    score (ties to the lower index) until the budget of ``sparse_budget`` is
    reached.  The scores stand in for a proxy's priority; they do not depend
    on Q or K.
    """
    rows = []
    for i in range(n_qblk):
        order = []
        for b in (0, i, i - 1):
            if 0 <= b <= i and b not in order:
                order.append(b)
        k_i = sparse_budget(i, budget)
        extra = k_i - len(order)
        if extra > 0:
            cand = np.arange(1, i - 1, dtype=np.int64)
            s = block_scores[i, cand]
            # descending score, ties to lower index: stable sort on -score
            pick = cand[np.argsort(-s, kind="stable")[:extra]]
            order.extend(int(x) for x in pick)
        rows.append(order)
    row_ptr = np.zeros(n_qblk + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col_idx = np.array([c for r in rows for c in r], dtype=np.int32)
    return row_ptr, col_idx


def full_causal_list(n_qblk: int, shuffle_seed: Optional[int] = None):
    """Every causally visible block (0..i) for each query block, optionally shuffled per row."""
    rng = np.random.default_rng(shuffle_seed) if shuffle_seed is not None else None
    rows = []
    for i in range(n_qblk):
        r = np.arange(i + 1, dtype=np.int32)
        if rng is not None:
            rng.shuffle(r)
        rows.append(r)
    row_ptr = np.zeros(n_qblk + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    return row_ptr, np.concatenate(rows).astype(np.int32)


def list_visibility(row_ptr: np.ndarray, col_idx: np.ndarray, n_kblk: int) -> np.ndarray:
    """bool [n_qblk, n_kblk]: True where a CSR block list names KV block kb for query block qb."""
    n_qblk = len(row_ptr) - 1
    vis = np.zeros((n_qblk, n_kblk), dtype=bool)
    for qb in range(n_qblk):
        ids = col_idx[row_ptr[qb]:row_ptr[qb + 1]]
        ids = ids[(ids >= 0) & (ids < n_kblk)]
        vis[qb, ids] = True
    return vis


def pack_block_mask(visible: np.ndarray) -> np.ndarray:
    """Bit-pack a block visibility matrix: bool [..., n_qblk, n_kblk] -> uint32
    [..., n_qblk, ceil(n_kblk/32)], KV block kb in bit kb % 32 of word kb // 32."""
    visible = np.asarray(visible, dtype=bool)
    n_k = visible.shape[-1]
    words = (n_k + 31) // 32
    padded = np.zeros(visible.shape[:-1] + (words * 32,), dtype=bool)
    padded[..., :n_k] = visible
    bits = padded.reshape(visible.shape[:-1] + (words, 32)).astype(np.uint64)
    return (bits << np.arange(32, dtype=np.uint64)).sum(axis=-1).astype(np.uint32)


def sample_positions(gen: np.random.Generator, s: int, n: int = 256) -> np.ndarray:
    """n distinct positions: {0, 127, 128, S-1} plus the rest drawn without replacement."""
    fixed = sorted({p for p in (0, 127, 128, s - 1) if 0 <= p < s})
    rest = np.setdiff1d(np.arange(s, dtype=np.int64), np.array(fixed, dtype=np.int64))
    draw = gen.choice(rest, size=max(0, min(n, s) - len(fixed)), replace=False)
    return np.sort(np.concatenate([np.array(fixed, dtype=np.int64), draw.astype(np.int64)]))


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------
def make_dense(name, seed, b, s, hq, hkv, d, causal, scale=None) -> Workload:
    g = streams(seed)
    return Workload(name=name, seed=seed, batch=b, seqlen=s, hq=hq, hkv=hkv, d=d, causal=causal,
                    scale=default_scale(d) if scale is None else float(np.float32(scale)),
                    q=normal_bf16(g["q"], (b, s, hq, d)), k=normal_bf16(g["k"], (b, s, hkv, d)),
                    v=normal_bf16(g["v"], (b, s, hkv, d)))


def varlen_lengths(seed: int, n: int = 8, lo: int = 512, hi: int = 16384) -> np.ndarray:
    return streams(seed)["lengths"].integers(lo, hi, size=n, endpoint=True).astype(np.int64)


def make_varlen(name, seed, lengths, hq, hkv, d, causal=True, scale=None) -> Workload:
    g = streams(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    t = int(cu[-1])
    return Workload(name=name, seed=seed, batch=len(lengths), seqlen=int(lengths.max()) if len(lengths) else 0,
                    hq=hq, hkv=hkv, d=d, causal=causal,
                    scale=default_scale(d) if scale is None else float(np.float32(scale)),
                    q=normal_bf16(g["q"], (t, hq, d)), k=normal_bf16(g["k"], (t, hkv, d)),
                    v=normal_bf16(g["v"], (t, hkv, d)), cu_seqlens=cu)


def make_sparse(name, seed, s, hq, hkv, d, budget=0.10, n_sample=256) -> Workload:
    g = streams(seed)
    n_qblk = (s + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    scores = g["block_scores"].random(size=(n_qblk, n_qblk))
    row_ptr, col_idx = build_block_list(n_qblk, scores, budget)
    return Workload(name=name, seed=seed, batch=1, seqlen=s, hq=hq, hkv=hkv, d=d, causal=True,
                    scale=default_scale(d),
                    q=normal_bf16(g["q"], (1, s, hq, d)), k=normal_bf16(g["k"], (1, s, hkv, d)),
                    v=normal_bf16(g["v"], (1, s, hkv, d)), row_ptr=row_ptr, col_idx=col_idx,
                    sample_rows=sample_positions(g["sample_rows"], s, n_sample))


def make_sparse_mask(name, seed, s, hq, hkv, d, budget=0.10, n_sample=256) -> Workload:
    """The block-sparse workload with a separate block set per KV head, given as
    a bit-packed mask [1, Hkv, n_qblk, words].  Each KV head's set follows the
    rule of ``build_block_list`` with its own seeded block scores."""
    g = streams(seed)
    n_qblk = (s + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    scores = g["block_scores"].random(size=(hkv, n_qblk, n_qblk))
    vis = np.zeros((1, hkv, n_qblk, n_qblk), dtype=bool)
    for c in range(hkv):
        row_ptr, col_idx = build_block_list(n_qblk, scores[c], budget)
        vis[0, c] = list_visibility(row_ptr, col_idx, n_qblk)
    return Workload(name=name, seed=seed, batch=1, seqlen=s, hq=hq, hkv=hkv, d=d, causal=True,
                    scale=default_scale(d),
                    q=normal_bf16(g["q"], (1, s, hq, d)), k=normal_bf16(g["k"], (1, s, hkv, d)),
                    v=normal_bf16(g["v"], (1, s, hkv, d)), block_mask=pack_block_mask(vis),
                    sample_rows=sample_positions(g["sample_rows"], s, n_sample))


def osk_list(n_qblk: int, proxy: np.ndarray, budget: float):
    """Ordered list for ordered skipping: query block i visits its own block
    first, then the ceil(budget * i) blocks of 0..i-1 with the highest proxy
    score, highest first (ties to the lower index)."""
    row_ptr = np.zeros(n_qblk + 1, dtype=np.int32)
    cols = []
    for i in range(n_qblk):
        k = int(math.ceil(budget * i))
        order = np.argsort(-proxy[:i], kind="stable")[:k]
        cols.append(np.concatenate([[i], order]).astype(np.int32))
        row_ptr[i + 1] = row_ptr[i] + len(cols[-1])
    return row_ptr, np.concatenate(cols) if cols else np.zeros(0, np.int32)


def make_osk(name, seed, s, hq, hkv, d, budget=0.25, mu=5.0, proxy_noise=0.5, n_sample=256) -> Workload:
    """Causal block-list workload with planted block relevance, for ordered skipping.

    Every 128-key block kb gets a relevance a_kb = 4 * Exp(1); KV head c has a
    unit direction e_c.  Keys are k_j = z_j + a_kb(j) * e_c and queries
    q_i = z_i' + mu * e_c (z i.i.d. N(0,1); z_i' is z_i with its component
    along e_c removed), so every key of block kb carries the same score boost
    scale * mu * a_kb for every query row of the head, on top of per-pair
    noise: a few blocks hold most of a row's softmax mass, and the rows of a
    query block agree on which, as in long-context attention.  A proxy scores blocks by
    a_kb plus N(0, proxy_noise) noise (an imperfect ranking); the list
    (``osk_list``) visits the diagonal block, then the top ``budget`` share of
    the earlier blocks by proxy score.  All draws come from the seed's
    streams; the values are rounded to bf16."""
    g = streams(seed)
    n_qblk = (s + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    gb = g["block_scores"]
    a = (4.0 * gb.exponential(size=n_qblk)).astype(np.float32)
    proxy = a.astype(np.float64) + proxy_noise * gb.standard_normal(n_qblk)
    e = gb.standard_normal((hkv, d)).astype(np.float32)
    e /= np.linalg.norm(e, axis=1, keepdims=True)
    group = hq // hkv
    eh = np.repeat(e, group, axis=0)                      # e of each query head's KV head
    zq = g["q"].standard_normal(size=(1, s, hq, d), dtype=np.float32)
    zq -= np.einsum("bshd,hd->bsh", zq, eh)[..., None] * eh[None, None]  # noise orthogonal to e
    zq += mu * eh[None, None]
    zk = g["k"].standard_normal(size=(1, s, hkv, d), dtype=np.float32)
    zk += np.repeat(a, SPARSE_BLOCK)[:s][None, :, None, None] * e[None, None]
    row_ptr, col_idx = osk_list(n_qblk, proxy, budget)
    return Workload(name=name, seed=seed, batch=1, seqlen=s, hq=hq, hkv=hkv, d=d, causal=True,
                    scale=default_scale(d), q=f32_to_bf16_bits(zq), k=f32_to_bf16_bits(zk),
                    v=normal_bf16(g["v"], (1, s, hkv, d)), row_ptr=row_ptr, col_idx=col_idx,
                    sample_rows=sample_positions(g["sample_rows"], s, n_sample))


CONFIG_NAMES = ("tiny", "mha", "gqa", "varlen_d64", "varlen_d128", "varlen_d256", "sparse",
                "sparse_mask", "sparse_osk")


def make(name: str) -> Workload:
    """Build one of the named workloads (seed 1..6 in the order tiny, mha, gqa, varlen, sparse,
    sparse_mask; seed 8 for sparse_osk)."""
    if name == "tiny":
        return make_dense("tiny", 1, 1, 128, 2, 2, 64, False)
    if name == "mha":
        return make_dense("mha", 2, 4, 2048, 16, 16, 128, True)
    if name == "gqa":
        return make_dense("gqa", 3, 2, 8192, 32, 8, 128, True)
    if name.startswith("varlen_d"):
        d = int(name[len("varlen_d"):])
        return make_varlen(name, 4, varlen_lengths(4), 32, 8, d, True)
    if name == "sparse":
        return make_sparse("sparse", 5, 131072, 32, 8, 128)
    if name == "sparse_mask":
        return make_sparse_mask("sparse_mask", 6, 131072, 32, 8, 128)
    if name == "sparse_osk":
        return make_osk("sparse_osk", 8, 131072, 32, 8, 128)
    raise KeyError(name)


# ---------------------------------------------------------------------------
# Pair and FLOP bookkeeping (the metric's convention)
# ---------------------------------------------------------------------------
def dense_pairs(n_q: int, n_k: int) -> int:
    """Query-key pairs of a full (unmasked) score grid."""
    return n_q * n_k


def counted_flops(w: Workload) -> float:
    """FLOPs counted by the metric: 4*D per counted (query, key) pair, times Hq.

    Dense non-causal counts the full grid, dense causal exactly half of it,
    and the block-list mode counts 128x128 pairs per listed off-diagonal block
    and half of that for the diagonal block.  Skipped blocks count nothing.
    """
    per_pair = 4.0 * w.d * w.hq
    if w.block_mask is not None:
        # per (sequence, kv head) set, counted for each of its g query heads
        m = w.block_mask
        vis = np.unpackbits(np.ascontiguousarray(m).view(np.uint8), axis=-1, bitorder="little")
        n_qblk = m.shape[2]
        vis = vis[..., :n_qblk].astype(bool)          # [S|1, H|1, n_qblk, n_kblk]
        qb = np.arange(n_qblk)[:, None]
        kb = np.arange(n_qblk)[None, :]
        if w.causal:
            w_blk = np.where(kb < qb, 1.0, np.where(kb == qb, 0.5, 0.0))
        else:
            w_blk = np.ones((n_qblk, n_qblk))
        per_set = (vis * w_blk).sum(axis=(-1, -2))     # [S|1, H|1]
        per_set = np.broadcast_to(per_set, (max(1, m.shape[0]), w.hkv))
        g = w.hq // w.hkv
        return 4.0 * w.d * g * SPARSE_BLOCK * SPARSE_BLOCK * float(per_set.sum())
    if w.row_ptr is not None:
        n_q = np.repeat(np.arange(len(w.row_ptr) - 1), np.diff(w.row_ptr))
        diag = int(np.sum(w.col_idx == n_q))
        off = int(len(w.col_idx)) - diag
        pairs = SPARSE_BLOCK * SPARSE_BLOCK * (off + 0.5 * diag)
        return per_pair * pairs
    pairs = sum(dense_pairs(int(l), int(l)) for l in w.lengths)
    if w.causal:
        pairs = 0.5 * pairs
    return per_pair * pairs


def algorithmic_bytes(w: Workload, with_lse: bool = True) -> int:
    """Bytes of Q, K, V read once plus O (and fp32 LSE) written once."""
    t = w.tokens
    b = 2 * t * w.d * (2 * w.hq + 2 * w.hkv)
    if with_lse:
        b += 4 * t * w.hq
    return b
