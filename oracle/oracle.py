"""Python face of the fp64 CPU oracle (``oracle_attn.c``, ``oracle_bwd.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path never imports this
module, and this module never imports the product package.

``attn_fwd`` computes exact softmax attention forward in float64 from the
definition (see the header of ``oracle_attn.c`` for the formula and the
passages of the pages it follows); ``attn_bwd`` its exact gradients (header
of ``oracle_bwd.c``); ``attn_fwd_osk`` ordered skipping along a block list
with the stopping rule stated in the header of ``oracle_osk.c``;
``entmax_fwd`` alpha-entmax attention (header of ``oracle_entmax.c``).  Every function's parity status is "pinned":
``tests/test_oracle_pins.py``, ``test_oracle_mask_pins.py`` and
``test_oracle_bwd_pins.py`` tie them to brute force, finite differences,
closed forms and invariants that do not go through this code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "oracle_attn.c"), os.path.join(HERE, "oracle_bwd.c"),
        os.path.join(HERE, "oracle_osk.c"), os.path.join(HERE, "oracle_entmax.c")]
LIB = os.path.join(HERE, "liboracle_attn.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, -O2, pthreads)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-Wall", "-Wextra", "-o", tmp, *SRCS, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=True)
        lib = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        lib.oracle_attn_fwd.restype = ctypes.c_int
        lib.oracle_attn_fwd.argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_double, P, P,
                                        ctypes.c_int, ctypes.c_int, P, ctypes.c_int64, P, P, P,
                                        ctypes.c_int]
        lib.oracle_attn_fwd_mask.restype = ctypes.c_int
        lib.oracle_attn_fwd_mask.argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_double, P,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, P, ctypes.c_int64, P, P,
                                             P, ctypes.c_int]
        lib.oracle_attn_bwd.restype = ctypes.c_int
        lib.oracle_attn_bwd.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_double, P,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                        P, P, P, ctypes.c_int]
        lib.oracle_attn_fwd_osk.restype = ctypes.c_int
        lib.oracle_attn_fwd_osk.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_double, P, P, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_double, ctypes.c_int, P, ctypes.c_int, P, P, P, P,
                                            ctypes.c_int]
        lib.oracle_entmax_fwd.restype = ctypes.c_int
        lib.oracle_entmax_fwd.argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_int, P, P, P,
                                          P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.oracle_default_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


MAX_THREADS = 16   # a GPU machine grants one GPU's jobs a share of 16 host CPUs, whatever it reports online


def default_threads() -> int:
    """Threads the oracle uses when asked for 0: the CPUs this process may run on
    (its affinity mask), at most MAX_THREADS."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = int(_load().oracle_default_threads())
    return max(1, min(MAX_THREADS, n))


def _threads(n: int) -> int:
    return int(n) if n and n > 0 else default_threads()


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def attn_fwd(q, k, v, cu_seqlens, causal: bool, scale: float, row_ptr=None, col_idx=None,
             block: int = 128, rows=None, nthreads: int = 0, with_psum: bool = False,
             block_mask=None):
    """Exact attention forward.

    q:  float64 [T, Hq, D] (all tokens) or [len(rows), Hq, D] when ``rows`` is given
    k, v: float64 [T, Hkv, D];  cu_seqlens: int [n+1]
    row_ptr/col_idx: optional block list (single sequence only), ``block`` rows per block
    block_mask: optional uint32 [n_seqs or 1, Hkv or 1, n_qblk, words] bit-packed
        block mask (bit kb%32 of word kb//32: KV block kb visible); a size-1
        leading dimension is shared by every sequence / kv head
    rows: optional packed token ids to compute
    Returns (O [n_q, Hq, D], LSE [n_q, Hq]) or (O, LSE, sum_j P) with ``with_psum``.
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    n_seqs = len(cu) - 1
    t = int(cu[-1])
    hq, d = q.shape[1], q.shape[2]
    hkv = k.shape[1]
    if k.shape != (t, hkv, d) or v.shape != (t, hkv, d):
        raise ValueError(f"k/v shape {k.shape}/{v.shape} != {(t, hkv, d)}")
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n_q = t if rows_a is None else len(rows_a)
    if q.shape[0] != n_q:
        raise ValueError(f"q has {q.shape[0]} rows, expected {n_q}")
    rp = None if row_ptr is None else np.ascontiguousarray(row_ptr, dtype=np.int32)
    ci = None if col_idx is None else np.ascontiguousarray(col_idx, dtype=np.int32)
    if rp is not None and ci is not None and len(ci) == 0:
        ci = np.zeros(1, dtype=np.int32)  # keep a valid pointer for an empty list
    out = np.zeros((n_q, hq, d), dtype=np.float64)
    lse = np.zeros((n_q, hq), dtype=np.float64)
    psum = np.zeros((n_q, hq), dtype=np.float64) if with_psum else None
    if block_mask is not None:
        if rp is not None:
            raise ValueError("a block list and a block mask together")
        m, ss, sh, words = _mask_strides(block_mask, n_seqs, hkv)
        n_qblk = m.shape[2]
        rc = _load().oracle_attn_fwd_mask(
            _ptr(q), _ptr(k), _ptr(v), _ptr(cu), n_seqs, hq, hkv, d, int(bool(causal)),
            float(scale), _ptr(m), ss, sh, words, n_qblk, int(block), _ptr(rows_a),
            0 if rows_a is None else len(rows_a), _ptr(out), _ptr(lse), _ptr(psum), _threads(nthreads))
    else:
        rc = _load().oracle_attn_fwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(cu), n_seqs, hq, hkv, d, int(bool(causal)),
            float(scale), _ptr(rp), _ptr(ci), 0 if rp is None else len(rp) - 1, int(block),
            _ptr(rows_a), 0 if rows_a is None else len(rows_a), _ptr(out), _ptr(lse), _ptr(psum),
            _threads(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_fwd failed with code {rc}")
    if with_psum:
        return out, lse, psum
    return out, lse


def _mask_strides(block_mask, n_seqs, hkv):
    m = np.ascontiguousarray(block_mask, dtype=np.uint32)
    if m.ndim != 4 or m.shape[0] not in (1, n_seqs) or m.shape[1] not in (1, hkv):
        raise ValueError(f"block_mask shape {m.shape}")
    n_qblk, words = m.shape[2], m.shape[3]
    ss = m.shape[1] * n_qblk * words if m.shape[0] > 1 else 0
    sh = n_qblk * words if m.shape[1] > 1 else 0
    return m, ss, sh, words


def attn_bwd(q, k, v, dout, cu_seqlens, causal: bool, scale: float, block_mask=None,
             block: int = 128, nthreads: int = 0):
    """Exact gradients of sum(O * dout) with respect to q, k and v.

    q, dout: float64 [T, Hq, D];  k, v: float64 [T, Hkv, D];  cu_seqlens: int [n+1]
    block_mask: optional uint32 [n_seqs or 1, Hkv or 1, n_qblk, words] (as in attn_fwd)
    Returns (dq [T, Hq, D], dk [T, Hkv, D], dv [T, Hkv, D]).
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    do = np.ascontiguousarray(dout, dtype=np.float64)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    n_seqs = len(cu) - 1
    t = int(cu[-1])
    hq, d = q.shape[1], q.shape[2]
    hkv = k.shape[1]
    if q.shape != (t, hq, d) or do.shape != q.shape:
        raise ValueError(f"q/dout shape {q.shape}/{do.shape} != {(t, hq, d)}")
    if k.shape != (t, hkv, d) or v.shape != (t, hkv, d):
        raise ValueError(f"k/v shape {k.shape}/{v.shape} != {(t, hkv, d)}")
    m, ss, sh, words = (None, 0, 0, 0) if block_mask is None else _mask_strides(block_mask, n_seqs, hkv)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rc = _load().oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(cu), n_seqs, hq, hkv, d,
                                 int(bool(causal)), float(scale), _ptr(m), ss, sh, words, int(block),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _threads(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_bwd failed with code {rc}")
    return dq, dk, dv


def attn_fwd_osk(q, k, v, causal: bool, scale: float, row_ptr, col_idx, tau: float, min_visit: int,
                 qblocks=None, block: int = 128, nthreads: int = 0):
    """Ordered skipping along a block list (rule in the header of ``oracle_osk.c``).

    q: float64 [T, Hq, D]; k, v: float64 [T, Hkv, D] (one sequence)
    row_ptr, col_idx: the ordered block list; tau, min_visit: the stopping rule
    qblocks: query blocks to compute (None: all)
    Returns (O [rows, Hq, D], LSE [rows, Hq], visited int32 [Hq, n_sel],
    ratio [Hq, nnz]) where rows are those of the selected blocks in order and
    ratio holds the test value max_i (n - e) d_i / L_i after each visited entry
    e of an n-entry list (NaN for entries after the stop).
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    t, hq, d = q.shape
    hkv = k.shape[1]
    rp = np.ascontiguousarray(row_ptr, dtype=np.int32)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    if len(ci) == 0:
        ci = np.zeros(1, dtype=np.int32)
    n_qblk = len(rp) - 1
    sel = np.arange(n_qblk, dtype=np.int32) if qblocks is None else np.ascontiguousarray(qblocks, dtype=np.int32)
    rows = sum(min(block, t - int(b) * block) for b in sel)
    out = np.zeros((rows, hq, d))
    lse = np.zeros((rows, hq))
    visited = np.zeros((hq, len(sel)), dtype=np.int32)
    ratio = np.full((hq, max(1, int(rp[-1]))), np.nan)
    rc = _load().oracle_attn_fwd_osk(_ptr(q), _ptr(k), _ptr(v), t, hq, hkv, d, int(bool(causal)), float(scale),
                                     _ptr(rp), _ptr(ci), n_qblk, int(block), float(tau), int(min_visit),
                                     _ptr(sel), len(sel), _ptr(out), _ptr(lse), _ptr(visited), _ptr(ratio),
                                     _threads(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_fwd_osk failed with code {rc}")
    return out, lse, visited, ratio


def entmax_fwd(q, k, v, cu_seqlens, causal: bool, scale: float, alpha: float, bins: int = 32,
               with_mask: bool = False, block: int = 128, nthreads: int = 0):
    """Exact alpha-entmax attention forward (header of ``oracle_entmax.c``).

    q: float64 [T, Hq, D]; k, v: float64 [T, Hkv, D]; cu_seqlens: int [n+1]
    Returns (O [T, Hq, D], tau [T, Hq], tau_hist [T, Hq]) and, with
    ``with_mask``, the block mask uint32 [n, Hq, n_qblk, words] (n_qblk from
    the longest sequence).
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    n_seqs = len(cu) - 1
    t, hq, d = q.shape
    hkv = k.shape[1]
    out = np.zeros((t, hq, d))
    tau = np.zeros((t, hq))
    tau_h = np.zeros((t, hq))
    mask = None
    n_qblk = words = 1
    if with_mask:
        lmax = int(np.diff(cu).max()) if n_seqs else 0
        n_qblk = max(1, -(-lmax // block))
        words = max(1, -(-n_qblk // 32))
        mask = np.zeros((n_seqs, hq, n_qblk, words), dtype=np.uint32)
    rc = _load().oracle_entmax_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu), n_seqs, hq, hkv, d, int(bool(causal)),
                                   float(scale), float(alpha), int(bins), _ptr(out), _ptr(tau), _ptr(tau_h),
                                   _ptr(mask), int(block), n_qblk, words, _threads(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_entmax_fwd failed with code {rc}")
    if with_mask:
        return out, tau, tau_h, mask
    return out, tau, tau_h


def run_workload(w, rows=None, nthreads: int = 0, with_psum: bool = False):
    """Oracle on an ``attn_workloads.Workload`` (bf16 inputs widened exactly to float64).

    Returns outputs in packed order: O [n_q, Hq, D], LSE [n_q, Hq] where n_q is
    every token or ``len(rows)`` (token ids in packed order).
    """
    from attn_workloads import bf16_bits_to_f32  # input module only (no attention arithmetic)

    q, k, v = w.packed_views()
    kf = bf16_bits_to_f32(k).astype(np.float64)
    vf = bf16_bits_to_f32(v).astype(np.float64)
    if rows is None:
        qf = bf16_bits_to_f32(q).astype(np.float64)
    else:
        qf = bf16_bits_to_f32(q[np.asarray(rows, dtype=np.int64)]).astype(np.float64)
    return attn_fwd(qf, kf, vf, w.cu_seqlens_or_fixed(), w.causal, w.scale, w.row_ptr, w.col_idx,
                    128, rows, nthreads, with_psum, getattr(w, "block_mask", None))
