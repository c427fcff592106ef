"""Helpers shared by the GPU parity tests and the smoke check.

Runs a workload through the HIP library (via the Python binding, which calls
the C ABI) and compares it with the fp64 oracle on the same seeded inputs.
"""
from __future__ import annotations

import numpy as np

import attn_workloads as W

# Tolerances for bf16 inputs/outputs with fp32 accumulation.
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3
O_REL_RMS = 1e-2   # ||O - O_ref||_2 / ||O_ref||_2, catches errors the loose max-abs bound can hide


def check_inputs(w: W.Workload) -> None:
    """Refuse a workload whose Q, K or V holds a non-finite value: every parity bound
    assumes finite inputs (an infinite score would make both sides' NaN agree or not
    by accident)."""
    for name, a in (("q", w.q), ("k", w.k), ("v", w.v)):
        x = W.bf16_bits_to_f32(a)
        if not np.all(np.isfinite(x)):
            raise ValueError(f"{w.name}: non-finite values in {name} ({int(np.sum(~np.isfinite(x)))} elements)")


def to_device(w: W.Workload, layout: str = "bshd"):
    """Device tensors for a workload: q, k, v (bf16), cu_seqlens, and the keyword
    arguments that carry its block sparsity ({} dense, block_list or block_mask).
    Non-finite inputs are refused (``check_inputs``)."""
    check_inputs(w)
    import torch

    dev = torch.device("cuda:0")

    def t(a):
        x = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        if layout == "bhsd" and x.dim() == 4:
            # same logical [B,S,H,D] tensor held in [B,H,S,D] memory order
            x = x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        return x

    q, k, v = t(w.q), t(w.k), t(w.v)
    cu = None if w.cu_seqlens is None else torch.from_numpy(w.cu_seqlens.astype(np.int32)).to(dev)
    sp = {}
    if w.row_ptr is not None:
        sp["block_list"] = (torch.from_numpy(w.row_ptr.astype(np.int32)).to(dev),
                            torch.from_numpy(w.col_idx.astype(np.int32)).to(dev))
    if w.block_mask is not None:
        sp["block_mask"] = torch.from_numpy(np.ascontiguousarray(w.block_mask).view(np.int32)).to(dev)
    return q, k, v, cu, sp


def run_gpu(w: W.Workload, layout: str = "bshd", tensors=None):
    """GPU output in packed order: O float64 [T, Hq, D], LSE float64 [T, Hq]."""
    import torch
    import attention_forward_flashattention_amd as attn

    q, k, v, cu, sp = tensors if tensors is not None else to_device(w, layout)
    out, lse = attn.attn_fwd(q, k, v, cu_seqlens=cu, causal=w.causal, scale=w.scale,
                             max_seqlen=w.seqlen if cu is not None else None, **sp)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    if cu is None:
        o = o.reshape(w.batch * w.seqlen, w.hq, w.d)
        l = l.transpose(0, 2, 1).reshape(w.batch * w.seqlen, w.hq)   # [B,H,S] -> tokens
    else:
        l = l.T                                                      # [H,T] -> [T,H]
    return o, l


def sample_tokens(w: W.Workload, per_seq: int = 48, seed: int = 0) -> np.ndarray:
    """Packed token ids: tile edges and ends of every sequence plus random rows."""
    rng = np.random.default_rng(seed)
    cu = w.cu_seqlens_or_fixed().astype(np.int64)
    out = []
    for b in range(len(cu) - 1):
        n = int(cu[b + 1] - cu[b])
        if n == 0:
            continue
        fixed = {0, 1, 63, 64, 127, 128, 129, 255, 256, n - 129, n - 128, n - 65, n - 64, n - 2, n - 1}
        fixed = {p for p in fixed if 0 <= p < n}
        rest = rng.choice(n, size=min(n, per_seq), replace=False)
        out.extend(int(cu[b]) + p for p in sorted(fixed | set(int(x) for x in rest)))
    return np.array(sorted(set(out)), dtype=np.int64)


def compare(o_gpu, l_gpu, o_ref, l_ref, label=""):
    """Check the tolerances; returns a dict of error statistics."""
    assert o_gpu.shape == o_ref.shape and l_gpu.shape == l_ref.shape, (label, o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{label}: non-finite O"
    assert not np.any(np.isnan(l_gpu)) and not np.any(l_gpu == np.inf), f"{label}: NaN or +inf in LSE"
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l_gpu), fin), f"{label}: LSE finiteness differs"
    assert np.all(l_gpu[~fin] == l_ref[~fin]), f"{label}: empty rows must give -inf"
    err = np.abs(o_gpu - o_ref)
    stats = {
        "o_max_abs": float(err.max()) if err.size else 0.0,
        "o_mean_abs": float(err.mean()) if err.size else 0.0,
        "lse_max_abs": float(np.abs(l_gpu[fin] - l_ref[fin]).max()) if fin.any() else 0.0,
        "o_rel_rms": float(np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-30)),
    }
    assert stats["o_max_abs"] <= O_MAX_ABS, (label, stats)
    assert stats["o_mean_abs"] <= O_MEAN_ABS, (label, stats)
    assert stats["lse_max_abs"] <= LSE_MAX_ABS, (label, stats)
    assert stats["o_rel_rms"] <= O_REL_RMS, (label, stats)
    return stats


def oracle_threads() -> int:
    """Threads for the oracle in tests (the oracle's own default: the CPUs this process
    may run on, at most 16)."""
    import oracle
    return oracle.default_threads()


def check_workload(w: W.Workload, rows=None, layout: str = "bshd", nthreads: int = 0):
    """GPU vs oracle on all rows (rows=None) or on the given packed token ids."""
    import oracle

    o, l = run_gpu(w, layout)
    o_ref, l_ref = oracle.run_workload(w, rows=rows, nthreads=nthreads or oracle_threads())
    if rows is not None:
        o, l = o[rows], l[rows]
    return compare(o, l, o_ref, l_ref, w.name)


def one_head_per_kv_head(w: W.Workload):
    """Query heads c*g + (c mod g) for each KV head c: one head of every GQA group,
    each at a different position within its group."""
    g = w.hq // w.hkv
    return [c * g + (c % g) for c in range(w.hkv)]


def oracle_heads(w: W.Workload, heads, nthreads: int = 0):
    """The oracle on every row of the given query heads (at most one per KV head):
    O [T, len(heads), D], LSE [T, len(heads)]."""
    import oracle

    g = w.hq // w.hkv
    kvh = [h // g for h in heads]
    assert len(set(kvh)) == len(kvh), "one query head per KV head"
    q, k, v = w.packed_views()
    f = lambda a: W.bf16_bits_to_f32(a).astype(np.float64)
    return oracle.attn_fwd(f(q[:, heads]), f(k[:, kvh]), f(v[:, kvh]), w.cu_seqlens_or_fixed(), w.causal,
                           w.scale, w.row_ptr, w.col_idx, 128, None, nthreads or oracle_threads(),
                           block_mask=None if w.block_mask is None else w.block_mask[:, kvh])


# ---------------------------------------------------------------------------
# Backward pass
# ---------------------------------------------------------------------------
# Gradient tolerances, per tensor: the GPU rounds P and dS to bf16 for the
# MFMAs and dq/dk/dv to bf16 on output (relative error 2^-9 each, random
# sign), and forms D from the bf16 forward output; the relative RMS error of
# a sum of such terms stays near 2^-9 ~ 2e-3.  The bounds leave a factor of
# about 5 on that.
G_REL_RMS = 1e-2   # ||g - g_ref||_2 / ||g_ref||_2
G_MAX_REL = 2e-2   # max |g - g_ref| / max |g_ref|


def bf16_tensor(a, dev, layout="bshd"):
    import torch
    x = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    if layout == "bhsd" and x.dim() == 4:
        x = x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    return x


def run_gpu_bwd(w: W.Workload, dout_bits, layout: str = "bshd", repeat: int = 1):
    """GPU forward then backward on the workload; returns dq, dk, dv as float64
    in packed order ([T, H, D]), one triple per repeat."""
    import torch
    import attention_forward_flashattention_amd as attn

    q, k, v, cu, sp = to_device(w, layout)
    if "block_list" in sp:
        raise ValueError("the backward takes a block mask, not a block list")
    do = bf16_tensor(dout_bits, q.device, layout)
    ms = w.seqlen if cu is not None else None
    out, lse = attn.attn_fwd(q, k, v, cu_seqlens=cu, causal=w.causal, scale=w.scale, max_seqlen=ms, **sp)
    res = []
    for _ in range(repeat):
        dq, dk, dv = attn.attn_bwd(q, k, v, out, do, lse, cu_seqlens=cu, causal=w.causal, scale=w.scale,
                                   max_seqlen=ms, block_mask=sp.get("block_mask"))
        torch.cuda.synchronize()
        t = w.tokens
        res.append(tuple(x.float().cpu().numpy().astype(np.float64).reshape(t, x.shape[-2], w.d)
                         for x in (dq, dk, dv)))
    return res if repeat > 1 else res[0]


def oracle_bwd(w: W.Workload, dout_bits, nthreads: int = 0):
    """fp64 oracle gradients on the same bf16 inputs, packed order."""
    import oracle
    from attn_workloads import bf16_bits_to_f32

    q, k, v = w.packed_views()
    f = lambda a: bf16_bits_to_f32(a).astype(np.float64)
    do = f(dout_bits).reshape(q.shape)
    return oracle.attn_bwd(f(q), f(k), f(v), do, w.cu_seqlens_or_fixed(), w.causal, w.scale,
                           w.block_mask, 128, nthreads)


def compare_grads(got, ref, label=""):
    """Check the gradient tolerances on (dq, dk, dv); returns the error statistics."""
    stats = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert g.shape == r.shape, (label, name, g.shape, r.shape)
        assert np.all(np.isfinite(g)), f"{label}: non-finite {name}"
        nrm = np.linalg.norm(r)
        err = np.abs(g - r)
        rel_rms = float(np.linalg.norm(g - r) / nrm) if nrm > 0 else float(np.linalg.norm(g))
        max_rel = float(err.max() / np.abs(r).max()) if np.abs(r).max() > 0 else float(err.max())
        stats[name] = (rel_rms, max_rel)
        assert rel_rms <= G_REL_RMS and max_rel <= G_MAX_REL, (label, name, stats[name])
    return stats


# ---------------------------------------------------------------------------
# Ordered skipping
# ---------------------------------------------------------------------------
OSK_BAND = 1e-3   # relative band around tau where fp32 and fp64 test values may disagree


def run_gpu_osk(w: W.Workload, tau: float, min_visit: int, tensors=None):
    """GPU ordered-skipping forward: O float64 [T, Hq, D], LSE [T, Hq], visited int [Hq, n_qblk]."""
    import torch
    import attention_forward_flashattention_amd as attn

    q, k, v, cu, sp = tensors if tensors is not None else to_device(w)
    out, lse, vis = attn.attn_fwd_osk(q, k, v, sp["block_list"], tau, min_visit, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64).reshape(w.seqlen, w.hq, w.d)
    l = lse.cpu().numpy().astype(np.float64)[0].T
    return o, l, vis.cpu().numpy()


def osk_trace(w: W.Workload, qblocks, nthreads: int = 0):
    """The oracle's test value after every entry of the selected query blocks'
    lists (tau = 0 walks each list to its end): [Hq, nnz] (NaN elsewhere)."""
    import oracle
    from attn_workloads import bf16_bits_to_f32

    q, k, v = (bf16_bits_to_f32(x).astype(np.float64).reshape(w.seqlen, -1, w.d) for x in (w.q, w.k, w.v))
    _, _, _, ratio = oracle.attn_fwd_osk(q, k, v, w.causal, w.scale, w.row_ptr, w.col_idx, 0.0, 1,
                                         qblocks=qblocks, nthreads=nthreads)
    return ratio


def check_visited(w: W.Workload, visited, ratio, tau: float, min_visit: int, qblocks):
    """Every GPU stop is a valid stop of the rule within the band: the test value
    at the stop is <= tau (unless the list ran out) and every earlier value from
    min_visit on is > tau, each up to OSK_BAND relative."""
    for h in range(w.hq):
        for qb in qblocks:
            e0, e1 = int(w.row_ptr[qb]), int(w.row_ptr[qb + 1])
            vis = int(visited[h, qb])
            r = ratio[h, e0:e1]
            assert 1 <= vis <= e1 - e0, (h, qb, vis)
            if vis < e1 - e0:
                assert vis >= min_visit and r[vis - 1] <= tau * (1 + OSK_BAND), (h, qb, vis, r[vis - 1])
            early = r[min_visit - 1:vis - 1]
            assert np.all(early > tau * (1 - OSK_BAND)), (h, qb, vis, early.min() if len(early) else None)
    return True


def oracle_prefix_rows(w: W.Workload, visited, rows, nthreads: int = 0):
    """Exact attention of the given rows over each (head, query block)'s visited
    prefix of the list: O [len(rows), Hq, D], LSE [len(rows), Hq]."""
    import oracle
    from attn_workloads import bf16_bits_to_f32

    q, k, v = (bf16_bits_to_f32(x).astype(np.float64).reshape(w.seqlen, -1, w.d) for x in (w.q, w.k, w.v))
    g = w.hq // w.hkv
    n_qblk = len(w.row_ptr) - 1
    O = np.zeros((len(rows), w.hq, w.d))
    L = np.zeros((len(rows), w.hq))
    for h in range(w.hq):
        rp = np.zeros(n_qblk + 1, np.int32)
        ci = []
        for qb in range(n_qblk):
            e0 = int(w.row_ptr[qb])
            ci.extend(w.col_idx[e0:e0 + int(visited[h, qb])])
            rp[qb + 1] = len(ci)
        o, l = oracle.attn_fwd(q[rows][:, h:h + 1], k[:, h // g:h // g + 1], v[:, h // g:h // g + 1],
                               np.array([0, w.seqlen], np.int32), w.causal, w.scale, rp,
                               np.array(ci, np.int32), 128, rows=rows, nthreads=nthreads)
        O[:, h] = o[:, 0]
        L[:, h] = l[:, 0]
    return O, L
