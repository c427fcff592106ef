"""Benchmark: fused attention forward on one MI355X.

A step is one forward pass (one ``attn_fwd`` launch) over the headline
workload, by default the long-context block-sparse causal GQA problem: B=1,
Hq=32, Hkv=8, S=131072, D=128, an ordered per-query-block list of 128x128 KV
blocks (sink, diagonal, previous block, then top-scoring blocks up to 10% of
the causally visible ones), bf16 inputs resident in HBM.  Prints ONE JSON line
with causal-adjusted TFLOP/s on the listed pairs, the roofline fraction of the
kernel against the bf16 dense MFMA peak, the dense causal launch on the same
inputs (its own fraction of peak, and the block-sparse speedup over it), the
other dense causal workloads (MHA S=2048 cold and warm cache, GQA S=8192) as
extra keys, and the fp64 CPU oracle timed on a bounded sample of the headline
workload.  Secondary objects time ``attn_bwd`` and ``attn_entmax_fwd`` on the
MHA workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload sparse]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import attn_workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E peak
METRIC = "attention fwd TFLOPS (bf16, causal-adjusted) and % of MFMA bf16 peak, 1 GPU"
KERNEL_SRCS = [os.path.join(ROOT, "attention_forward_flashattention_amd", "csrc", f)
               for f in ("attn_fwd.hip", "attn_common.h")]
PROFILES = os.path.join(ROOT, "profiles")

DESCRIPTIONS = {
    "tiny": "tiny dense non-causal B=1 H=2 S=128 D=64",
    "mha": "dense causal MHA B=4 H=16 S=2048 D=128",
    "gqa": "causal GQA B=2 Hq=32 Hkv=8 S=8192 D=128",
    "varlen_d64": "packed varlen causal GQA, 8 seqs of 512..16384, Hq=32 Hkv=8 D=64",
    "varlen_d128": "packed varlen causal GQA, 8 seqs of 512..16384, Hq=32 Hkv=8 D=128",
    "varlen_d256": "packed varlen causal GQA, 8 seqs of 512..16384, Hq=32 Hkv=8 D=256",
    "sparse": ("block-sparse causal GQA B=1 Hq=32 Hkv=8 S=131072 D=128, ordered per-query-block list "
               "of 128x128 blocks (sink, diagonal, previous, top-scoring up to 10% of the visible blocks)"),
    "sparse_mask": ("block-sparse causal GQA B=1 Hq=32 Hkv=8 S=131072 D=128, bit-packed mask per KV head "
                    "(same rule, own block scores per KV head)"),
    "sparse_osk": ("ordered skipping, causal GQA B=1 Hq=32 Hkv=8 S=131072 D=128, planted block relevance, "
                   "lists of a quarter of the causal blocks"),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    """sha256[:16] of the forward kernel's sources (attn_fwd.hip, then attn_common.h)."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the forward kernel on this workload, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs (profiles/traffic_attn_fwd_<workload>.json),
    or None when there is no record for this workload or the kernel source changed
    since the counters were taken."""
    try:
        rec = json.load(open(os.path.join(PROFILES, f"traffic_attn_fwd_{workload}.json")))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_src_sha256_16") != kernel_hash() or rec.get("workload_name") != workload:
        return None
    return rec.get("bytes_per_launch")


def roofline(w: W.Workload, flops: float, ms: float, workload: str):
    """Roofline object of one launch: the bound follows from the arithmetic intensity
    (counted FLOPs over algorithmic bytes) against the ridge peak_flops / peak_bw."""
    byt = W.algorithmic_bytes(w)
    intensity = flops / byt
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if intensity >= ridge:
        achieved, peak, unit, bound = flops / (ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = byt / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": measured_traffic(workload),
            "algorithmic_bytes": byt, "flop_per_byte": round(intensity, 1)}


def host_cpus():
    """What the host reports about its CPUs: online count, this process's affinity,
    the cgroup CPU quota and the model name."""
    info = {"online": os.cpu_count()}
    try:
        info["affinity"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()
        info["cgroup_quota_cpus"] = None if quota == "max" else round(int(quota) / int(period), 2)
    except (OSError, ValueError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return info


def row_pairs(w: W.Workload, rows: np.ndarray) -> np.ndarray:
    """Counted (query, key) pairs per query row (packed token ids): the size of the
    row's allowed set (causal, packed, or under the block list)."""
    cu = w.cu_seqlens_or_fixed().astype(np.int64)
    seq = np.searchsorted(cu, rows, side="right") - 1
    pos = rows - cu[seq]
    length = cu[seq + 1] - cu[seq]
    if w.row_ptr is None:
        return (pos + 1).astype(np.float64) if w.causal else length.astype(np.float64)
    out = np.zeros(len(rows))
    for n, (i, L) in enumerate(zip(pos, length)):
        qb = int(i) // W.SPARSE_BLOCK
        for cb in w.col_idx[w.row_ptr[qb]:w.row_ptr[qb + 1]]:
            lo = int(cb) * W.SPARSE_BLOCK
            hi = min(lo + W.SPARSE_BLOCK, int(L), int(i) + 1 if w.causal else int(L))
            out[n] += max(0, hi - lo)
    return out


def cpu_baseline(w: W.Workload, budget_s: float = 15.0):
    """The fp64 oracle timed on the host cores on a bounded sample of the workload's
    query rows (all heads of each row), scaled by counted pairs to the whole workload.

    The sample is the workload's own checked rows when it has them (the 128K
    block-sparse workload: 256 rows), then random rows sized to about
    ``budget_s`` of oracle time; the reported rate is that of the larger sample.
    Reported in the metric's unit: counted FLOPs per second."""
    import oracle

    threads = oracle.default_threads()
    rng = np.random.default_rng(1234)
    t_all = w.tokens
    total_pairs = float(row_pairs(w, np.arange(t_all)).sum()) if w.row_ptr is None else \
        W.counted_flops(w) / (4.0 * w.d * w.hq)
    first = w.sample_rows if w.sample_rows is not None else np.sort(rng.choice(t_all, min(256, t_all), False))
    t0 = time.perf_counter()
    oracle.run_workload(w, rows=first, nthreads=threads)
    t_first = time.perf_counter() - t0
    p_first = float(row_pairs(w, first).sum())
    rate = p_first / t_first          # pairs x heads / s, per head below
    n = int(min(t_all, max(len(first), budget_s * rate / max(total_pairs / t_all, 1.0))))
    rows, spent, pairs = first, t_first, p_first
    if n > 2 * len(first):
        rows = np.sort(rng.choice(t_all, size=n, replace=False))
        t0 = time.perf_counter()
        oracle.run_workload(w, rows=rows, nthreads=threads)
        spent = time.perf_counter() - t0
        pairs = float(row_pairs(w, rows).sum())
    flops = 4.0 * w.d * w.hq * pairs
    full_s = spent * total_pairs / pairs
    sample = (f"{len(rows)} query rows x {w.hq} heads of the same workload "
              f"({'every row' if len(rows) == t_all else 'random rows'}), fp64 oracle on {threads} threads, "
              f"{spent:.1f} s; scaled by counted pairs to a full-run estimate of {full_s:.0f} s "
              f"(extrapolated); the {len(first)} checked rows alone took {t_first:.2f} s")
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": sample, "full_run_s_extrapolated": round(full_s, 1), "host_cpus": host_cpus()}


def osk_flops(w: W.Workload, visited: np.ndarray):
    """FLOPs of the visited prefixes (4*D per counted pair, the diagonal block
    counted half under causal masking) and the fraction of listed entries skipped."""
    n_qblk = len(w.row_ptr) - 1
    pairs = 0.0
    listed = 0
    for qb in range(n_qblk):
        e0, e1 = int(w.row_ptr[qb]), int(w.row_ptr[qb + 1])
        ents = w.col_idx[e0:e1]
        wgt = np.where(ents == qb, 0.5, 1.0) if w.causal else np.ones(len(ents))
        cum = np.concatenate([[0.0], np.cumsum(wgt)])
        pairs += float(cum[visited[:, qb]].sum())
        listed += (e1 - e0) * w.hq
    flops = 4.0 * w.d * W.SPARSE_BLOCK * W.SPARSE_BLOCK * pairs
    return flops, 1.0 - float(visited.sum()) / listed


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------
def settle(torch, fn, ms: float):
    """Back-to-back launches for ``ms`` milliseconds: the GPU raises its engine clock
    over the first tens of milliseconds of load."""
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms or n < 2:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def time_back_to_back(torch, fn, n: int) -> float:
    """Average ms of n back-to-back launches between two events on the launch stream
    (torch's current stream, which the binding passes to the library)."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def time_cold(torch, fn, reps: int, device):
    """Single launches with L2 and the 256 MiB Infinity Cache evicted before each
    (a 512 MiB write outside the events): median and min ms."""
    if reps <= 0:
        return None
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=device)
    t = []
    for _ in range(reps):
        scratch.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1))
    del scratch
    return float(np.median(t)), float(min(t))


def fwd_step(attn, w, t, out, lse, dense=False):
    q, k, v, cu, sp = t
    kw = {} if dense else sp

    def step():
        attn.attn_fwd(q, k, v, cu_seqlens=cu, causal=w.causal, scale=w.scale, out=out, lse=lse,
                      max_seqlen=w.seqlen if cu is not None else None, **kw)
    return step


def lse_buffer(torch, w, q, cu):
    if cu is None:
        return torch.empty((w.batch, w.hq, w.seqlen), dtype=torch.float32, device=q.device)
    return torch.empty((w.hq, q.shape[0]), dtype=torch.float32, device=q.device)


def dense_extra(attn, torch, P, name: str, steps: int, settle_ms: float, cold_reps: int):
    """A dense causal workload timed warm (back to back) and cold (caches evicted)."""
    w = W.make(name)
    t = P.to_device(w)
    out = torch.empty_like(t[0])
    lse = lse_buffer(torch, w, t[0], t[3])
    step = fwd_step(attn, w, t, out, lse)
    flops = W.counted_flops(w)
    settle(torch, step, settle_ms)
    warm = time_back_to_back(torch, step, steps)
    cold = time_cold(torch, step, cold_reps, t[0].device)
    res = {"workload": DESCRIPTIONS[name], "flops_per_launch": flops,
           "warm_ms": round(warm, 5), "warm_tflops": round(flops / warm / 1e9, 2),
           "warm_frac_of_peak": round(flops / warm / 1e9 / PEAK_BF16_TFLOPS, 4)}
    if cold:
        res.update({"cold_ms_median": round(cold[0], 5), "cold_ms_min": round(cold[1], 5),
                    "cold_tflops": round(flops / cold[0] / 1e9, 2),
                    "cold_frac_of_peak": round(flops / cold[0] / 1e9 / PEAK_BF16_TFLOPS, 4)})
    log(f"{name}: warm {warm * 1e3:.1f} us = {res['warm_tflops']} TFLOP/s ({100 * res['warm_frac_of_peak']:.1f}%)"
        + (f", cold median {cold[0] * 1e3:.1f} us = {res['cold_tflops']} TFLOP/s" if cold else ""))
    return res, (w, t, out, lse, warm)


def time_entmax(attn, torch, w, q, k, v, softmax_ms, n, settle_ms, alpha=1.5):
    """Average time of one attn_entmax_fwd call (alpha-entmax forward, solver
    run to convergence) on the same inputs, against the softmax forward's
    time, and the share of causal blocks its output pass visits."""
    out = torch.empty_like(q)

    def run():
        return attn.attn_entmax_fwd(q, k, v, alpha, causal=w.causal, scale=w.scale, n_iter=16, out=out,
                                    return_mask=True)
    settle(torch, run, settle_ms)
    ms_e = time_back_to_back(torch, run, n)
    _, _, mask = run()
    torch.cuda.synchronize()
    visited = int(np.unpackbits(mask.cpu().numpy().view(np.uint8)).sum())
    nq = (w.seqlen + 127) // 128
    blocks = w.batch * w.hq * (nq * (nq + 1) // 2 if w.causal else nq * nq)
    return {"workload": DESCRIPTIONS.get(w.name, w.name), "alpha": alpha, "ms_per_call": round(ms_e, 5),
            "calls": n, "time_vs_softmax_forward": round(ms_e / softmax_ms, 3),
            "output_pass_block_fraction": round(visited / blocks, 4),
            "kernel": "attn_entmax_kernel (max and histogram pass, refinement passes to convergence, sparse output pass)"}


def time_backward(attn, torch, w, q, k, v, cu, sp, out, lse, flops, n, settle_ms):
    """Average time of one attn_bwd call (its dQ and dK/dV kernels) over n
    back-to-back calls on the launch stream, after the forward filled out/lse.

    TFLOP/s use the usual backward count: 2.5 x the forward's counted FLOPs
    (five matrix products of the forward's size: S, dP, dV, dK, dQ); the
    kernels recompute S and dP once more for dQ, which that count leaves out."""
    g = torch.from_numpy(W.make_dout(w).view(np.int16)).view(torch.bfloat16).to(q.device)
    ms = w.seqlen if cu is not None else None
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(16, 8 * w.hq * w.batch * w.seqlen), dtype=torch.uint8, device=q.device)

    def run():
        attn.attn_bwd(q, k, v, out, g, lse, cu_seqlens=cu, causal=w.causal, scale=w.scale, max_seqlen=ms,
                      block_mask=sp.get("block_mask"), dq=dq, dk=dk, dv=dv, workspace=ws)

    settle(torch, run, settle_ms)
    ms_b = time_back_to_back(torch, run, n)
    tf = 2.5 * flops / (ms_b * 1e-3) / 1e12
    return {"workload": DESCRIPTIONS.get(w.name, w.name), "ms_per_call": round(ms_b, 5), "calls": n,
            "tflops": round(tf, 3), "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            "flop_convention": "2.5 x forward counted FLOPs (S, dP, dV, dK, dQ products)",
            "kernels": "attn_bwd_dq_kernel then attn_bwd_dkdv_kernel"}


def results_table(attn, torch, P, settle_ms: float):
    """One measured row per workload (tiny, mha, gqa, varlen D=64/128/256, the 128K
    block list and its dense leg): errors against the fp64 oracle, kernel time
    warm (back to back) and cold (caches evicted), TFLOP/s and % of the bf16
    peak, and the oracle's CPU time.  Printed as a markdown table.

    Parity is over every output for tiny, mha and gqa; for the packed varlen
    workloads over every row of one query head per KV head (the oracle time is
    that of those heads, scaled by Hq / Hkv to all heads); for the 128K list over
    its 256 checked rows on all heads (scaled by counted pairs to the full run).
    """
    import oracle

    threads = oracle.default_threads()
    rows_md = []
    for name in ("tiny", "mha", "gqa", "varlen_d64", "varlen_d128", "varlen_d256", "sparse"):
        w = W.make(name)
        t = P.to_device(w)
        q, cu = t[0], t[3]
        out = torch.empty_like(q)
        lse = lse_buffer(torch, w, q, cu)
        legs = [("", fwd_step(attn, w, t, out, lse), W.counted_flops(w))]
        if name == "sparse":
            wd = W.Workload(w.name, w.seed, w.batch, w.seqlen, w.hq, w.hkv, w.d, w.causal, w.scale, w.q, w.k, w.v)
            legs.append((" (dense causal, same inputs)", fwd_step(attn, w, t, out, lse, dense=True),
                         W.counted_flops(wd)))
        timing = []
        for label, step, flops in legs:
            settle(torch, step, settle_ms)
            one = time_back_to_back(torch, step, 1)
            warm = time_back_to_back(torch, step, max(3, min(200, int(300.0 / max(one, 1e-3)))))
            cold = time_cold(torch, step, 5, q.device)
            timing.append((label, flops, warm, cold))
        # parity: the run of the workload's own step (the first leg)
        legs[0][1]()
        torch.cuda.synchronize()
        o, l = P.run_gpu(w, tensors=t)
        t0 = time.perf_counter()
        if name in ("tiny", "mha", "gqa"):
            o_ref, l_ref = oracle.run_workload(w, nthreads=threads)
            cpu_s = time.perf_counter() - t0
            st = P.compare(o, l, o_ref, l_ref, name)
            cpu_note = f"{cpu_s:.1f} s"
        elif name.startswith("varlen"):
            heads = P.one_head_per_kv_head(w)
            o_ref, l_ref = P.oracle_heads(w, heads, nthreads=threads)
            cpu_s = (time.perf_counter() - t0) * w.hq / len(heads)
            st = P.compare(o[:, heads], l[:, heads], o_ref, l_ref, name)
            cpu_note = f"{cpu_s:.0f} s (from {len(heads)} of {w.hq} heads)"
        else:
            rows = w.sample_rows
            o_ref, l_ref = oracle.run_workload(w, rows=rows, nthreads=threads)
            spent = time.perf_counter() - t0
            cpu_s = spent * (W.counted_flops(w) / (4.0 * w.d * w.hq)) / float(row_pairs(w, rows).sum())
            st = P.compare(o[rows], l[rows], o_ref, l_ref, name)
            cpu_note = f"{spent:.1f} s for {len(rows)} rows; {cpu_s:.0f} s full run (extrapolated)"
        for i, (label, flops, warm, cold) in enumerate(timing):
            tf = flops / warm / 1e9
            err = (f"{st['o_max_abs']:.2e} | {st['o_mean_abs']:.2e} | {st['lse_max_abs']:.2e}" if i == 0
                   else "— | — | —")
            rows_md.append(f"| {name}{label} | {err} | {warm:.4f} / {cold[0]:.4f} | {tf:.1f} | "
                           f"{100 * tf / PEAK_BF16_TFLOPS:.1f} | {cpu_note if i == 0 else '—'} |")
            log(rows_md[-1])
        del t, q, out, lse
        torch.cuda.empty_cache()
    head = ("| config | O max abs err | O mean abs err | LSE max abs err | kernel ms warm / cold (median) | "
            "TFLOP/s (warm) | % of bf16 peak | CPU oracle time (" + str(threads) + " threads) |\n"
            "|---|---|---|---|---|---|---|---|")
    print(head)
    print("\n".join(rows_md), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed back-to-back launches for this long before the warm-up steps "
                         "(the GPU clock takes tens of milliseconds of load to reach its sustained level)")
    ap.add_argument("--workload", default="sparse", choices=list(W.CONFIG_NAMES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-reps", type=int, default=5,
                    help="launches timed one by one after evicting the caches (secondary figure)")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the workload alone: no dense leg, no other workloads, no backward or entmax")
    ap.add_argument("--osk-tau", type=float, default=1e-2,
                    help="sparse_osk workload: the ordered-skipping stop threshold tau")
    ap.add_argument("--osk-min-visit", type=int, default=2,
                    help="sparse_osk workload: entries visited before the stop test applies")
    ap.add_argument("--no-entmax", action="store_true", help="skip the alpha-entmax timing")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (HBM counter calibration)")
    ap.add_argument("--results-table", action="store_true",
                    help="measure every workload once (errors against the oracle, warm and cold kernel time, "
                         "TFLOP/s, CPU oracle time) and print a markdown table instead of the JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the attention forward here is a "
              "single-GPU kernel and no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give the
        # scale between those counters and bytes actually moved.
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {args.warmup + args.steps} copies of {n} bytes")
        return

    import attention_forward_flashattention_amd as attn
    from tests import _parity as P

    log(f"library {attn.LIB_PATH} built from sources {attn.source_sha()} (forward kernel {kernel_hash()})")
    if args.results_table:
        results_table(attn, torch, P, args.settle_ms)
        return
    t_gen = time.perf_counter()
    w = W.make(args.workload)
    flops = W.counted_flops(w)
    t = P.to_device(w)
    q, k, v, cu, sp = t
    out = torch.empty_like(q)
    lse = lse_buffer(torch, w, q, cu)
    log(f"workload {w.name}: inputs generated and resident in {time.perf_counter() - t_gen:.1f} s")

    osk = w.name == "sparse_osk"
    if osk:
        visited = torch.empty((w.hq, len(w.row_ptr) - 1), dtype=torch.int32, device=q.device)

        def step():
            attn.attn_fwd_osk(q, k, v, sp["block_list"], args.osk_tau, args.osk_min_visit, causal=w.causal,
                              scale=w.scale, out=out, lse=lse, visited=visited)

        # the FLOPs of ordered skipping are those of the entries it visits
        step()
        torch.cuda.synchronize()
        flops, skip_rate = osk_flops(w, visited.cpu().numpy())
    else:
        step = fwd_step(attn, w, t, out, lse)

    # Timed region: K back-to-back steps between two events on the launch stream,
    # after the clock settled and W warm-up steps.  A step is one kernel launch, so
    # the per-step time is the average launch duration.
    n_settle = settle(torch, step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_per_step = time_back_to_back(torch, step, args.steps)
    wall = time.perf_counter() - t0
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    log(f"workload {w.name}: {flops / 1e12:.3f} TFLOP/launch, {ms_per_step:.4f} ms/step back to back "
        f"(wall {wall * 1e3 / args.steps:.4f} ms/step, {n_settle} settle launches): {tflops:.1f} TFLOP/s = "
        f"{100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak")
    extra = {}
    cold = time_cold(torch, step, args.cold_reps, q.device)
    if cold:
        extra["cold_cache_ms_median"] = round(cold[0], 5)
        extra["cold_cache_ms_min"] = round(cold[1], 5)
        log(f"cold cache (L2 and Infinity Cache evicted before each launch): median {cold[0]:.4f} ms, "
            f"min {cold[1]:.4f} ms over {args.cold_reps} launches")

    if osk:
        # ordered skipping against the static list on the same inputs: speedup,
        # and the error it makes against the static list's exact result
        o_osk = out.float().clone()
        out_s = torch.empty_like(out)

        def static():
            attn.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out=out_s, lse=lse, **sp)
        static()
        static_ms = time_back_to_back(torch, static, max(2, args.steps // 5))
        ref = out_s.float()
        diff = o_osk - ref
        extra["osk"] = {"tau": args.osk_tau, "min_visit": args.osk_min_visit,
                        "skipped_entry_fraction": round(skip_rate, 4),
                        "static_list_ms_per_step": round(static_ms, 4),
                        "speedup_vs_static_list": round(static_ms / ms_per_step, 3),
                        "o_rel_rms_vs_static_list": float(diff.norm() / ref.norm()),
                        "o_max_abs_vs_static_list": float(diff.abs().max()),
                        "flops_convention": "4*D per visited (query, key) pair x Hq"}
        log(f"ordered skipping tau={args.osk_tau}: {extra['osk']}")

    if sp and not osk and not args.no_extras:
        # the dense causal launch on the same inputs: its own fraction of peak, and
        # the block-sparse speedup over it
        dense = fwd_step(attn, w, t, out, lse, dense=True)
        dense()
        dense_ms = time_back_to_back(torch, dense, max(2, args.steps // 7))
        wd = W.Workload(w.name, w.seed, w.batch, w.seqlen, w.hq, w.hkv, w.d, w.causal, w.scale, w.q, w.k, w.v,
                        cu_seqlens=w.cu_seqlens)
        dflops = W.counted_flops(wd)
        extra["dense_causal"] = {"ms_per_step": round(dense_ms, 4), "flops_per_launch": dflops,
                                 "tflops": round(dflops / dense_ms / 1e9, 2),
                                 "frac_of_peak": round(dflops / dense_ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
        extra["sparse_speedup"] = round(dense_ms / ms_per_step, 3)
        extra["sparse_speedup_ideal"] = round(dflops / flops, 3)
        log(f"dense causal on the same inputs: {dense_ms:.2f} ms/step = {extra['dense_causal']['tflops']} TFLOP/s; "
            f"block-sparse speedup {extra['sparse_speedup']}x (ideal {extra['sparse_speedup_ideal']}x)")

    bwd = ent = None
    if not args.no_extras and not osk:
        # the other dense causal workloads, and the backward / entmax objects on MHA
        for name in ("mha", "gqa"):
            if name == w.name:
                continue
            res, keep = dense_extra(attn, torch, P, name, max(args.steps, 50) if name == "mha" else args.steps,
                                    args.settle_ms / 2, 10 if name == "mha" else 3)
            extra[name] = res
            if name == "mha":
                mha_keep = keep
        if w.name == "mha":
            mha_keep = (w, t, out, lse, ms_per_step)
        wm, tm, outm, lsem, msm = mha_keep
        fm = W.counted_flops(wm)
        if not args.no_backward:
            bwd = time_backward(attn, torch, wm, tm[0], tm[1], tm[2], tm[3], tm[4], outm, lsem, fm, 20,
                                args.settle_ms / 2)
            log(f"backward: {bwd}")
        if not args.no_entmax:
            ent = time_entmax(attn, torch, wm, tm[0], tm[1], tm[2], msm, 10, args.settle_ms / 2)
            log(f"entmax: {ent}")

    cpu = None
    if not args.no_cpu_baseline and not osk:
        cpu = cpu_baseline(w)
        log(f"cpu oracle: {cpu}")

    rec = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": ("synthetic: seeded N(0,1) noise plus planted block relevance, rounded to bf16" if osk else
                 "synthetic: i.i.d. N(0,1) inputs rounded to bf16, seeded"),
        "config": {"workload": f"{w.name}: {DESCRIPTIONS.get(w.name, w.name)}",
                   "batch": w.batch, "seq_len": w.seqlen, "heads_q": w.hq, "heads_kv": w.hkv,
                   "head_dim": w.d, "causal": w.causal, "flops_per_step": flops,
                   "flop_convention": "4*D per counted (query, key) pair x Hq; causal grids halved; a listed "
                                      "diagonal block counts half; skipped blocks count nothing",
                   "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
                   "library_source_sha": attn.source_sha(), **extra},
        "roofline": roofline(w, flops, ms_per_step, w.name),
        "cpu_baseline": cpu,
        "backward": bwd,
        "entmax": ent,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
