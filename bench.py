"""Benchmark: fused attention forward on one MI355X.

A step is one forward pass (one ``attn_fwd`` launch) over the dense causal
multi-head workload B=4, H=16, S=2048, D=128 (bf16, inputs resident in HBM).
Prints ONE JSON line with causal-adjusted TFLOP/s, the roofline fraction of
the kernel against the bf16 dense MFMA peak, and the fp64 CPU oracle timed on
a bounded sample of the same workload.  A secondary ``backward`` object times
``attn_bwd`` (dq, dk, dv from the saved LSE) on the same inputs.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload mha]
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
METRIC = "attention fwd TFLOPS (bf16, causal-adjusted) and % of MFMA bf16 peak, 1 GPU"
KERNEL_SRCS = [os.path.join(ROOT, "attention_forward_flashattention_amd", "csrc", f)
               for f in ("attn_fwd.hip", "attn_common.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn_fwd_mha.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    """sha256[:16] of the forward kernel's sources (attn_fwd.hip, then attn_common.h)."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they match this kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_src_sha256_16") != kernel_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w: W.Workload, budget_s: float = 20.0):
    """fp64 oracle timed on the host cores, on the whole workload when that fits the
    time budget, else on a bounded random sample of query rows (all heads).

    A sample's time is scaled by (pairs of the whole workload) / (pairs of the
    sample) to a full-run estimate.  Reported in the metric's unit: the
    workload's causal-adjusted FLOPs divided by the (estimated) full-run time.
    """
    import oracle

    threads = min(oracle.default_threads(), 16)
    rng = np.random.default_rng(1234)
    t_all = w.batch * w.seqlen

    def pairs(rows):
        pos = rows % w.seqlen
        return float(np.sum(pos + 1)) if w.causal else float(len(rows) * w.seqlen)

    total_pairs = pairs(np.arange(t_all))
    calib = np.sort(rng.choice(t_all, size=min(256, t_all), replace=False))
    t0 = time.perf_counter()
    oracle.run_workload(w, rows=calib, nthreads=threads)
    est_full = (time.perf_counter() - t0) * total_pairs / pairs(calib)
    if est_full <= budget_s:
        t0 = time.perf_counter()
        oracle.run_workload(w, nthreads=threads)
        full_s = time.perf_counter() - t0
        sample = f"the whole workload ({t_all} query rows x {w.hq} heads), fp64 oracle, {full_s:.1f} s"
    else:
        n = max(1, int(t_all * budget_s / est_full))
        rows = np.sort(rng.choice(t_all, size=n, replace=False))
        t0 = time.perf_counter()
        oracle.run_workload(w, rows=rows, nthreads=threads)
        spent = time.perf_counter() - t0
        full_s = spent * total_pairs / pairs(rows)
        sample = (f"{n} random query rows x {w.hq} heads of the same workload, fp64 oracle, {spent:.1f} s, "
                  f"scaled by pair count to a full-run estimate of {full_s:.0f} s")
    return {"value": W.counted_flops(w) / full_s / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "sample": sample}


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


def time_entmax(attn, torch, w, q, k, v, softmax_ms, n, settle_s, alpha=1.5):
    """Average time of one attn_entmax_fwd call (alpha-entmax forward, solver
    run to convergence) on the same inputs, against the softmax forward's
    time, and the share of causal blocks its output pass visits."""
    out = torch.empty_like(q)

    def run():
        return attn.attn_entmax_fwd(q, k, v, alpha, causal=w.causal, scale=w.scale, n_iter=16, out=out,
                                    return_mask=True)
    t0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t0 < settle_s or n_settle < 3:
        run()
        n_settle += 1
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms_e = e0.elapsed_time(e1) / n
    _, _, mask = run()
    torch.cuda.synchronize()
    visited = int(np.unpackbits(mask.cpu().numpy().view(np.uint8)).sum())
    nq = (w.seqlen + 127) // 128
    blocks = w.batch * w.hq * (nq * (nq + 1) // 2 if w.causal else nq * nq)
    return {"alpha": alpha, "ms_per_call": round(ms_e, 5), "calls": n,
            "time_vs_softmax_forward": round(ms_e / softmax_ms, 3),
            "output_pass_block_fraction": round(visited / blocks, 4),
            "kernel": "attn_entmax_kernel (max, histogram, refinement passes to convergence, sparse output pass)"}


def time_backward(attn, torch, w, q, k, v, cu, sp, out, lse, flops, n, settle_s):
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

    # settle the clock again (the cold-cache launches before this leave it low)
    t0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t0 < settle_s or n_settle < 3:
        run()
        n_settle += 1
        if n_settle % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms_b = e0.elapsed_time(e1) / n
    tf = 2.5 * flops / (ms_b * 1e-3) / 1e12
    return {"ms_per_call": round(ms_b, 5), "calls": n, "tflops": round(tf, 3),
            "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            "flop_convention": "2.5 x forward counted FLOPs (S, dP, dV, dK, dQ products)",
            "kernels": "attn_bwd_dq_kernel then attn_bwd_dkdv_kernel"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed back-to-back launches for this long before the warm-up steps "
                         "(the GPU clock takes tens of milliseconds of load to reach its sustained level)")
    ap.add_argument("--workload", default="mha", choices=list(W.CONFIG_NAMES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="launches timed one by one after evicting the caches (secondary figure)")
    ap.add_argument("--osk-tau", type=float, default=1e-2,
                    help="sparse_osk workload: the ordered-skipping stop threshold tau")
    ap.add_argument("--osk-min-visit", type=int, default=2,
                    help="sparse_osk workload: entries visited before the stop test applies")
    ap.add_argument("--no-entmax", action="store_true",
                    help="skip the secondary timing of the alpha-entmax forward")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the secondary timing of the backward pass")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (HBM counter calibration)")
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

    w = W.make(args.workload)
    flops = W.counted_flops(w)
    q, k, v, cu, sp = P.to_device(w)
    out = torch.empty_like(q)
    if cu is None:
        lse = torch.empty((w.batch, w.hq, w.seqlen), dtype=torch.float32, device=q.device)
    else:
        lse = torch.empty((w.hq, q.shape[0]), dtype=torch.float32, device=q.device)

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
        def step():
            attn.attn_fwd(q, k, v, cu_seqlens=cu, causal=w.causal, scale=w.scale, out=out, lse=lse,
                          max_seqlen=w.seqlen if cu is not None else None, **sp)

    # Settle the clock: the GPU ramps its engine clock over the first tens of
    # milliseconds of load; without this the timed steps of a short kernel run
    # partly at a lower clock than the sustained one.
    t_settle = time.perf_counter()
    n_settle = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        step()
        n_settle += 1
        if n_settle % 16 == 0:
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K back-to-back steps between two events on the launch stream
    # (torch's current stream, which the binding passes to the library).  A step
    # is one kernel launch, so the per-step time is the average launch duration.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start_all = torch.cuda.Event(enable_timing=True)
    end_all = torch.cuda.Event(enable_timing=True)
    start_all.record()
    for _ in range(args.steps):
        step()
    end_all.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start_all.elapsed_time(end_all) / args.steps
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    achieved = tflops
    # diagnostic only: spread of single-launch times (each bracketed by its own events)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for e0, e1 in evs:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    per_launch = [a.elapsed_time(b) for a, b in evs]
    log(f"workload {w.name}: {flops / 1e9:.2f} GFLOP/launch, {ms_per_step * 1e3:.1f} us/step back to back "
        f"(single launches: median {np.median(per_launch) * 1e3:.1f} us, min {min(per_launch) * 1e3:.1f} us), "
        f"wall {wall * 1e6 / args.steps:.1f} us/step, {n_settle} settle launches, {tflops:.1f} TFLOP/s = "
        f"{100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak")

    # Cold-cache launches (secondary): a 512 MiB write evicts L2 and the 256 MiB
    # Infinity Cache before each launch, outside the timed events.
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=q.device)
    cold = []
    for _ in range(args.cold_reps):
        scratch.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del scratch
    extra = {}
    if cold:
        extra["cold_cache_ms_median"] = round(float(np.median(cold)), 5)
        extra["cold_cache_ms_min"] = round(float(min(cold)), 5)
        log(f"cold cache (L2 and Infinity Cache evicted before each launch): median {np.median(cold) * 1e3:.1f} us, "
            f"min {min(cold) * 1e3:.1f} us over {len(cold)} launches")

    if osk:
        # ordered skipping against the static list on the same inputs: speedup,
        # and the error it makes against the static list's exact result
        o_osk = out.float().clone()
        out_s = torch.empty_like(out)

        def static():
            attn.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out=out_s, lse=lse, **sp)
        static()
        torch.cuda.synchronize()
        n_s = max(2, args.steps // 20)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_s):
            static()
        e1.record()
        torch.cuda.synchronize()
        static_ms = e0.elapsed_time(e1) / n_s
        ref = out_s.float()
        diff = o_osk - ref
        extra["osk"] = {"tau": args.osk_tau, "min_visit": args.osk_min_visit,
                        "skipped_entry_fraction": round(skip_rate, 4),
                        "static_list_ms_per_step": round(static_ms, 4),
                        "speedup_vs_static_list": round(static_ms / ms_per_step, 3),
                        "o_rel_rms_vs_static_list": float(diff.norm() / ref.norm()),
                        "o_max_abs_vs_static_list": float(diff.abs().max()),
                        "flops_convention": "4*D per visited (query, key) pair x Hq"}
        log(f"ordered skipping tau={args.osk_tau}: skipped {skip_rate:.3f} of the listed entries; static list "
            f"{static_ms:.2f} ms/step -> speedup {static_ms / ms_per_step:.2f}x; O vs static list: rel RMS "
            f"{extra['osk']['o_rel_rms_vs_static_list']:.2e}, max abs {extra['osk']['o_max_abs_vs_static_list']:.2e}")

    if sp and not osk:
        # block-sparse speedup: the dense causal launch on the same inputs
        def dense():
            attn.attn_fwd(q, k, v, cu_seqlens=cu, causal=w.causal, scale=w.scale, out=out, lse=lse,
                          max_seqlen=w.seqlen if cu is not None else None)
        dense()
        torch.cuda.synchronize()
        n_dense = max(2, args.steps // 20)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_dense):
            dense()
        e1.record()
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / n_dense
        wd = W.Workload(w.name, w.seed, w.batch, w.seqlen, w.hq, w.hkv, w.d, w.causal, w.scale, w.q, w.k, w.v)
        ideal = W.counted_flops(wd) / flops
        extra["dense_causal_ms_per_step"] = round(dense_ms, 4)
        extra["sparse_speedup"] = round(dense_ms / ms_per_step, 3)
        extra["sparse_speedup_ideal"] = round(ideal, 3)
        log(f"dense causal on the same inputs: {dense_ms:.2f} ms/step; block-sparse speedup "
            f"{dense_ms / ms_per_step:.2f}x (ideal {ideal:.2f}x)")

    bwd = None
    if not args.no_backward and "block_list" not in sp and not osk:
        bwd = time_backward(attn, torch, w, q, k, v, cu, sp, out, lse, flops, max(10, args.steps // 4),
                            args.settle_ms / 2e3)
        log(f"backward: {bwd}")

    ent = None
    if not args.no_entmax and not w.packed and not sp:
        ent = time_entmax(attn, torch, w, q, k, v, ms_per_step, max(10, args.steps // 10), args.settle_ms / 2e3)
        log(f"entmax: {ent}")

    cpu = None
    if not args.no_cpu_baseline and not w.packed and not sp:
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
        "config": {"workload": f"{w.name}: dense causal MHA B={w.batch} H={w.hq} S={w.seqlen} D={w.d}"
                   if w.name == "mha" else w.name,
                   "batch": w.batch, "seq_len": w.seqlen, "heads_q": w.hq, "heads_kv": w.hkv,
                   "head_dim": w.d, "causal": w.causal, "flops_per_step": flops,
                   "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2), **extra},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic()},
        "cpu_baseline": cpu,
        "backward": bwd,
        "entmax": ent,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
