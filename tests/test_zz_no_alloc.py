"""attn_bwd_noalloc: the backward with the library's static scratch in place of a
caller workspace, called through the C ABI (the binding's ctypes call).

On the GPU it must give exactly what attn_bwd gives on the same inputs (the
same kernels; only the per-row workspace lives elsewhere), and both must meet
the gradient tolerances against the fp64 oracle, over two calls in a row with
the second on a smaller problem (the scratch keeps the first call's values,
which the second must not read).  On the CPU: a problem whose workspace
exceeds the scratch is rejected before anything is launched.
"""
import ctypes

import numpy as np
import pytest

import attention_forward_flashattention_amd as attn
import attn_workloads as W
from attention_forward_flashattention_amd import AttnTensor
from tests import _parity as P

FAKE = 0x10000  # 16-byte aligned, never dereferenced: the call returns before any launch


def test_noalloc_rejects_problems_beyond_the_scratch():
    lib = attn.load_library()
    s = 131072
    h = attn.ATTN_BWD_SCRATCH_BYTES // (8 * s) + 1   # one head more than the scratch holds
    q = AttnTensor(FAKE, 1, s, h, 128, s * h * 128, h * 128, 128)
    kv = AttnTensor(FAKE, 1, s, 1, 128, s * 128, 128, 128)
    r = ctypes.byref
    st = lib.attn_bwd_noalloc(r(q), r(kv), r(kv), r(q), r(q), FAKE, None, 1, 0.125, None, r(q), r(kv), r(kv),
                              None)
    assert st == attn.ATTN_ERR_TOO_LARGE
    assert "static scratch" in attn.status_str(st)
    assert lib.attn_bwd_workspace_size(r(q)) > attn.ATTN_BWD_SCRATCH_BYTES
    # the same sizes with one head fewer fit (checked without launching: invalid causal flag)
    h2 = h - 1
    q2 = AttnTensor(FAKE, 1, s, h2, 128, s * h2 * 128, h2 * 128, 128)
    assert lib.attn_bwd_workspace_size(r(q2)) <= attn.ATTN_BWD_SCRATCH_BYTES
    st2 = lib.attn_bwd_noalloc(r(q2), r(kv), r(kv), r(q2), r(q2), FAKE, None, 2, 0.125, None, r(q2), r(kv),
                               r(kv), None)
    assert st2 == attn.ATTN_ERR_INVALID_ARG


def _grads(w, do, noalloc: bool):
    import torch

    q, k, v, cu, sp = P.to_device(w)
    g = P.bf16_tensor(do, q.device)
    ms = w.seqlen if cu is not None else None
    out, lse = attn.attn_fwd(q, k, v, cu_seqlens=cu, causal=w.causal, scale=w.scale, max_seqlen=ms, **sp)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))   # every valid element must be written
    if noalloc:
        attn.attn_bwd_noalloc(q, k, v, out, g, lse, dq, dk, dv, cu_seqlens=cu, causal=w.causal, scale=w.scale,
                              max_seqlen=ms, block_mask=sp.get("block_mask"))
    else:
        attn.attn_bwd(q, k, v, out, g, lse, cu_seqlens=cu, causal=w.causal, scale=w.scale, max_seqlen=ms,
                      block_mask=sp.get("block_mask"), dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return tuple(x.float().cpu().numpy().astype(np.float64).reshape(w.tokens, x.shape[-2], w.d)
                 for x in (dq, dk, dv))


@pytest.mark.gpu
def test_noalloc_matches_attn_bwd_on_two_calls():
    big = W.make_dense("na_big", 71, 2, 700, 8, 2, 128, True)
    small = W.make_varlen("na_small", 72, [300, 1, 129], 4, 2, 64, True)
    n_qblk = (small.seqlen + 127) // 128
    rng = np.random.default_rng(73)
    vis = rng.random((3, 2, n_qblk, n_qblk)) < 0.6
    for i in range(n_qblk):
        vis[..., i, i] = True
    small.block_mask = W.pack_block_mask(vis)
    for w in (big, small):   # the second call is the smaller problem
        print(f"noalloc case {w.name}", flush=True)
        do = W.make_dout(w)
        got = _grads(w, do, noalloc=True)
        ref_ws = _grads(w, do, noalloc=False)
        for name, a, b in zip(("dq", "dk", "dv"), got, ref_ws):
            assert np.array_equal(a, b), (w.name, name)
        stats = P.compare_grads(got, P.oracle_bwd(w, do), w.name)
        print(f"  {stats}", flush=True)
