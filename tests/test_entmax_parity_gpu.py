"""GPU parity of alpha-entmax attention (attn_entmax_fwd) against the fp64 oracle.

O is compared element by element with the oracle's exact entmax (tau from
bisection to rounding) at the forward's tolerances.  The GPU's tau must
solve the normalisation: sum_j [(alpha-1) z_j - tau]_+^(1/(alpha-1)),
recomputed in fp64 at the GPU's tau, within MASS_TOL of 1; for alpha <= 2 it
must also lie within TAU_ABS of the exact root.  The histogram start must
keep its bound tau* - 1/31 <= tau_h <= tau* (32 bins of width W/31, W =
1/(alpha-1); plus fp32 rounding), and the
GPU's block mask must contain every block the exact weights touch.
"""
import numpy as np
import pytest

import attn_workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu

TAU_ABS = 2e-4      # |tau_gpu - tau*| for alpha <= 2 (fp32 scores and power sums)
MASS_TOL = 1e-3     # |sum p(tau_gpu) - 1| in fp64: the kernel stops at 4e-6 in fp32, and its fp32
                    # scores differ from the exact ones by ~1e-6 relative, which the steep part of
                    # u^(1/(alpha-1)) (alpha > 2) magnifies
TAU_H_SLACK = 2e-5  # fp32 rounding of the histogram bins and of its root


def run(w, alpha, n_iter, layout="bshd"):
    import torch
    import attention_forward_flashattention_amd as attn

    q, k, v, _, _ = P.to_device(w, layout)
    out, tau, mask, tau0 = attn.attn_entmax_fwd(q, k, v, alpha, causal=w.causal, scale=w.scale, n_iter=n_iter,
                                                return_mask=True, return_tau_init=True)
    torch.cuda.synchronize()
    t = w.batch * w.seqlen
    o = out.float().cpu().numpy().astype(np.float64).reshape(t, w.hq, w.d)
    tr = lambda x: x.cpu().numpy().astype(np.float64).transpose(0, 2, 1).reshape(t, w.hq)
    return o, tr(tau), tr(tau0), mask.cpu().numpy().view(np.uint32)


def oracle_entmax(w, alpha):
    import oracle
    from attn_workloads import bf16_bits_to_f32

    q, k, v = (bf16_bits_to_f32(x).astype(np.float64) for x in w.packed_views())
    return oracle.entmax_fwd(q, k, v, w.cu_seqlens_or_fixed(), w.causal, w.scale, alpha, bins=32, with_mask=True)


def mass_error(w, alpha, tau):
    """max over rows of |sum_j [(alpha-1) z_j - tau]_+^(1/(alpha-1)) - 1| in fp64 at the given tau."""
    from attn_workloads import bf16_bits_to_f32

    q, k, _ = (bf16_bits_to_f32(x).astype(np.float64) for x in w.packed_views())
    g = w.hq // w.hkv
    worst = 0.0
    S = w.seqlen
    for b in range(w.batch):
        rows = slice(b * S, (b + 1) * S)
        for h in range(w.hq):
            z = w.scale * q[rows, h] @ k[rows, h // g].T
            u = (alpha - 1.0) * z - tau[rows, h][:, None]
            if w.causal:
                u = np.where(np.tri(S, dtype=bool), u, -1.0)
            m = (np.clip(u, 0.0, None) ** (1.0 / (alpha - 1.0))).sum(1)
            worst = max(worst, float(np.abs(m - 1.0).max()))
    return worst


def check(w, alpha, n_iter, layout="bshd"):
    print(f"entmax case {w.name} alpha={alpha} n_iter={n_iter}", flush=True)
    o, tau, tau0, mask = run(w, alpha, n_iter, layout)
    o_ref, tau_ref, _, mask_ref = oracle_entmax(w, alpha)
    lse_like = np.zeros_like(tau)
    stats = P.compare(o, lse_like, o_ref, lse_like, f"entmax {w.name} alpha={alpha}")
    terr = float(np.abs(tau - tau_ref).max())
    merr = mass_error(w, alpha, tau)
    assert merr <= MASS_TOL, (w.name, alpha, merr)
    if alpha <= 2:
        assert terr <= TAU_ABS, (w.name, alpha, terr)
    assert np.all(tau0 <= tau_ref + TAU_H_SLACK) and np.all(tau0 >= tau_ref - 1.0 / 31 - TAU_H_SLACK)
    assert np.array_equal(mask & mask_ref, mask_ref), "a block with non-zero weight was not visited"
    n_vis, n_need = int(np.unpackbits(mask.view(np.uint8)).sum()), int(np.unpackbits(mask_ref.view(np.uint8)).sum())
    stats.update(tau_max_abs=terr, mass_err=merr, blocks_visited=n_vis, blocks_needed=n_need)
    print(f"  {stats}", flush=True)
    return stats


CASES = [
    # name, seed, B, S, Hq, Hkv, D, causal, alpha, n_iter (the cap on refinement steps)
    ("e_tiny", 61, 1, 128, 2, 2, 64, False, 1.5, 16),
    ("e_causal", 62, 2, 300, 4, 2, 128, True, 1.5, 16),
    ("e_sparsemax", 63, 1, 257, 2, 1, 128, True, 2.0, 16),
    ("e_halley", 64, 1, 200, 2, 2, 64, False, 1.25, 16),
    ("e_secant", 65, 1, 390, 4, 4, 128, True, 3.0, 32),
    ("e_secant_mid", 69, 1, 260, 2, 1, 64, False, 2.5, 32),
    ("e_newton", 66, 2, 129, 2, 1, 128, False, 1.75, 16),
    ("e_alpha_low", 70, 1, 200, 2, 1, 64, True, 1.05, 16),   # e = 20: the steepest weights allowed
    ("e_d256_causal", 71, 2, 300, 4, 2, 256, True, 1.5, 16),  # head_dim 256: 32-key tiles
    ("e_d256_secant", 72, 1, 230, 2, 1, 256, False, 2.5, 32),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_entmax_parity(case):
    name, seed, b, s, hq, hkv, d, causal, alpha, n_iter = case
    check(W.make_dense(name, seed, b, s, hq, hkv, d, causal), alpha, n_iter)


def test_entmax_strided_layout_bitwise():
    w = W.make_dense("e_bhsd", 67, 2, 190, 4, 2, 128, True)
    a = run(w, 1.5, 16)
    b = run(w, 1.5, 16, layout="bhsd")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_entmax_sparse_blocks_skipped():
    """Planted block relevance (a few key blocks hold the mass, as in long
    context): most causal blocks carry no weight and are not visited."""
    w = W.make_osk("e_planted", 68, 4096, 2, 1, 64)
    w.row_ptr = w.col_idx = None          # dense causal attention over these inputs
    st = check(w, 1.5, 16)
    n_qblk = 32
    causal_blocks = n_qblk * (n_qblk + 1) // 2 * w.hq
    print(f"  visited {st['blocks_visited']} of {causal_blocks} causal blocks", flush=True)
    assert st["blocks_visited"] < 0.5 * causal_blocks


def test_entmax_full_size_sampled_heads():
    """The dense causal MHA workload (B=4, H=16, S=2048, D=128) at alpha = 1.5:
    two (sequence, head) units against the oracle."""
    import oracle
    from attn_workloads import bf16_bits_to_f32

    w = W.make("mha")
    print("entmax full size", flush=True)
    o, tau, _, mask = run(w, 1.5, 16)
    f = lambda a: bf16_bits_to_f32(a).astype(np.float64)
    S = w.seqlen
    for b, h in ((0, 3), (3, 14)):
        o_ref, tau_ref, _ = oracle.entmax_fwd(f(w.q[b, :, h:h + 1]), f(w.k[b, :, h:h + 1]), f(w.v[b, :, h:h + 1]),
                                              np.array([0, S], np.int32), True, w.scale, 1.5)
        rows = slice(b * S, (b + 1) * S)
        z = np.zeros((S, 1))
        print(f"  unit b={b} h={h}: {P.compare(o[rows, h:h + 1], z, o_ref, z, 'entmax mha')}, "
              f"tau {np.abs(tau[rows, h] - tau_ref[:, 0]).max():.2e}", flush=True)
        assert np.abs(tau[rows, h] - tau_ref[:, 0]).max() <= TAU_ABS
