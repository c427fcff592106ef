"""The parity checker itself (tests/_parity.py): it must accept what a correct
bf16 kernel produces and reject each kind of fault a kernel could make.  Every
parity claim of the GPU tests rests on these functions, so here each is fed the
oracle's own result, first rounded to bf16 as a kernel's output would be
(accepted), then with one planted fault (rejected): one element off by 0.05, a
NaN, an LSE off by 2e-3, an LSE that is finite where it should be -inf (and
the reverse), a small bias on every element, a wrong shape; for the gradients
one element off by 5% of the largest, a NaN, a 2% scale error.  Non-finite
inputs are refused before anything runs.  CPU only: no kernel is involved.
"""
import numpy as np
import pytest

import attn_workloads as W
import oracle
from tests import _parity as P


def bf16_round(x):
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(x.astype(np.float32))).astype(np.float64)


@pytest.fixture(scope="module")
def fwd_ref():
    w = W.make_dense("chk", 81, 2, 300, 4, 2, 64, True)
    w.row_ptr = None
    o, l = oracle.run_workload(w)
    return o, l


@pytest.fixture(scope="module")
def fwd_ref_empty_rows():
    """A block list whose query block 1 lists only a future block: rows 128..255 have
    an empty allowed set (O = 0, LSE = -inf)."""
    w = W.make_dense("chk_e", 82, 1, 384, 2, 1, 64, True)
    w.row_ptr = np.array([0, 1, 2, 4], np.int32)
    w.col_idx = np.array([0, 2, 2, 1], np.int32)
    o, l = oracle.run_workload(w)
    assert np.all(np.isneginf(l[128:256]))
    return o, l


def test_accepts_a_bf16_rounded_result(fwd_ref, fwd_ref_empty_rows):
    for o, l in (fwd_ref, fwd_ref_empty_rows):
        P.compare(bf16_round(o), l.astype(np.float32).astype(np.float64), o, l, "rounded")


def _fails(o, l, o_ref, l_ref):
    with pytest.raises(AssertionError):
        P.compare(o, l, o_ref, l_ref, "planted")


def test_rejects_one_element_off(fwd_ref):
    o, l = fwd_ref
    bad = bf16_round(o)
    bad[123, 1, 7] += 0.05
    _fails(bad, l.copy(), o, l)


def test_rejects_nan_in_o(fwd_ref):
    o, l = fwd_ref
    bad = bf16_round(o)
    bad[5, 0, 0] = np.nan
    _fails(bad, l.copy(), o, l)


def test_rejects_lse_off(fwd_ref):
    o, l = fwd_ref
    bad = l.copy()
    bad[42, 3] += 2e-3
    _fails(bf16_round(o), bad, o, l)
    bad = l.copy()
    bad[42, 3] = np.nan
    _fails(bf16_round(o), bad, o, l)


def test_rejects_finite_where_minus_inf_and_reverse(fwd_ref_empty_rows):
    o, l = fwd_ref_empty_rows
    bad = l.copy()
    bad[130, 0] = 0.0            # an empty row given a finite LSE
    _fails(bf16_round(o), bad, o, l)
    bad = l.copy()
    bad[3, 1] = -np.inf          # a non-empty row given -inf
    _fails(bf16_round(o), bad, o, l)


def test_rejects_small_bias_everywhere(fwd_ref):
    o, l = fwd_ref
    _fails(bf16_round(o) + 3e-3, l.copy(), o, l)      # mean abs 3e-3 > 2e-3


def test_rejects_wrong_row_set(fwd_ref):
    """Rows swapped between two heads: each value is plausible, the rows are not."""
    o, l = fwd_ref
    bad = bf16_round(o)
    bad[:, [0, 1]] = bad[:, [1, 0]]
    _fails(bad, l.copy(), o, l)


def test_rejects_wrong_shape(fwd_ref):
    o, l = fwd_ref
    _fails(bf16_round(o)[:-1], l[:-1].copy(), o, l)


@pytest.fixture(scope="module")
def bwd_ref():
    w = W.make_dense("chk_b", 83, 1, 200, 4, 2, 64, True)
    do = W.make_dout(w)
    return P.oracle_bwd(w, do)


def test_grads_accept_bf16_rounded(bwd_ref):
    P.compare_grads(tuple(bf16_round(g) for g in bwd_ref), bwd_ref, "rounded")


@pytest.mark.parametrize("which", [0, 1, 2])
def test_grads_reject_planted_faults(bwd_ref, which):
    def planted(f):
        got = [bf16_round(g) for g in bwd_ref]
        got[which] = f(got[which].copy())
        with pytest.raises(AssertionError):
            P.compare_grads(tuple(got), bwd_ref, "planted")

    def one_off(g):
        g.flat[17] += 0.05 * np.abs(g).max()
        return g

    def nan(g):
        g.flat[3] = np.nan
        return g

    planted(one_off)
    planted(nan)
    planted(lambda g: g * 1.02)


def test_non_finite_inputs_are_refused():
    w = W.make_dense("chk_in", 84, 1, 64, 2, 1, 64, False)
    P.check_inputs(w)
    for name, val in (("q", np.nan), ("k", np.inf), ("v", -np.inf)):
        bad = W.make_dense("chk_in", 84, 1, 64, 2, 1, 64, False)
        arr = getattr(bad, name)
        arr.flat[10] = W.f32_to_bf16_bits(np.array([val], np.float32))[0]
        with pytest.raises(ValueError, match="non-finite"):
            P.check_inputs(bad)
        with pytest.raises(ValueError, match="non-finite"):
            P.to_device(bad)
