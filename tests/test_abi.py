"""The C-ABI library: loads, exports what include/*.h declare, and
rejects bad arguments with the documented status codes (host-only checks; no
kernel is launched, so these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import attention_forward_flashattention_amd as attn
from attention_forward_flashattention_amd import AttnBlockList, AttnBlockMask, AttnTensor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def declared_functions():
    names = set()
    for f in sorted(os.listdir(INCLUDE)):
        if f.endswith(".h"):
            text = open(os.path.join(INCLUDE, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_entry_points():
    assert declared_functions() == ["attn_block_list_to_mask", "attn_bwd", "attn_bwd_noalloc", "attn_bwd_validate",
                                    "attn_bwd_workspace_size", "attn_entmax_fwd", "attn_entmax_fwd_validate",
                                    "attn_fwd", "attn_fwd_mask", "attn_fwd_mask_validate", "attn_fwd_osk",
                                    "attn_fwd_osk_validate", "attn_fwd_validate", "attn_source_sha",
                                    "attn_status_str", "attn_version"]


def test_library_exports_every_declared_symbol():
    lib = attn.load_library()
    out = subprocess.run(["nm", "-D", "--defined-only", attn.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert lib.attn_version() == 301
    assert attn.status_str(0) == "ok" and attn.status_str(-3) == "kernel launch failed"


def test_library_was_built_from_these_sources():
    """The library carries the hash of the sources it was compiled from; it must be
    the hash of the sources in this tree (load_library refuses a stale library)."""
    from attention_forward_flashattention_amd import build

    assert attn.source_sha() == build.source_sha()
    assert len(attn.source_sha()) == 16 and attn.source_sha() != "unknown"


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation only reads the descriptors


def desc(b=2, s=256, h=8, d=128, data=FAKE, layout="bshd"):
    if layout == "bshd":
        return AttnTensor(data, b, s, h, d, s * h * d, h * d, d)
    return AttnTensor(data, b, s, h, d, h * s * d, d, s * d)


def validate(q, k, v, cu=None, causal=1, scale=0.125, bl=None, out=None):
    lib = attn.load_library()
    out = out if out is not None else q
    return lib.attn_fwd_validate(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), cu, causal, scale,
                                 ctypes.byref(bl) if bl is not None else None, ctypes.byref(out))


def test_valid_arguments_pass():
    assert validate(desc(), desc(h=2), desc(h=2)) == 0
    k, v = desc(h=2), desc(h=2)
    k.stride_seq = v.stride_seq = (1 << 24) - 8  # the largest K/V row stride accepted
    assert validate(desc(), k, v) == 0
    assert validate(desc(layout="bhsd"), desc(h=8, layout="bhsd"), desc(h=8, layout="bhsd")) == 0
    for d in (64, 128, 256):
        assert validate(desc(d=d), desc(d=d, h=4), desc(d=d, h=4)) == 0


@pytest.mark.parametrize("mut,code", [
    (lambda q, k, v: setattr(k, "heads", 3), -1),             # Hq % Hkv != 0
    (lambda q, k, v: setattr(v, "heads", 4), -1),             # k/v head mismatch
    (lambda q, k, v: setattr(k, "seqlen", 255), -1),          # seqlen mismatch
    (lambda q, k, v: setattr(v, "batch", 1), -1),             # batch mismatch
    (lambda q, k, v: setattr(k, "head_dim", 64), -1),         # head_dim mismatch
    (lambda q, k, v: setattr(q, "data", None), -1),           # null data
    (lambda q, k, v: [setattr(t, "head_dim", 96) for t in (q, k, v)], -2),  # unsupported D (out too)
    (lambda q, k, v: setattr(q, "data", FAKE + 8), -2),       # misaligned pointer
    (lambda q, k, v: setattr(k, "stride_seq", 2 * 128 + 4), -2),  # stride*2 not multiple of 16
    (lambda q, k, v: setattr(k, "stride_seq", 1 << 24), -2),   # K rows too far apart for 32-bit offsets
    (lambda q, k, v: setattr(v, "stride_seq", -256), -2),      # negative V row stride
    (lambda q, k, v: setattr(q, "batch", -1), -1),
])
def test_invalid_arguments(mut, code):
    q, k, v = desc(), desc(h=2), desc(h=2)
    o = desc()
    mut(q, k, v)
    o.head_dim = q.head_dim if q.head_dim == 96 else o.head_dim
    assert validate(q, k, v, out=o) == code


def test_scalar_arguments():
    q, k, v = desc(), desc(h=2), desc(h=2)
    assert validate(q, k, v, causal=2) == -1
    assert validate(q, k, v, scale=float("nan")) == -1
    assert validate(q, k, v, scale=float("inf")) == -1
    assert validate(q, k, v, scale=0.0) == -2
    assert validate(q, k, v, scale=-0.5) == -2
    assert validate(q, k, v, out=desc(h=4)) == -1  # out heads != Hq


def test_block_list_arguments():
    q, k, v = desc(b=1, s=1000), desc(b=1, s=1000, h=2), desc(b=1, s=1000, h=2)
    ok = AttnBlockList(FAKE, FAKE, 128, 128, 8)
    assert validate(q, k, v, bl=ok) == 0
    assert validate(q, k, v, bl=AttnBlockList(FAKE, FAKE, 64, 128, 8)) == -2
    assert validate(q, k, v, bl=AttnBlockList(FAKE, FAKE, 128, 128, 7)) == -1
    assert validate(q, k, v, bl=AttnBlockList(None, FAKE, 128, 128, 8)) == -1
    q2, k2, v2 = desc(b=2, s=1000), desc(b=2, s=1000, h=2), desc(b=2, s=1000, h=2)
    assert validate(q2, k2, v2, bl=ok) == -2          # batch > 1 with a list
    assert validate(q, k, v, cu=ctypes.c_void_p(FAKE), bl=ok) == -2   # packed with a list


def test_empty_problem_is_ok_without_data():
    q, k, v = desc(b=0, data=None), desc(b=0, h=2, data=None), desc(b=0, h=2, data=None)
    assert validate(q, k, v, out=desc(b=0, data=None)) == 0


def test_attn_fwd_returns_validation_errors_without_launching():
    lib = attn.load_library()
    q, k, v = desc(), desc(h=3), desc(h=3)
    st = lib.attn_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), None, 1, 0.1, None,
                      ctypes.byref(desc()), None, None)
    assert st == -1
    # an empty problem returns OK and launches nothing
    e = desc(b=0, data=None)
    st = lib.attn_fwd(ctypes.byref(e), ctypes.byref(e), ctypes.byref(e), None, 1, 0.1, None,
                      ctypes.byref(e), None, None)
    assert st == 0


def validate_mask(q, k, v, mask, cu=None, causal=1, scale=0.125, out=None):
    lib = attn.load_library()
    out = out if out is not None else q
    return lib.attn_fwd_mask_validate(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), cu, causal, scale,
                                      ctypes.byref(mask) if mask is not None else None, ctypes.byref(out))


def mask_desc(n_qblk=2, words=1, ss=0, sh=0, bq=128, bk=128, bits=FAKE):
    return AttnBlockMask(bits, bq, bk, n_qblk, words, ss, sh)


def test_block_mask_validation():
    q, k, v = desc(b=2, s=256), desc(b=2, s=256, h=2), desc(b=2, s=256, h=2)
    assert validate_mask(q, k, v, mask_desc()) == 0
    assert validate_mask(q, k, v, mask_desc(ss=4, sh=2)) == 0           # per sequence and head
    assert validate_mask(q, k, v, None) == -1                          # no descriptor
    assert validate_mask(q, k, v, mask_desc(bits=None)) == -1          # no bits
    assert validate_mask(q, k, v, mask_desc(n_qblk=1)) == -1           # fewer rows than query blocks
    assert validate_mask(q, k, v, mask_desc(words=0)) == -1
    assert validate_mask(q, k, v, mask_desc(ss=-1)) == -1
    assert validate_mask(q, k, v, mask_desc(bq=64)) == -2              # block size other than 128
    # 33 blocks need 2 words per row
    q2, k2, v2 = desc(b=1, s=33 * 128), desc(b=1, s=33 * 128, h=2), desc(b=1, s=33 * 128, h=2)
    assert validate_mask(q2, k2, v2, mask_desc(n_qblk=33, words=1)) == -1
    assert validate_mask(q2, k2, v2, mask_desc(n_qblk=33, words=2)) == 0
    # shared checks still apply
    k.heads = 3
    assert validate_mask(q, k, v, mask_desc()) == -1


# ---------------------------------------------------------------------------
# attn_bwd argument checks (host only)
# ---------------------------------------------------------------------------
def bwd_validate(q, k, v, out=None, dout=None, dq=None, dk=None, dv=None, lse=FAKE, ws=FAKE,
                 ws_bytes=None, mask=None, causal=1, scale=0.125, cu=None):
    lib = attn.load_library()
    out = out if out is not None else q
    dout = dout if dout is not None else q
    dq = dq if dq is not None else q
    dk = dk if dk is not None else k
    dv = dv if dv is not None else v
    if ws_bytes is None:
        ws_bytes = lib.attn_bwd_workspace_size(ctypes.byref(q))
    r = lambda t: ctypes.byref(t)
    return lib.attn_bwd_validate(r(q), r(k), r(v), r(out), r(dout), lse, cu, causal, scale,
                                 r(mask) if mask is not None else None, r(dq), r(dk), r(dv), ws, ws_bytes)


def test_bwd_workspace_size():
    lib = attn.load_library()
    assert lib.attn_bwd_workspace_size(ctypes.byref(desc(b=2, s=256, h=8))) == 2 * 4 * 2 * 256 * 8
    assert lib.attn_bwd_workspace_size(ctypes.byref(desc(b=0))) == 0
    assert lib.attn_bwd_workspace_size(None) == 0


def test_bwd_valid_arguments_pass():
    assert bwd_validate(desc(), desc(h=2), desc(h=2)) == 0
    assert bwd_validate(desc(d=64), desc(h=8, d=64), desc(h=8, d=64), causal=0) == 0
    m = AttnBlockMask(FAKE, 128, 128, 2, 1, 2, 0)
    assert bwd_validate(desc(), desc(h=2), desc(h=2), mask=m) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(lse=None), -1),                                   # no LSE
    (dict(ws=None), -1),                                    # no workspace
    (dict(ws_bytes=1024), -1),                              # workspace too small
    (dict(dq=desc(h=4)), -1),                               # dq heads differ from q
    (dict(dk=desc(h=4), dv=desc(h=4)), -1),                 # dk/dv heads differ from k
    (dict(dout=desc(s=128)), -1),                           # dout seqlen differs
    (dict(dv=desc(h=2, d=64)), -1),                         # dv head_dim differs
    (dict(ws=FAKE + 4), -2),                                # misaligned workspace
    (dict(causal=2), -1),
    (dict(mask=AttnBlockMask(FAKE, 64, 128, 2, 1, 0, 0)), -2),  # block size 64
])
def test_bwd_invalid_arguments(kw, code):
    assert bwd_validate(desc(), desc(h=2), desc(h=2), **kw) == code


def test_bwd_head_dims_and_long_masked_sequences():
    for d in (64, 128, 256):
        assert bwd_validate(desc(d=d), desc(h=2, d=d), desc(h=2, d=d)) == 0
    assert bwd_validate(desc(d=96), desc(h=2, d=96), desc(h=2, d=96)) == -2
    s = 128 * 16385  # more query blocks than the key kernel's column bitmap holds
    q, kv = desc(b=1, s=s, h=1), desc(b=1, s=s, h=1)
    m = AttnBlockMask(FAKE, 128, 128, 16385, 513, 0, 0)
    assert bwd_validate(q, kv, desc(b=1, s=s, h=1), mask=m) == -2
    m2 = AttnBlockMask(FAKE, 128, 128, 16384, 512, 0, 0)
    s2 = 128 * 16384
    assert bwd_validate(desc(b=1, s=s2, h=1), desc(b=1, s=s2, h=1), desc(b=1, s=s2, h=1), mask=m2) == 0


def test_bwd_query_row_stride_limit():
    """The dK/dV kernel addresses a Q or dO tile's rows with 32-bit byte offsets, as every
    kernel does for K and V: their row strides are limited the same way."""
    q = desc()
    q.stride_seq = (1 << 24) - 8  # the largest accepted
    assert bwd_validate(q, desc(h=2), desc(h=2), out=desc(), dq=desc()) == 0
    q.stride_seq = 1 << 24
    assert bwd_validate(q, desc(h=2), desc(h=2), out=desc(), dq=desc()) == -2
    g = desc()
    g.stride_seq = 1 << 24
    assert bwd_validate(desc(), desc(h=2), desc(h=2), dout=g) == -2


def test_bwd_empty_problem_needs_no_buffers():
    q, k = desc(b=0), desc(b=0, h=2)
    assert bwd_validate(q, k, desc(b=0, h=2), lse=None, ws=None, ws_bytes=0) == 0


# ---------------------------------------------------------------------------
# attn_fwd_osk argument checks (host only)
# ---------------------------------------------------------------------------
def osk_validate(q, k, v, bl, tau=0.01, min_visit=2, causal=1, scale=0.125):
    lib = attn.load_library()
    return lib.attn_fwd_osk_validate(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), causal, scale,
                                     ctypes.byref(bl) if bl is not None else None, tau, min_visit,
                                     ctypes.byref(q))


def test_osk_argument_checks():
    q, kv = desc(b=1, s=256, h=4), desc(b=1, s=256, h=2)
    bl = AttnBlockList(FAKE, FAKE, 128, 128, 2)
    assert osk_validate(q, kv, kv, bl) == 0
    assert osk_validate(q, kv, kv, bl, tau=0.0, min_visit=1) == 0
    assert osk_validate(q, kv, kv, None) == -1                      # the list is required
    assert osk_validate(q, kv, kv, bl, tau=-0.1) == -1
    assert osk_validate(q, kv, kv, bl, tau=float("inf")) == -1
    assert osk_validate(q, kv, kv, bl, tau=float("nan")) == -1
    assert osk_validate(q, kv, kv, bl, min_visit=0) == -1
    assert osk_validate(desc(b=2, s=256, h=4), desc(b=2, s=256, h=2), desc(b=2, s=256, h=2), bl) == -2  # batch > 1
    assert osk_validate(q, kv, kv, AttnBlockList(FAKE, FAKE, 64, 128, 4)) == -2                          # block size


# ---------------------------------------------------------------------------
# attn_entmax_fwd argument checks (host only)
# ---------------------------------------------------------------------------
def test_entmax_argument_checks():
    lib = attn.load_library()
    q, kv = desc(b=2, s=256, h=4), desc(b=2, s=256, h=2)

    def val(alpha=1.5, n_iter=2, words=0, qd=q, kd=kv):
        return lib.attn_entmax_fwd_validate(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(kd), 1, 0.125,
                                            alpha, n_iter, ctypes.byref(qd), words)
    assert val() == 0 and val(alpha=2.0, words=1) == 0 and val(alpha=3.0, n_iter=32) == 0
    assert val(alpha=1.0) == -1 and val(alpha=float("nan")) == -1 and val(alpha=float("inf")) == -1
    assert val(n_iter=0) == -1 and val(n_iter=33) == -1
    assert val(alpha=1.01) == -2 and val(alpha=3.5) == -2
    assert val(qd=desc(b=2, s=256, h=4, d=256), kd=desc(b=2, s=256, h=2, d=256)) == 0
    assert val(qd=desc(b=2, s=256, h=4, d=96), kd=desc(b=2, s=256, h=2, d=96)) == -2
    s = 128 * 33                                        # 33 blocks need 2 mask words
    assert val(words=1, qd=desc(b=1, s=s, h=4), kd=desc(b=1, s=s, h=2)) == -1
    assert val(words=2, qd=desc(b=1, s=s, h=4), kd=desc(b=1, s=s, h=2)) == 0


# ---------------------------------------------------------------------------
# attn_block_list_to_mask argument checks (host only: every call here fails
# its checks, or has no query block, before any launch)
# ---------------------------------------------------------------------------
def test_block_list_to_mask_argument_checks():
    lib = attn.load_library()

    def conv(bl, n_kv=4, words=1, mask=FAKE):
        return lib.attn_block_list_to_mask(ctypes.byref(bl) if bl is not None else None, n_kv, mask, words, None)
    assert conv(AttnBlockList(FAKE, FAKE, 128, 128, 0)) == 0                    # no query block: nothing to do
    assert conv(None) == -1
    assert conv(AttnBlockList(FAKE, FAKE, 128, 128, -1)) == -1
    assert conv(AttnBlockList(FAKE, FAKE, 128, 128, 3), n_kv=-1) == -1
    assert conv(AttnBlockList(FAKE, FAKE, 64, 128, 3)) == -2                    # block size
    assert conv(AttnBlockList(FAKE, FAKE, 128, 128, 3), n_kv=16385, words=513) == -2
    assert conv(AttnBlockList(FAKE, FAKE, 128, 128, 3), n_kv=33, words=1) == -1  # 33 blocks need 2 words
    assert conv(AttnBlockList(FAKE, FAKE, 128, 128, 3), n_kv=4, words=513) == -1
    assert conv(AttnBlockList(None, FAKE, 128, 128, 3)) == -1
    assert conv(AttnBlockList(FAKE, FAKE, 128, 128, 3), mask=None) == -1


# ---------------------------------------------------------------------------
# Binding shape checks: every tensor the kernels index is checked against the
# shape derived from q, k and cu_seqlens before any descriptor reaches the C
# layer (host tensors suffice: the shape checks come before the device checks).
# ---------------------------------------------------------------------------
def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def test_binding_rejects_mismatched_kv():
    q = _t(2, 64, 4, 64)
    with pytest.raises(ValueError, match="k must have shape"):
        attn.attn_fwd(q, _t(2, 32, 2, 64), _t(2, 32, 2, 64))          # k shorter than q
    with pytest.raises(ValueError, match="v must have shape"):
        attn.attn_fwd(q, _t(2, 64, 2, 64), _t(2, 64, 1, 64))          # v heads differ from k
    with pytest.raises(ValueError, match="k must have shape"):
        attn.attn_fwd(_t(100, 4, 64), _t(90, 2, 64), _t(90, 2, 64), cu_seqlens=_t(3, dtype=None), max_seqlen=64)


def test_binding_rejects_undersized_outputs():
    import torch
    q, k = _t(2, 64, 4, 64), _t(2, 64, 2, 64)
    with pytest.raises(ValueError, match="out must have shape"):
        attn.attn_fwd(q, k, k, out=_t(2, 64, 2, 64))
    with pytest.raises(ValueError, match="lse must have shape"):
        attn.attn_fwd(q, k, k, lse=torch.zeros((2, 4, 63)))
    with pytest.raises(ValueError, match="lse must have shape"):
        attn.attn_fwd(_t(100, 4, 64), _t(100, 2, 64), _t(100, 2, 64), cu_seqlens=torch.zeros(3, dtype=torch.int32),
                      max_seqlen=64, lse=torch.zeros((4, 99)))
    with pytest.raises(ValueError, match="visited must have shape"):
        attn.attn_fwd_osk(_t(1, 256, 4, 64), _t(1, 256, 2, 64), _t(1, 256, 2, 64),
                          (torch.zeros(3, dtype=torch.int32), torch.zeros(4, dtype=torch.int32)), 0.1,
                          visited=torch.zeros((4, 1), dtype=torch.int32))
    with pytest.raises(ValueError, match="row_ptr"):
        attn.attn_fwd(_t(1, 256, 4, 64), _t(1, 256, 2, 64), _t(1, 256, 2, 64),
                      block_list=(torch.zeros(2, dtype=torch.int32), torch.zeros(4, dtype=torch.int32)))


def test_binding_rejects_bad_block_masks():
    import torch
    q, k = _t(2, 300, 4, 64), _t(2, 300, 2, 64)
    ok = torch.zeros((1, 2, 3, 1), dtype=torch.int32)
    for bad, what in ((torch.zeros((3, 1, 3, 1), dtype=torch.int32), "dim 0"),
                      (torch.zeros((1, 4, 3, 1), dtype=torch.int32), "dim 1"),
                      (torch.zeros((1, 1, 2, 1), dtype=torch.int32), "rows"),
                      (torch.zeros((2, 2, 3), dtype=torch.int32), "4-d")):
        with pytest.raises(ValueError, match=what):
            attn.attn_fwd(q, k, k, causal=True, block_mask=bad)
    with pytest.raises(ValueError, match="device"):      # a valid shape reaches the device check
        attn.attn_fwd(q, k, k, causal=True, block_mask=ok)


def test_binding_rejects_bad_backward_tensors():
    import torch
    q, k = _t(2, 64, 4, 64), _t(2, 64, 2, 64)
    lse = torch.zeros((2, 4, 64))
    with pytest.raises(ValueError, match="dout must have shape"):
        attn.attn_bwd(q, k, k, q, _t(2, 64, 4, 32), lse)
    with pytest.raises(ValueError, match="lse must have shape"):
        attn.attn_bwd(q, k, k, q, q, torch.zeros((2, 4, 32)))
    with pytest.raises(ValueError, match="dk must have shape"):
        attn.attn_bwd(q, k, k, q, q, lse, dk=_t(2, 64, 4, 64))
    with pytest.raises(ValueError, match="dq must have shape"):
        attn.attn_bwd(q, k, k, q, q, lse, dq=_t(2, 32, 4, 64))
