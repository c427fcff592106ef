"""Fused softmax attention, forward and backward, for AMD Instinct MI355X (gfx950).

The work happens in ``libattn_fwd.so`` (hand-written HIP, C ABI declared in
``include/attn_fwd.h`` and ``include/attn_bwd.h``).  This module only marshals torch tensors into the C
descriptors: every step of the computation runs in the library's kernels.
There is no fallback: if the library is missing, calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

from . import build as _build

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn_fwd.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = -1
ATTN_ERR_UNSUPPORTED = -2
ATTN_ERR_LAUNCH = -3
ATTN_ERR_TOO_LARGE = -4
ATTN_BWD_SCRATCH_BYTES = 32 << 20   # the static scratch of attn_bwd_noalloc (include/attn_bwd.h)


class AttnTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("stride_batch", ctypes.c_int64), ("stride_seq", ctypes.c_int64),
                ("stride_head", ctypes.c_int64)]


class AttnBlockList(ctypes.Structure):
    _fields_ = [("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
                ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("num_q_blocks", ctypes.c_int32)]


class AttnBlockMask(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_void_p), ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("num_q_blocks", ctypes.c_int32), ("words_per_row", ctypes.c_int32),
                ("stride_seq", ctypes.c_int64), ("stride_head", ctypes.c_int64)]


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str, what: str = "attn_fwd"):
        super().__init__(f"{what} failed: {msg} (status {status})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime; importing it first makes this library
        # bind to the same runtime instance that owns torch's memory and streams
        import torch  # noqa: F401
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m attention_forward_flashattention_amd.build`")
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        T = ctypes.POINTER(AttnTensor)
        BL = ctypes.POINTER(AttnBlockList)
        lib.attn_fwd.restype = ctypes.c_int
        lib.attn_fwd.argtypes = [T, T, T, P, ctypes.c_int, ctypes.c_float, BL, T, P, P]
        lib.attn_fwd_validate.restype = ctypes.c_int
        lib.attn_fwd_validate.argtypes = [T, T, T, P, ctypes.c_int, ctypes.c_float, BL, T]
        BM = ctypes.POINTER(AttnBlockMask)
        lib.attn_fwd_mask.restype = ctypes.c_int
        lib.attn_fwd_mask.argtypes = [T, T, T, P, ctypes.c_int, ctypes.c_float, BM, T, P, P]
        lib.attn_fwd_mask_validate.restype = ctypes.c_int
        lib.attn_fwd_mask_validate.argtypes = [T, T, T, P, ctypes.c_int, ctypes.c_float, BM, T]
        lib.attn_fwd_osk.restype = ctypes.c_int
        lib.attn_fwd_osk.argtypes = [T, T, T, ctypes.c_int, ctypes.c_float, BL, ctypes.c_float, ctypes.c_int,
                                     T, P, P, P]
        lib.attn_fwd_osk_validate.restype = ctypes.c_int
        lib.attn_fwd_osk_validate.argtypes = [T, T, T, ctypes.c_int, ctypes.c_float, BL, ctypes.c_float,
                                              ctypes.c_int, T]
        lib.attn_entmax_fwd.restype = ctypes.c_int
        lib.attn_entmax_fwd.argtypes = [T, T, T, ctypes.c_int, ctypes.c_float, ctypes.c_float, ctypes.c_int, T,
                                        P, P, ctypes.c_int, P, P]
        lib.attn_entmax_fwd_validate.restype = ctypes.c_int
        lib.attn_entmax_fwd_validate.argtypes = [T, T, T, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                                 ctypes.c_int, T, ctypes.c_int]
        lib.attn_bwd.restype = ctypes.c_int
        lib.attn_bwd.argtypes = [T, T, T, T, T, P, P, ctypes.c_int, ctypes.c_float, BM, T, T, T, P,
                                 ctypes.c_size_t, P]
        lib.attn_bwd_validate.restype = ctypes.c_int
        lib.attn_bwd_validate.argtypes = [T, T, T, T, T, P, P, ctypes.c_int, ctypes.c_float, BM, T, T,
                                          T, P, ctypes.c_size_t]
        lib.attn_bwd_noalloc.restype = ctypes.c_int
        lib.attn_bwd_noalloc.argtypes = [T, T, T, T, T, P, P, ctypes.c_int, ctypes.c_float, BM, T, T, T, P]
        lib.attn_block_list_to_mask.restype = ctypes.c_int
        lib.attn_block_list_to_mask.argtypes = [BL, ctypes.c_int, P, ctypes.c_int, P]
        lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
        lib.attn_bwd_workspace_size.argtypes = [T]
        lib.attn_status_str.restype = ctypes.c_char_p
        lib.attn_status_str.argtypes = [ctypes.c_int]
        lib.attn_version.restype = ctypes.c_int
        lib.attn_version.argtypes = []
        lib.attn_source_sha.restype = ctypes.c_char_p
        lib.attn_source_sha.argtypes = []
        built = lib.attn_source_sha().decode()
        if path == LIB_PATH and os.path.isdir(_build.CSRC):
            tree = _build.source_sha()
            if built != tree:
                raise RuntimeError(f"{path} was built from other sources (library {built}, sources here {tree}): "
                                   "rebuild it with `python -m attention_forward_flashattention_amd.build`")
        _lib = lib
    return _lib


def source_sha() -> str:
    """sha256[:16] of the sources the loaded library was built from (``attn_source_sha``)."""
    return load_library().attn_source_sha().decode()


def status_str(status: int) -> str:
    return load_library().attn_status_str(int(status)).decode()


def describe(t, batch: int, seqlen: int, packed: bool) -> AttnTensor:
    """C descriptor of a [B, S, H, D] (or packed [T, H, D]) tensor; strides in elements."""
    if packed:
        _, h, d = t.shape
        sb, ss, sh, sd = 0, t.stride(0), t.stride(1), t.stride(2)
    else:
        _, _, h, d = t.shape
        sb, ss, sh, sd = t.stride(0), t.stride(1), t.stride(2), t.stride(3)
    if sd != 1 and d > 1:
        raise ValueError("head_dim must be contiguous")
    return AttnTensor(t.data_ptr(), batch, seqlen, h, d, sb, ss, sh)


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# Shape checks.  The C layer sees only the descriptors built here (sizes taken
# from q), so every tensor the kernels index is checked against the shape
# derived from q, k and cu_seqlens before any descriptor is built: an
# undersized buffer would otherwise be read or written out of bounds.
# ---------------------------------------------------------------------------
def _shape(t):
    return tuple(int(x) for x in t.shape)


def _need_shape(name: str, t, shape) -> None:
    if _shape(t) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {_shape(t)}")


def _need(name: str, t, dtype, device: bool = True, contiguous: bool = False) -> None:
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _problem(q, k, v, cu_seqlens, max_seqlen):
    """(packed, batch, seqlen, hq, hkv, d) from q, k, v and cu_seqlens; checks that
    k and v match q in every size but heads, and each other exactly."""
    packed = cu_seqlens is not None
    if packed:
        if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
            raise ValueError("packed q, k, v must be [T, H, D]")
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must be a 1-d tensor [batch + 1]")
        if max_seqlen is None:
            raise ValueError("max_seqlen is required with cu_seqlens")
        batch, seqlen = int(cu_seqlens.numel()) - 1, int(max_seqlen)
    else:
        if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
            raise ValueError("q, k, v must be [B, S, H, D]")
        batch, seqlen = int(q.shape[0]), int(q.shape[1])
    hq, d = int(q.shape[-2]), int(q.shape[-1])
    hkv = int(k.shape[-2])
    _need_shape("k", k, _shape(q)[:-2] + (hkv, d))
    _need_shape("v", v, _shape(k))
    return packed, batch, seqlen, hq, hkv, d


def _lse_shape(packed, batch, seqlen, hq, q):
    return (hq, int(q.shape[0])) if packed else (batch, hq, seqlen)


def _check_block_mask(mask, batch: int, hkv: int, seqlen: int) -> None:
    """A bit-packed block mask [B|1, Hkv|1, n_qblk, words] covering ceil(S/128) query
    blocks of ceil(S/128) KV blocks each."""
    if mask.dim() != 4:
        raise ValueError("block_mask must be 4-d [B|1, Hkv|1, n_qblk, words]")
    n_qblk = (seqlen + 127) // 128
    b0, h0, rows, words = _shape(mask)
    if b0 not in (1, batch):
        raise ValueError(f"block_mask dim 0 must be 1 or the batch size {batch}, got {b0}")
    if h0 not in (1, hkv):
        raise ValueError(f"block_mask dim 1 must be 1 or the KV head count {hkv}, got {h0}")
    if rows < n_qblk or words < max(1, (n_qblk + 31) // 32):
        raise ValueError(f"block_mask must hold at least {n_qblk} rows of {max(1, (n_qblk + 31) // 32)} "
                         f"words, got {rows} x {words}")


def _check_block_list(block_list, seqlen: int) -> None:
    row_ptr, col_idx = block_list
    n_qblk = (seqlen + 127) // 128
    if row_ptr.dim() != 1 or int(row_ptr.numel()) != n_qblk + 1 or col_idx.dim() != 1:
        raise ValueError(f"block list row_ptr must be 1-d [{n_qblk + 1}] and col_idx 1-d")


def block_mask_descriptor(mask) -> AttnBlockMask:
    """C descriptor of a bit-packed block mask tensor.

    mask: int32 or uint32 device tensor [B or 1, Hkv or 1, num_q_blocks, words]; a
    size-1 leading dimension is shared by every sequence / KV head.  Bit kb % 32
    of word kb // 32 of row qb: KV block kb visible to query block qb.
    """
    import torch

    if mask.dim() != 4 or not mask.is_cuda or mask.dtype not in (torch.int32, torch.uint32):
        raise ValueError("block_mask must be a 4-d int32/uint32 device tensor [B|1, Hkv|1, n_qblk, words]")
    if mask.stride(3) != 1 or mask.stride(2) != mask.shape[3]:
        raise ValueError("block_mask rows must be contiguous")
    ss = mask.stride(0) if mask.shape[0] > 1 else 0
    sh = mask.stride(1) if mask.shape[1] > 1 else 0
    return AttnBlockMask(mask.data_ptr(), 128, 128, int(mask.shape[2]), int(mask.shape[3]), ss, sh)


def _list_descriptor(block_list) -> AttnBlockList:
    import torch

    row_ptr, col_idx = block_list
    for t in (row_ptr, col_idx):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("block list tensors must be contiguous int32 device tensors")
    return AttnBlockList(row_ptr.data_ptr(), col_idx.data_ptr() if col_idx.numel() else row_ptr.data_ptr(),
                         128, 128, int(row_ptr.numel()) - 1)


def attn_fwd(q, k, v, cu_seqlens=None, causal: bool = False, scale: Optional[float] = None,
             block_list: Optional[Tuple] = None, out=None, lse=None, max_seqlen: Optional[int] = None,
             return_lse: bool = True, stream=None, block_mask=None):
    """O = softmax(scale * Q K^T + mask) V and the natural-log LSE per row.

    q: bf16 [B, S, Hq, D] (or packed [T, Hq, D] with ``cu_seqlens`` int32 [B+1])
    k, v: bf16 [B, S, Hkv, D] (or packed [T, Hkv, D])
    block_list: optional (row_ptr, col_idx) int32 device tensors, 128x128 blocks
    block_mask: optional bit-packed block mask (see ``block_mask_descriptor``);
        not together with ``block_list``
    out: optional bf16 output shaped like q;  lse: optional fp32 [B, Hq, S] (packed [Hq, T])
    max_seqlen: packed form only, an upper bound on every sequence length (the
        kernel trusts it and the contents of cu_seqlens, which live on the device)
    Returns (out, lse) (lse None when ``return_lse`` is false and none is given).
    """
    import torch

    if block_list is not None and block_mask is not None:
        raise ValueError("give a block list or a block mask, not both")
    lib = load_library()
    packed, batch, seqlen, hq, hkv, d = _problem(q, k, v, cu_seqlens, max_seqlen)
    if out is not None:
        _need_shape("out", out, _shape(q))
        _need("out", out, torch.bfloat16)
    if lse is not None:
        _need_shape("lse", lse, _lse_shape(packed, batch, seqlen, hq, q))
        _need("lse", lse, torch.float32, contiguous=True)
    if block_mask is not None:
        _check_block_mask(block_mask, batch, hkv, seqlen)
    if block_list is not None:
        _check_block_list(block_list, seqlen)
    if packed:
        _need("cu_seqlens", cu_seqlens, torch.int32, contiguous=True)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(name, t, torch.bfloat16)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty(_lse_shape(packed, batch, seqlen, hq, q), dtype=torch.float32, device=q.device)
    dq = describe(q, batch, seqlen, packed)
    dk = describe(k, batch, seqlen, packed)
    dv = describe(v, batch, seqlen, packed)
    do = describe(out, batch, seqlen, packed)
    bl = _list_descriptor(block_list) if block_list is not None else None
    cu_p = ctypes.c_void_p(cu_seqlens.data_ptr()) if packed else None
    lse_p = ctypes.c_void_p(lse.data_ptr()) if lse is not None else None
    if block_mask is not None:
        bm = block_mask_descriptor(block_mask)
        st = lib.attn_fwd_mask(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), cu_p,
                               int(bool(causal)), float(scale), ctypes.byref(bm), ctypes.byref(do),
                               lse_p, ctypes.c_void_p(_stream_handle(stream)))
    else:
        st = lib.attn_fwd(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), cu_p,
                          int(bool(causal)), float(scale), ctypes.byref(bl) if bl is not None else None,
                          ctypes.byref(do), lse_p, ctypes.c_void_p(_stream_handle(stream)))
    if st != ATTN_OK:
        raise AttnError(st, status_str(st))
    return out, lse


def attn_fwd_osk(q, k, v, block_list: Tuple, tau: float, min_visit: int = 2, causal: bool = True,
                 scale: Optional[float] = None, out=None, lse=None, visited=None, stream=None):
    """Block-list forward with ordered skipping (the stopping rule of
    ``attn_fwd_osk`` in include/attn_fwd.h): each (query head, query block)
    walks its list in order and stops once (entries left) x the newest entry's
    mass is at most ``tau`` of every row's mass, after ``min_visit`` entries.

    q: bf16 [1, S, Hq, D]; k, v: bf16 [1, S, Hkv, D]; block_list: (row_ptr, col_idx)
    Returns (out, lse, visited) with visited int32 [Hq, num_q_blocks].
    """
    import torch

    lib = load_library()
    _, batch, seqlen, hq, _, d = _problem(q, k, v, None, None)
    _check_block_list(block_list, seqlen)
    n_qblk = (seqlen + 127) // 128
    if out is not None:
        _need_shape("out", out, _shape(q))
        _need("out", out, torch.bfloat16)
    if lse is not None:
        _need_shape("lse", lse, (batch, hq, seqlen))
        _need("lse", lse, torch.float32, contiguous=True)
    if visited is not None:
        _need_shape("visited", visited, (hq, n_qblk))
        _need("visited", visited, torch.int32, contiguous=True)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(name, t, torch.bfloat16)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    if lse is None:
        lse = torch.empty((batch, hq, seqlen), dtype=torch.float32, device=q.device)
    if visited is None:
        visited = torch.empty((hq, n_qblk), dtype=torch.int32, device=q.device)
    bl = _list_descriptor(block_list)
    dq, dk, dv, do = (describe(t, batch, seqlen, False) for t in (q, k, v, out))
    st = lib.attn_fwd_osk(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), int(bool(causal)), float(scale),
                          ctypes.byref(bl), float(tau), int(min_visit), ctypes.byref(do),
                          ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(visited.data_ptr()),
                          ctypes.c_void_p(_stream_handle(stream)))
    if st != ATTN_OK:
        raise AttnError(st, status_str(st), "attn_fwd_osk")
    return out, lse, visited


def attn_entmax_fwd(q, k, v, alpha: float, causal: bool = False, scale: Optional[float] = None,
                    n_iter: int = 16, out=None, return_mask: bool = False, return_tau_init: bool = False,
                    stream=None):
    """alpha-entmax attention forward (``attn_entmax_fwd`` in include/attn_fwd.h).

    q: bf16 [B, S, Hq, D]; k, v: bf16 [B, S, Hkv, D]
    Returns (out, tau) plus the block mask int32 [B, Hq, n_qblk, words] with
    ``return_mask`` and the histogram bound [B, Hq, S] with ``return_tau_init``.
    """
    import torch

    lib = load_library()
    _, batch, seqlen, hq, _, d = _problem(q, k, v, None, None)
    if out is not None:
        _need_shape("out", out, _shape(q))
        _need("out", out, torch.bfloat16)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(name, t, torch.bfloat16)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    tau = torch.empty((batch, hq, seqlen), dtype=torch.float32, device=q.device)
    n_qblk = (seqlen + 127) // 128
    words = max(1, (n_qblk + 31) // 32)
    mask = torch.zeros((batch, hq, n_qblk, words), dtype=torch.int32, device=q.device) if return_mask else None
    tau0 = torch.empty_like(tau) if return_tau_init else None
    dq, dk, dv, do = (describe(t, batch, seqlen, False) for t in (q, k, v, out))
    st = lib.attn_entmax_fwd(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), int(bool(causal)),
                             float(scale), float(alpha), int(n_iter), ctypes.byref(do),
                             ctypes.c_void_p(tau.data_ptr()),
                             ctypes.c_void_p(mask.data_ptr()) if mask is not None else None, words,
                             ctypes.c_void_p(tau0.data_ptr()) if tau0 is not None else None,
                             ctypes.c_void_p(_stream_handle(stream)))
    if st != ATTN_OK:
        raise AttnError(st, status_str(st), "attn_entmax_fwd")
    res = (out, tau)
    if return_mask:
        res += (mask,)
    if return_tau_init:
        res += (tau0,)
    return res


def _bwd_prepare(q, k, v, out, dout, lse, cu_seqlens, max_seqlen, block_mask, dq, dk, dv, scale):
    """Shape and dtype checks of the backward's tensors; returns the descriptors, the
    problem sizes and the (possibly allocated) gradient tensors."""
    import torch

    packed, batch, seqlen, hq, hkv, d = _problem(q, k, v, cu_seqlens, max_seqlen)
    _need_shape("out", out, _shape(q))
    _need_shape("dout", dout, _shape(q))
    _need_shape("lse", lse, _lse_shape(packed, batch, seqlen, hq, q))
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is not None:
            _need_shape(name, t, _shape(like))
    if block_mask is not None:
        _check_block_mask(block_mask, batch, hkv, seqlen)
    if packed:
        _need("cu_seqlens", cu_seqlens, torch.int32, contiguous=True)
    _need("lse", lse, torch.float32, contiguous=True)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        if t is not None:
            _need(name, t, torch.bfloat16)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    descs = [describe(t, batch, seqlen, packed) for t in (q, k, v, out, dout, dq, dk, dv)]
    bm = block_mask_descriptor(block_mask) if block_mask is not None else None
    cu_p = ctypes.c_void_p(cu_seqlens.data_ptr()) if packed else None
    return descs, bm, cu_p, float(scale), (dq, dk, dv)


def block_list_to_mask(block_list: Tuple, seqlen: int, stream=None):
    """The bit-packed block mask of a block list's set (``attn_block_list_to_mask``):
    int32 [1, 1, ceil(S/128), words], one sequence's mask shared by every KV head, the
    form ``attn_bwd``'s ``block_mask`` takes for the backward of a forward that took
    the list (ids outside the sequence are dropped, as the forward skips them)."""
    import torch

    lib = load_library()
    _check_block_list(block_list, seqlen)
    n_blk = (seqlen + 127) // 128
    words = max(1, (n_blk + 31) // 32)
    mask = torch.empty((1, 1, n_blk, words), dtype=torch.int32, device=block_list[0].device)
    st = lib.attn_block_list_to_mask(ctypes.byref(_list_descriptor(block_list)), n_blk,
                                     ctypes.c_void_p(mask.data_ptr()), words, ctypes.c_void_p(_stream_handle(stream)))
    if st != ATTN_OK:
        raise AttnError(st, status_str(st), "attn_block_list_to_mask")
    return mask


def attn_bwd(q, k, v, out, dout, lse, cu_seqlens=None, causal: bool = False,
             scale: Optional[float] = None, max_seqlen: Optional[int] = None, block_mask=None,
             dq=None, dk=None, dv=None, workspace=None, stream=None, block_list: Optional[Tuple] = None):
    """Gradients (dq, dk, dv) of sum(out * dout) for out, lse = attn_fwd(q, k, v, ...).

    q, out, dout: bf16 [B, S, Hq, D] (packed [T, Hq, D] with ``cu_seqlens``)
    k, v: bf16 [B, S, Hkv, D] (packed [T, Hkv, D]);  lse: the forward's fp32 LSE
    causal, scale, max_seqlen, block_mask: as for ``attn_fwd`` (the same values)
    block_list: the forward's block list instead of a mask (batch 1, no cu_seqlens):
        the backward runs on the mask of its set (``block_list_to_mask``)
    dq, dk, dv: optional bf16 outputs shaped like q, k, v
    workspace: optional device buffer of at least ``attn_bwd_workspace_size`` bytes
    """
    import torch

    lib = load_library()
    if block_list is not None:
        if block_mask is not None:
            raise ValueError("give a block list or a block mask, not both")
        if cu_seqlens is not None or q.dim() != 4 or q.shape[0] != 1:
            raise ValueError("a block list goes with one fixed-length sequence (batch 1, no cu_seqlens)")
        block_mask = block_list_to_mask(block_list, int(q.shape[1]), stream)
    descs, bm, cu_p, scale, grads = _bwd_prepare(q, k, v, out, dout, lse, cu_seqlens, max_seqlen, block_mask,
                                                 dq, dk, dv, scale)
    need = int(lib.attn_bwd_workspace_size(ctypes.byref(descs[0])))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.attn_bwd(*(ctypes.byref(d) for d in descs[:5]), ctypes.c_void_p(lse.data_ptr()), cu_p,
                      int(bool(causal)), scale, ctypes.byref(bm) if bm is not None else None,
                      *(ctypes.byref(d) for d in descs[5:]), ctypes.c_void_p(workspace.data_ptr()),
                      ws_bytes, ctypes.c_void_p(_stream_handle(stream)))
    if st != ATTN_OK:
        raise AttnError(st, status_str(st), "attn_bwd")
    return grads


def attn_bwd_noalloc(q, k, v, out, dout, lse, dq, dk, dv, cu_seqlens=None, causal: bool = False,
                     scale: Optional[float] = None, max_seqlen: Optional[int] = None, block_mask=None,
                     stream=None):
    """``attn_bwd`` without a workspace: the library's static per-device scratch holds
    the per-row values instead, so neither this call nor the library allocates (the
    caller passes dq, dk, dv).  Problems needing more than ``ATTN_BWD_SCRATCH_BYTES`` of
    workspace raise ``AttnError`` with status ``ATTN_ERR_TOO_LARGE``; calls that overlap
    on one GPU race on the shared scratch."""
    lib = load_library()
    if dq is None or dk is None or dv is None:
        raise ValueError("attn_bwd_noalloc writes into caller-provided dq, dk, dv")
    descs, bm, cu_p, scale, grads = _bwd_prepare(q, k, v, out, dout, lse, cu_seqlens, max_seqlen, block_mask,
                                                 dq, dk, dv, scale)
    st = lib.attn_bwd_noalloc(*(ctypes.byref(d) for d in descs[:5]), ctypes.c_void_p(lse.data_ptr()), cu_p,
                              int(bool(causal)), scale, ctypes.byref(bm) if bm is not None else None,
                              *(ctypes.byref(d) for d in descs[5:]), ctypes.c_void_p(_stream_handle(stream)))
    if st != ATTN_OK:
        raise AttnError(st, status_str(st), "attn_bwd_noalloc")
    return grads
