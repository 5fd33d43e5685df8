"""Exact attention (FlashAttention forward and split backward) on MI355X.

A thin Python binding over the C ABI of ``libfa.so`` (``include/fa.h``).
Every step of the computation runs in the library's gfx950 HIP kernels; this
module only checks tensors, allocates outputs with torch on the inputs'
device and passes raw device pointers and the current torch stream.  There
is no CPU or PyTorch fallback: if the library is missing, calls raise.

Layout: q, k, v, o, dO, dq, dk, dv are [B, H, N, D] contiguous; lse and
delta are float32 [B, H, N].  ``fwd_kv`` takes q [B, H, Nq, D] and k, v
[B, H, Nk, D].
"""

from __future__ import annotations

import math

from . import _lib
from ._lib import FAError  # noqa: F401

__all__ = ["fwd", "fwd_kv", "fwd_kv_noalloc", "kv_splits", "fwd_sparse", "SPARSE_BLOCK", "bwd_dq", "bwd_dkdv", "bwd", "FAError", "library_path", "version"]


def library_path() -> str:
    return _lib.load()._name


def version() -> int:
    return _lib.load().fa_version()


def _torch():
    import torch

    return torch


def _check_bhnd(name, t, dtype, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, D], got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_rows(name, t, shape):
    torch = _torch()
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()):
        raise TypeError(f"{name} must be a contiguous float32 GPU tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream_ptr(t, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes_void(stream.cuda_stream)


def ctypes_void(x):
    import ctypes

    return ctypes.c_void_p(x)


def _ptr(t):
    import ctypes

    return ctypes.c_void_p(t.data_ptr())


def fwd(q, k, v, scale: float | None = None, causal: bool = False, out=None, lse=None, stream=None):
    """O = softmax(scale q k^T) v and L = logsumexp rows, on the GPU.

    bf16 inputs run ``fa_fwd`` (bf16 output), float32 inputs ``fa_fwd_f32``.
    Returns (o, lse).  ``scale`` defaults to 1/sqrt(D).
    """
    torch = _torch()
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bfloat16 or float32")
    _check_bhnd("q", q, dtype)
    B, H, N, D = q.shape
    _check_bhnd("k", k, dtype, q.shape)
    _check_bhnd("v", v, dtype, q.shape)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bhnd("out", out, dtype, q.shape)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_rows("lse", lse, (B, H, N))
    lib = _lib.load()
    fn = lib.fa_fwd if dtype == torch.bfloat16 else lib.fa_fwd_f32
    name = "fa_fwd" if dtype == torch.bfloat16 else "fa_fwd_f32"
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, D, float(scale), int(bool(causal)), _stream_ptr(q, stream))
    _lib.check(name, rc)
    return out, lse


def kv_splits(B: int, H: int, Nq: int, Nk: int, D: int, causal: bool = False) -> int:
    """The key-range count ``fa_fwd_kv`` picks for ``num_splits=0``."""
    n = _lib.load().fa_fwd_kv_splits(B, H, Nq, Nk, D, int(bool(causal)))
    _lib.check("fa_fwd_kv_splits", min(n, 0))
    return n


def fwd_kv(q, k, v, scale: float | None = None, causal: bool = False, num_splits: int = 0, out=None, lse=None,
           workspace=None, stream=None):
    """``fa_fwd_kv``: attention of q [B, H, Nq, D] over k, v [B, H, Nk, D].

    Under ``causal`` the query rows are the last Nq positions of the key
    sequence (row i sees keys 0 .. i + Nk - Nq).  The keys of each query
    block are split into ``num_splits`` ranges (0: the library's choice)
    whose results are merged on the GPU.  The workspace they need is
    allocated here with torch unless one is passed (a uint8 GPU tensor of at
    least ``fa_fwd_kv_workspace_bytes`` bytes).  Returns (o, lse).
    """
    torch = _torch()
    _check_bhnd("q", q, torch.bfloat16)
    B, H, Nq, D = q.shape
    _check_bhnd("k", k, torch.bfloat16)
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, D):
        raise ValueError(f"k has shape {tuple(k.shape)}, expected ({B}, {H}, Nk, {D})")
    _check_bhnd("v", v, torch.bfloat16, k.shape)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lib = _lib.load()
    splits = int(num_splits) if num_splits else kv_splits(B, H, Nq, Nk, D, causal)
    need = lib.fa_fwd_kv_workspace_bytes(B, H, Nq, D, splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None and (not workspace.is_cuda or workspace.dtype != torch.uint8 or not workspace.is_contiguous()):
        raise TypeError("workspace must be a contiguous uint8 GPU tensor")
    ws_ptr = _ptr(workspace) if workspace is not None else ctypes_void(None)
    ws_bytes = workspace.numel() if workspace is not None else 0
    out = torch.empty_like(q) if out is None else out
    _check_bhnd("out", out, torch.bfloat16, q.shape)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_rows("lse", lse, (B, H, Nq))
    rc = lib.fa_fwd_kv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, D, float(scale), int(bool(causal)), splits,
        ws_ptr, ws_bytes, _stream_ptr(q, stream),
    )
    _lib.check("fa_fwd_kv", rc)
    return out, lse


def fwd_kv_noalloc(q, k, v, out, lse, scale: float | None = None, causal: bool = False, num_splits: int = 0,
                   stream=None):
    """``fa_fwd_kv_noalloc``: ``fwd_kv`` with the key-range partials in the
    library's per-device scratch array instead of a workspace.  The caller
    passes the outputs (o [B, H, Nq, D] bf16, lse [B, H, Nq] float32); the
    call allocates nothing.  Calls that overlap on one device race on the
    scratch.  Returns (out, lse)."""
    torch = _torch()
    _check_bhnd("q", q, torch.bfloat16)
    B, H, Nq, D = q.shape
    _check_bhnd("k", k, torch.bfloat16)
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, D):
        raise ValueError(f"k has shape {tuple(k.shape)}, expected ({B}, {H}, Nk, {D})")
    _check_bhnd("v", v, torch.bfloat16, k.shape)
    _check_bhnd("out", out, torch.bfloat16, q.shape)
    _check_rows("lse", lse, (B, H, Nq))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = _lib.load().fa_fwd_kv_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, D, float(scale), int(bool(causal)),
        int(num_splits), _stream_ptr(q, stream),
    )
    _lib.check("fa_fwd_kv_noalloc", rc)
    return out, lse


SPARSE_BLOCK = 64  # rows of a query block and of a key block in fa_fwd_sparse's mask


def fwd_sparse(q, k, v, block_mask, scale: float | None = None, causal: bool = False, out=None, lse=None, stream=None):
    """``fa_fwd_sparse``: the forward restricted to the (query block, key
    block) pairs of ``block_mask``.

    block_mask: uint8 GPU tensor [nb, nb] (one mask for every head) or
    [B, H, nb, nb] / [B*H, nb, nb] (per head), nb = ceil(N / 64); a nonzero
    entry (a, c) lets query rows 64a.. see key rows 64c...  Rows that see no
    key get O = 0 and L = -inf.  Returns (o, lse).
    """
    torch = _torch()
    _check_bhnd("q", q, torch.bfloat16)
    B, H, N, D = q.shape
    _check_bhnd("k", k, torch.bfloat16, q.shape)
    _check_bhnd("v", v, torch.bfloat16, q.shape)
    nb = -(-N // SPARSE_BLOCK)
    if not (isinstance(block_mask, torch.Tensor) and block_mask.is_cuda and block_mask.dtype == torch.uint8
            and block_mask.is_contiguous()):
        raise TypeError("block_mask must be a contiguous uint8 GPU tensor")
    if tuple(block_mask.shape) == (nb, nb):
        heads = 1
    elif tuple(block_mask.shape) in ((B, H, nb, nb), (B * H, nb, nb)):
        heads = B * H
    else:
        raise ValueError(f"block_mask has shape {tuple(block_mask.shape)}, expected ({nb}, {nb}) or per head")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = torch.empty_like(q) if out is None else out
    _check_bhnd("out", out, torch.bfloat16, q.shape)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_rows("lse", lse, (B, H, N))
    rc = _lib.load().fa_fwd_sparse(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, D, float(scale), int(bool(causal)),
        _ptr(block_mask), heads, _stream_ptr(q, stream),
    )
    _lib.check("fa_fwd_sparse", rc)
    return out, lse


def bwd_dq(q, k, v, o, do, lse, scale: float | None = None, causal: bool = False, dq=None, delta=None, stream=None):
    """dQ (bf16) and delta = rowsum(dO * O) (float32) via ``fa_bwd_dq``."""
    torch = _torch()
    _check_bhnd("q", q, torch.bfloat16)
    B, H, N, D = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        _check_bhnd(name, t, torch.bfloat16, q.shape)
    _check_rows("lse", lse, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if delta is None else delta
    _check_bhnd("dq", dq, torch.bfloat16, q.shape)
    _check_rows("delta", delta, (B, H, N))
    rc = _lib.load().fa_bwd_dq(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(delta), _ptr(dq),
        B, H, N, D, float(scale), int(bool(causal)), _stream_ptr(q, stream),
    )
    _lib.check("fa_bwd_dq", rc)
    return dq, delta


def bwd_dkdv(q, k, v, do, lse, delta, scale: float | None = None, causal: bool = False, dk=None, dv=None, stream=None):
    """dK and dV (bf16) via ``fa_bwd_dkdv``; ``delta`` comes from :func:`bwd_dq`."""
    torch = _torch()
    _check_bhnd("q", q, torch.bfloat16)
    B, H, N, D = q.shape
    for name, t in (("k", k), ("v", v), ("do", do)):
        _check_bhnd(name, t, torch.bfloat16, q.shape)
    _check_rows("lse", lse, (B, H, N))
    _check_rows("delta", delta, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_bhnd("dk", dk, torch.bfloat16, q.shape)
    _check_bhnd("dv", dv, torch.bfloat16, q.shape)
    rc = _lib.load().fa_bwd_dkdv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(delta), _ptr(dk), _ptr(dv),
        B, H, N, D, float(scale), int(bool(causal)), _stream_ptr(q, stream),
    )
    _lib.check("fa_bwd_dkdv", rc)
    return dk, dv


def bwd(q, k, v, o, do, lse, scale: float | None = None, causal: bool = False, stream=None):
    """Full backward: (dq, dk, dv, delta).  Two launches on one stream."""
    dq, delta = bwd_dq(q, k, v, o, do, lse, scale, causal, stream=stream)
    dk, dv = bwd_dkdv(q, k, v, do, lse, delta, scale, causal, stream=stream)
    return dq, dk, dv, delta
