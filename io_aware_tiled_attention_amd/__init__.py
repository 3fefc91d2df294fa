"""Exact IO-aware tiled attention for AMD MI355X (gfx950), forward and backward.

Thin torch-facing binding over the C ABI of ``libfa_gfx950.so`` (see
include/fa.h).  torch provides device memory and the current stream; every
step of the computation runs in the library's HIP kernels.  Tensors are
contiguous [B, H, N, d] in float32 or bfloat16 on a ROCm device; lse is
[B, H, N] float32.

    o, lse = forward(q, k, v, causal=True)
    dq, dk, dv = backward(q, k, v, o, do, lse, causal=True)
    o, lse = forward_block_sparse(q, k, v, block_mask, block_q=128, block_k=64)
    dq, dk, dv = backward_block_sparse(q, k, v, o, do, lse, block_mask, block_q=128, block_k=64)
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

from . import _lib
from ._lib import (FA_BF16, FA_F32, FaError, fa_backward, fa_backward_block_sparse, fa_backward_dkdv,
                   fa_backward_dq, fa_backward_dropout, fa_backward_noalloc,
                   fa_backward_preprocess, fa_backward_workspace_size, fa_decode, fa_decode_num_splits,
                   fa_decode_workspace_size, fa_forward, fa_forward_block_sparse, fa_forward_dropout,
                   fa_forward_fp8, fa_strerror)

__all__ = ["forward", "forward_block_sparse", "forward_fp8", "backward", "backward_block_sparse", "decode",
           "workspace_size", "FaError", "FA_F32", "FA_BF16", "fa_forward", "fa_forward_block_sparse", "fa_backward",
           "fa_backward_block_sparse", "fa_backward_workspace_size",
           "fa_backward_preprocess", "fa_backward_dkdv", "fa_backward_dq", "fa_forward_dropout",
           "fa_backward_dropout", "fa_forward_fp8", "fa_decode",
           "fa_decode_workspace_size", "fa_decode_num_splits", "fa_strerror", "load_library",
           "backward_stages", "backward_noalloc", "fa_backward_noalloc"]


def load_library():
    """Load the HIP library now (raises if it has not been built)."""
    return _lib.load()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.float32 or torch.bfloat16")


def _check(name, t, shape, dtype, device):
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B, H, N, d]")


def _stream_ptr(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def forward(q, k, v, causal: bool = False, scale: Optional[float] = None,
            out=None, lse=None, dropout_p: float = 0.0, seed: int = 0,
            offset: int = 0) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """O = softmax(scale * Q K^T) V and lse = ln rowsum exp(scale * Q K^T).

    ``dropout_p`` > 0: dropout on the probabilities, O = (P o Z) V / (1 - t/256)
    with t = round(256 dropout_p); the mask Z is regenerated from (seed,
    offset), so :func:`backward` must get the same three values."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    if q.device.type != "cuda":
        raise ValueError("tensors must live on a ROCm device")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(name, t, q.shape, q.dtype, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check("out", out, q.shape, q.dtype, q.device)
    _check("lse", lse, (B, H, N), torch.float32, q.device)
    if dropout_p:
        st = fa_forward_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                B, H, N, d, causal, scale, _dtype_code(q), dropout_p, seed, offset,
                                _stream_ptr(q.device))
        if st != 0:
            raise FaError(st, "fa_forward_dropout")
        return out, lse
    st = fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, H, N, d, causal, scale, _dtype_code(q), _stream_ptr(q.device))
    if st != 0:
        raise FaError(st, "fa_forward")
    return out, lse


def forward_fp8(q, k, v, causal: bool = False, scale: Optional[float] = None, q_descale: float = 1.0,
                k_descale: float = 1.0, v_descale: float = 1.0, out=None, lse=None):
    """Attention of FP8 (OCP E4M3) inputs with per-tensor descale factors.

    q, k, v: [B, H, N, d] tensors of dtype torch.float8_e4m3fn (or uint8 holding
    the codes); O is returned in bfloat16, lse in float32.
    """
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    if q.device.type != "cuda":
        raise ValueError("tensors must live on a ROCm device")
    if q.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise TypeError("q, k, v must be torch.float8_e4m3fn (or uint8 codes)")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(name, t, q.shape, q.dtype, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check("out", out, (B, H, N, d), torch.bfloat16, q.device)
    _check("lse", lse, (B, H, N), torch.float32, q.device)
    st = fa_forward_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                        causal, scale, q_descale, k_descale, v_descale, _stream_ptr(q.device))
    if st != 0:
        raise FaError(st, "fa_forward_fp8")
    return out, lse


def forward_block_sparse(q, k, v, block_mask, block_q: int, block_k: int, causal: bool = False,
                         scale: Optional[float] = None, out=None, lse=None):
    """Block-sparse attention: like :func:`forward`, with the keys of each row
    restricted to the blocks that ``block_mask`` keeps.

    block_mask: uint8 tensor [Hm, ceil(N / block_q), ceil(N / block_k)] on the
    same device, Hm = 1 (every head) or H (per head, shared by the batch);
    non-zero keeps a block of block_q query rows by block_k keys.  block_q must
    be a multiple of 32 and block_k of 64.  Rows that keep no key get O = 0 and
    lse = -inf.
    """
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    if q.device.type != "cuda":
        raise ValueError("tensors must live on a ROCm device")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(name, t, q.shape, q.dtype, q.device)
    if block_mask.dim() != 3:
        raise ValueError("block_mask must be [Hm, ceil(N / block_q), ceil(N / block_k)]")
    tq, tk = -(-N // block_q), -(-N // block_k)
    _check("block_mask", block_mask, (block_mask.shape[0], tq, tk), torch.uint8, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check("out", out, q.shape, q.dtype, q.device)
    _check("lse", lse, (B, H, N), torch.float32, q.device)
    st = fa_forward_block_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                 block_mask.data_ptr(), block_mask.shape[0], block_q, block_k, B, H, N, d, causal,
                                 scale, _dtype_code(q), _stream_ptr(q.device))
    if st != 0:
        raise FaError(st, "fa_forward_block_sparse")
    return out, lse


def backward_block_sparse(q, k, v, o, do, lse, block_mask, block_q: int, block_k: int, causal: bool = False,
                          scale: Optional[float] = None, dq=None, dk=None, dv=None, workspace=None):
    """dQ, dK, dV of :func:`forward_block_sparse` for the upstream gradient dO
    (o and lse from that forward with the same mask, blocks, causal, scale)."""
    import torch
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, q.shape, q.dtype, q.device)
    _check("lse", lse, (B, H, N), torch.float32, q.device)
    if block_mask.dim() != 3:
        raise ValueError("block_mask must be [Hm, ceil(N / block_q), ceil(N / block_k)]")
    tq, tk = -(-N // block_q), -(-N // block_k)
    _check("block_mask", block_mask, (block_mask.shape[0], tq, tk), torch.uint8, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(name, t, q.shape, q.dtype, q.device)
    need = fa_backward_workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = fa_backward_block_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                  lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), block_mask.data_ptr(),
                                  block_mask.shape[0], block_q, block_k, B, H, N, d, causal, scale, _dtype_code(q),
                                  workspace.data_ptr(), workspace.numel(), _stream_ptr(q.device))
    if st != 0:
        raise FaError(st, "fa_backward_block_sparse")
    return dq, dk, dv


def decode(q, k, v, causal: bool = True, scale: Optional[float] = None, num_splits: int = 0,
           out=None, lse=None, workspace=None):
    """Split-KV decoding: Nq <= 32 new queries against a cache of Nk keys/values.

    q: [B, H, Nq, d]; k, v: [B, H, Nk, d] (same dtype and device).  The
    queries are the last Nq positions: with ``causal`` query i sees keys
    0 .. Nk - Nq + i, otherwise all Nk.  ``num_splits`` = 0 lets the library
    choose how many key chunks each head is cut into.  ``workspace``: an
    optional uint8 scratch buffer of at least fa_decode_workspace_size bytes.
    """
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H, Nk, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if q.device.type != "cuda":
        raise ValueError("tensors must live on a ROCm device")
    _check("q", q, q.shape, q.dtype, q.device)
    for name, t in (("k", k), ("v", v)):
        _check(name, t, (B, H, Nk, d), q.dtype, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check("out", out, q.shape, q.dtype, q.device)
    _check("lse", lse, (B, H, Nq), torch.float32, q.device)
    need = fa_decode_workspace_size(B, H, Nq, Nk, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d,
                   causal, scale, _dtype_code(q), num_splits, workspace.data_ptr(), workspace.numel(),
                   _stream_ptr(q.device))
    if st != 0:
        raise FaError(st, "fa_decode")
    return out, lse


def workspace_size(B: int, H: int, N: int, d: int) -> int:
    return fa_backward_workspace_size(B, H, N, d)


def backward(q, k, v, o, do, lse, causal: bool = False, scale: Optional[float] = None,
             dq=None, dk=None, dv=None, workspace=None, dropout_p: float = 0.0, seed: int = 0,
             offset: int = 0):
    """dQ, dK, dV of O = attention(Q, K, V) for the upstream gradient dO
    (with dropout: the same dropout_p, seed and offset as the forward)."""
    import torch
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, q.shape, q.dtype, q.device)
    _check("lse", lse, (B, H, N), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(name, t, q.shape, q.dtype, q.device)
    need = fa_backward_workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if dropout_p:
        st = fa_backward_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                 lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                                 causal, scale, _dtype_code(q), dropout_p, seed, offset, workspace.data_ptr(),
                                 workspace.numel(), _stream_ptr(q.device))
        if st != 0:
            raise FaError(st, "fa_backward_dropout")
        return dq, dk, dv
    st = fa_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                     lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                     causal, scale, _dtype_code(q), workspace.data_ptr(), workspace.numel(),
                     _stream_ptr(q.device))
    if st != 0:
        raise FaError(st, "fa_backward")
    return dq, dk, dv


def backward_stages(q, k, v, o, do, lse, causal: bool = False, scale: Optional[float] = None,
                    dq=None, dk=None, dv=None, workspace=None):
    """The same result as :func:`backward`, through the three staged entry points
    (dQ before dK/dV here, to exercise the documented freedom of order)."""
    import torch
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, q.shape, q.dtype, q.device)
    _check("lse", lse, (B, H, N), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    need = fa_backward_workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dt, s, ws, wn = _dtype_code(q), _stream_ptr(q.device), workspace.data_ptr(), workspace.numel()
    st = fa_backward_preprocess(o.data_ptr(), do.data_ptr(), lse.data_ptr(), B, H, N, d, dt, ws, wn, s)
    if st != 0:
        raise FaError(st, "fa_backward_preprocess")
    st = fa_backward_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), dq.data_ptr(),
                        B, H, N, d, causal, scale, dt, ws, wn, s)
    if st != 0:
        raise FaError(st, "fa_backward_dq")
    st = fa_backward_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), dk.data_ptr(),
                          dv.data_ptr(), B, H, N, d, causal, scale, dt, ws, wn, s)
    if st != 0:
        raise FaError(st, "fa_backward_dkdv")
    return dq, dk, dv


def backward_noalloc(q, k, v, o, do, lse, causal: bool = False, scale: Optional[float] = None,
                     dq=None, dk=None, dv=None):
    """The same result as :func:`backward` through fa_backward_noalloc, whose
    workspace is the library's own per-GPU device array (no allocation by the
    library; problems past FA_NOALLOC_SCRATCH_BYTES of workspace raise
    FA_ERR_SCRATCH).  Calls that overlap in time on one GPU share that array
    and race."""
    import torch
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, q.shape, q.dtype, q.device)
    _check("lse", lse, (B, H, N), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(name, t, q.shape, q.dtype, q.device)
    st = fa_backward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                             lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                             causal, scale, _dtype_code(q), _stream_ptr(q.device))
    if st != 0:
        raise FaError(st, "fa_backward_noalloc")
    return dq, dk, dv
