"""MI355X (gfx950) dense flash-attention forward and Sq=1 decode.

Thin Python binding over libfa.so: it checks tensors, then passes device
pointers and torch's current HIP stream through the C ABI (include/fa.h).
Every step of the computation runs in the library's HIP kernels; there is no
other code path.

    fwd(q, k, v, causal=..., scale=...)         -> o           (and lse on request)
    decode(q, kcache, vcache, valid_len, ...)   -> o
"""
from __future__ import annotations

import ctypes
import math

from ._lib import (FA_BF16, FA_FP16, FaError, FwdPlan, check, lib)  # noqa: F401

__all__ = ["fwd", "fwd_varlen", "bwd", "decode", "decode_noalloc", "decode_paged", "fwd_plan", "decode_workspace_bytes", "DecodeWorkspace", "FaError",
           "lib", "build"]


def build(verbose: bool = False) -> str:
    from .build import build as _b
    return _b(verbose=verbose)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float16:
        return FA_FP16
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float16")


def _stream_ptr(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_tensor(name, t, shape, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, return_lse=False,
        schedule: dict | None = None):
    """Dense attention forward: q [B,Hq,Sq,D], k/v [B,Hkv,Sk,D] -> o [B,Hq,Sq,D].

    Bottom-right aligned causal mask when causal=True.  scale defaults to
    1/sqrt(D).  With return_lse=True also returns the fp32 row log-sum-exp
    [B,Hq,Sq].  `schedule` (keys persistent, hkv_major, xcd_map, each 0/1,
    and optionally queue 0/1 and split_tiles >= 0) overrides the automatic
    launch schedule
    (fa_fwd_planned); without a split the result is bitwise the same, with
    one it differs by rounding only."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("fwd needs GPU tensors")
    _check_tensor("k", k, (B, Hkv, Sk, D), q.dtype, dev)
    _check_tensor("v", v, (B, Hkv, Sk, D), q.dtype, dev)
    _check_tensor("q", q, (B, Hq, Sq, D), q.dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, (B, Hq, Sq, D), q.dtype, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dt = _dtype_code(q)
    stream = _stream_ptr(q)
    if schedule is not None:
        plan = FwdPlan()
        for key in ("persistent", "hkv_major", "xcd_map"):
            setattr(plan, key, int(schedule[key]))
        plan.split_tiles = int(schedule.get("split_tiles", 0))
        plan.queue = int(schedule.get("queue", 0))
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev) if return_lse else None
        st = lib().fa_fwd_planned(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse.data_ptr() if lse is not None else None, B, Hq, Hkv, Sq, Sk,
                                  D, int(bool(causal)), float(scale), dt, ctypes.byref(plan), stream)
        check(st, "fa_fwd_planned")
        return (out, lse) if return_lse else out
    if return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
        st = lib().fa_fwd_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), B, Hq, Hkv, Sq, Sk, D, int(bool(causal)),
                              float(scale), dt, stream)
        check(st, "fa_fwd_lse")
        return out, lse
    st = lib().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, Sq,
                      Sk, D, int(bool(causal)), float(scale), dt, stream)
    check(st, "fa_fwd")
    return out


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
               causal: bool = False, scale: float | None = None, out=None, return_lse=False):
    """Attention over a batch of sequences packed along the token dimension:
    q [total_q, Hq, D], k/v [total_k, Hkv, D], cu_seqlens_q/k int32 [B+1] on
    the device (sequence b owns rows cu[b] .. cu[b+1]-1) -> o [total_q, Hq, D].

    max_seqlen_q/k bound the sequence lengths (host integers).  Rows that
    belong to no sequence are left as they are in `out` (uninitialised when
    `out` is None).  With return_lse=True also returns the fp32 row
    log-sum-exp [Hq, total_q]."""
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be 3-D [total, H, D]")
    total_q, Hq, D = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("fwd_varlen needs GPU tensors")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.shape != cu_seqlens_k.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B + 1]")
    B = cu_seqlens_q.shape[0] - 1
    if B < 0:
        raise ValueError("cu_seqlens must hold at least one entry")
    _check_tensor("cu_seqlens_q", cu_seqlens_q, (B + 1,), torch.int32, dev)
    _check_tensor("cu_seqlens_k", cu_seqlens_k, (B + 1,), torch.int32, dev)
    _check_tensor("k", k, (total_k, Hkv, D), q.dtype, dev)
    _check_tensor("v", v, (total_k, Hkv, D), q.dtype, dev)
    _check_tensor("q", q, (total_q, Hq, D), q.dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, (total_q, Hq, D), q.dtype, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lse = torch.empty((Hq, total_q), dtype=torch.float32, device=dev) if return_lse else None
    st = lib().fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr() if lse is not None else None,
                             cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, Hq, Hkv,
                             total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), D,
                             int(bool(causal)), float(scale), _dtype_code(q), _stream_ptr(q))
    check(st, "fa_fwd_varlen")
    return (out, lse) if return_lse else out


def fwd_plan(B, Hq, Hkv, Sq, Sk, D, causal) -> dict:
    """The launch plan fa_fwd uses for these sizes (host only)."""
    plan = FwdPlan()
    check(lib().fa_fwd_plan(B, Hq, Hkv, Sq, Sk, D, int(bool(causal)), ctypes.byref(plan)),
          "fa_fwd_plan")
    return {f: getattr(plan, f) for f, _ in FwdPlan._fields_}


def decode_workspace_bytes(B, Hq, Hkv, D, capacity, Sq: int = 1) -> int:
    if Sq == 1:
        return int(lib().fa_decode_workspace_bytes(B, Hq, Hkv, D, capacity))
    return int(lib().fa_decode_multi_workspace_bytes(B, Sq, Hq, Hkv, D, capacity))


class DecodeWorkspace:
    """Zero-filled device workspace for decode, reusable call after call on
    one stream (each call leaves its run-complete flags at zero).  Sq > 1
    sizes it for multi-token decode steps of Sq query tokens."""

    def __init__(self, B, Hq, Hkv, D, capacity, device="cuda", Sq: int = 1):
        torch = _torch()
        n = decode_workspace_bytes(B, Hq, Hkv, D, capacity, Sq)
        if n == 0:
            raise ValueError("invalid decode sizes")
        self.key = (B, Sq, Hq, Hkv, D, capacity)
        self.nbytes = n
        self.buf = torch.zeros(n + 256, dtype=torch.uint8, device=device)
        off = (-self.buf.data_ptr()) % 256
        self.ptr = self.buf.data_ptr() + off


def _q_shape(q):
    """[B, Hq, D] (one query token) or [B, Sq, Hq, D] -> (B, Sq, Hq, D)."""
    if q.dim() == 3:
        return q.shape[0], 1, q.shape[1], q.shape[2]
    if q.dim() == 4:
        return tuple(q.shape)
    raise ValueError("q must be [B, Hq, D] or [B, Sq, Hq, D]")


def decode(q, kcache, vcache, valid_len, causal: bool = False, scale: float | None = None,
           out=None, workspace: DecodeWorkspace | None = None):
    """Decode attention over kcache/vcache [B,capacity,Hkv,D] with valid_len
    int32[B] on the device.  q [B,Hq,D] -> o [B,Hq,D] (one token), or
    q [B,Sq,Hq,D] -> o [B,Sq,Hq,D]: Sq query tokens at positions
    L-Sq .. L-1, bottom-right causal among themselves when causal=True."""
    torch = _torch()
    if kcache.dim() != 4:
        raise ValueError("the caches must be [B, capacity, Hkv, D]")
    B, Sq, Hq, D = _q_shape(q)
    cap, Hkv = kcache.shape[1], kcache.shape[2]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("decode needs GPU tensors")
    _check_tensor("q", q, tuple(q.shape), q.dtype, dev)
    _check_tensor("kcache", kcache, (B, cap, Hkv, D), q.dtype, dev)
    _check_tensor("vcache", vcache, (B, cap, Hkv, D), q.dtype, dev)
    _check_tensor("valid_len", valid_len, (B,), torch.int32, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, tuple(q.shape), q.dtype, dev)
    if workspace is None:
        workspace = DecodeWorkspace(B, Hq, Hkv, D, cap, device=dev, Sq=Sq)
    if workspace.key != (B, Sq, Hq, Hkv, D, cap):
        raise ValueError("workspace was sized for other shapes")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if q.dim() == 3:
        st = lib().fa_decode(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(),
                             valid_len.data_ptr(), cap, out.data_ptr(), B, Hq, Hkv, D,
                             int(bool(causal)), float(scale), _dtype_code(q), workspace.ptr,
                             workspace.nbytes, _stream_ptr(q))
        check(st, "fa_decode")
    else:
        st = lib().fa_decode_multi(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(),
                                   valid_len.data_ptr(), cap, out.data_ptr(), B, Sq, Hq, Hkv, D,
                                   int(bool(causal)), float(scale), _dtype_code(q), workspace.ptr,
                                   workspace.nbytes, _stream_ptr(q))
        check(st, "fa_decode_multi")
    return out


def decode_noalloc(q, kcache, vcache, valid_len, out, causal: bool = False,
                   scale: float | None = None):
    """decode() for one query token through the entry point that allocates
    nothing (fa_decode_noalloc): its workspace is built into the library, so
    neither the call nor this wrapper allocates; `out` [B,Hq,D] is required.
    Calls that overlap in time on one GPU race."""
    torch = _torch()
    if q.dim() != 3 or kcache.dim() != 4:
        raise ValueError("q must be [B, Hq, D] and the caches [B, capacity, Hkv, D]")
    B, Hq, D = q.shape
    cap, Hkv = kcache.shape[1], kcache.shape[2]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("decode_noalloc needs GPU tensors")
    _check_tensor("kcache", kcache, (B, cap, Hkv, D), q.dtype, dev)
    _check_tensor("vcache", vcache, (B, cap, Hkv, D), q.dtype, dev)
    _check_tensor("valid_len", valid_len, (B,), torch.int32, dev)
    _check_tensor("out", out, (B, Hq, D), q.dtype, dev)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = lib().fa_decode_noalloc(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(),
                                 valid_len.data_ptr(), cap, out.data_ptr(), B, Hq, Hkv, D,
                                 int(bool(causal)), float(scale), _dtype_code(q), _stream_ptr(q))
    check(st, "fa_decode_noalloc")
    return out


def decode_paged(q, k_pages, v_pages, page_table, valid_len, causal: bool = False,
                 scale: float | None = None, out=None, workspace: DecodeWorkspace | None = None):
    """Sq=1 attention over a paged cache: q [B,Hq,D], k_pages/v_pages
    [num_pages, page_size, Hkv, D], page_table int32 [B, pages_per_seq] and
    valid_len int32[B] on the device -> o [B,Hq,D].  Token t of batch b is
    row t % page_size of page page_table[b, t // page_size]; page_size must be
    a multiple of 32.  q [B,Sq,Hq,D] decodes Sq tokens as decode() does."""
    torch = _torch()
    if k_pages.dim() != 4 or page_table.dim() != 2:
        raise ValueError("the pools must be [num_pages, page_size, Hkv, D] and page_table "
                         "[B, pages_per_seq]")
    B, Sq, Hq, D = _q_shape(q)
    num_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    pages_per_seq = page_table.shape[1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("decode_paged needs GPU tensors")
    _check_tensor("q", q, tuple(q.shape), q.dtype, dev)
    _check_tensor("k_pages", k_pages, (num_pages, page_size, Hkv, D), q.dtype, dev)
    _check_tensor("v_pages", v_pages, (num_pages, page_size, Hkv, D), q.dtype, dev)
    _check_tensor("page_table", page_table, (B, pages_per_seq), torch.int32, dev)
    _check_tensor("valid_len", valid_len, (B,), torch.int32, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, tuple(q.shape), q.dtype, dev)
    cap = pages_per_seq * page_size
    if workspace is None:
        workspace = DecodeWorkspace(B, Hq, Hkv, D, cap, device=dev, Sq=Sq)
    if workspace.key != (B, Sq, Hq, Hkv, D, cap):
        raise ValueError("workspace was sized for other shapes")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    args = (q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), page_table.data_ptr(),
            valid_len.data_ptr(), page_size, pages_per_seq, num_pages, out.data_ptr(), B)
    tail = (Hq, Hkv, D, int(bool(causal)), float(scale), _dtype_code(q), workspace.ptr,
            workspace.nbytes, _stream_ptr(q))
    if q.dim() == 3:
        check(lib().fa_decode_paged(*args, *tail), "fa_decode_paged")
    else:
        check(lib().fa_decode_paged_multi(*args, Sq, *tail), "fa_decode_paged_multi")
    return out


def bwd(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None,
        dq=None, dk=None, dv=None):
    """Backward pass: gradients (dq, dk, dv) of o = fwd(q, k, v) for an output
    gradient dout, from the forward's output o and row log-sum-exp lse
    (fwd(..., return_lse=True)).  Layouts as fwd; dk/dv add over the query
    heads of a GQA group."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v, o, dout must be 4-D [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("bwd needs GPU tensors")
    for name, t, shape in (("q", q, (B, Hq, Sq, D)), ("k", k, (B, Hkv, Sk, D)),
                           ("v", v, (B, Hkv, Sk, D)), ("o", o, (B, Hq, Sq, D)),
                           ("dout", dout, (B, Hq, Sq, D))):
        _check_tensor(name, t, shape, q.dtype, dev)
    _check_tensor("lse", lse, (B, Hq, Sq), torch.float32, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensor("dq", dq, (B, Hq, Sq, D), q.dtype, dev)
    _check_tensor("dk", dk, (B, Hkv, Sk, D), q.dtype, dev)
    _check_tensor("dv", dv, (B, Hkv, Sk, D), q.dtype, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    n = int(lib().fa_bwd_workspace_bytes(B, Hq, Sq))
    buf = torch.empty(n + 256, dtype=torch.uint8, device=dev)
    ws = buf.data_ptr() + (-buf.data_ptr()) % 256
    st = lib().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                      lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv,
                      Sq, Sk, D, int(bool(causal)), float(scale), _dtype_code(q), ws, n,
                      _stream_ptr(q))
    check(st, "fa_bwd")
    return dq, dk, dv
