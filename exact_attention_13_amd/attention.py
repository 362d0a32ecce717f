"""Tensor-level call of the attention forward: checks shapes, allocates o and lse with torch, calls the C ABI.

    o, lse = forward(q, k, v, causal=False, scale=None, kv_len=None)

q: [B, H, N, d], k and v: [B, H_kv, N, d] contiguous CUDA (ROCm) tensors, all bf16 or all fp32, d in {64, 128}.
H_kv < H (grouped/multi-query attention: H_kv divides H, query head h reads key/value head h // (H // H_kv)) and
kv_len (a device int32 [B] tensor of valid-key counts, key padding) are bf16 only. The entry point is fa_fwd,
fa_fwd_gqa, fa_fwd_kpad or fa_fwd_f32 accordingly. scale defaults to 1/sqrt(d). Returns o (same dtype and shape
as q) and lse ([B, H, N] fp32, natural log). The kernel is enqueued on torch's current stream (or `stream`, a raw
hipStream_t int).
"""
from __future__ import annotations

import math

import torch

from . import binding


def _check(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> None:
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device, got {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous ([B, H, N, d] row-major)")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d], got shape {tuple(t.shape)}")
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[2:] != k.shape[2:] or k.shape[1] < 1 \
            or q.shape[1] % k.shape[1] != 0:
        raise ValueError(f"q [B,H,N,d] and k, v [B,H_kv,N,d] (H_kv dividing H) disagree: {tuple(q.shape)} "
                         f"{tuple(k.shape)} {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"q, k, v must all be bfloat16 or all float32, got {q.dtype} {k.dtype} {v.dtype}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")


def _resolve_stream(stream: int | None, device: torch.device) -> tuple[int, torch.cuda.Stream | None]:
    """The raw stream handle to launch on, and (when it is not torch's current stream) a torch handle of it for
    record_stream: memory this module allocates belongs to the current stream, so tensors used by a kernel on
    another stream are recorded on that stream and are not reused before the kernel has finished."""
    with torch.cuda.device(device):
        cur = torch.cuda.current_stream()
        if stream is None or int(stream) == cur.cuda_stream:
            return cur.cuda_stream, None
        return int(stream), torch.cuda.ExternalStream(int(stream), device=device)


def _record(foreign: torch.cuda.Stream | None, *tensors: torch.Tensor) -> None:
    if foreign is not None:
        for t in tensors:
            t.record_stream(foreign)


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, scale: float | None = None,
            out: torch.Tensor | None = None, lse: torch.Tensor | None = None, stream: int | None = None,
            kv_len: torch.Tensor | None = None):
    _check(q, k, v)
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if (H_kv != H or kv_len is not None) and q.dtype != torch.bfloat16:
        raise TypeError("grouped key/value heads and kv_len are supported for bfloat16 inputs")
    if kv_len is not None and (not isinstance(kv_len, torch.Tensor) or kv_len.dtype != torch.int32
                               or kv_len.shape != (B,) or not kv_len.is_contiguous() or kv_len.device != q.device):
        raise ValueError("kv_len must be a contiguous int32 [B] tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor of q's shape, dtype and device")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    stream, foreign = _resolve_stream(stream, q.device)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr())
    c, sc, st = int(bool(causal)), float(scale), int(stream)
    with torch.cuda.device(q.device):
        if kv_len is not None:
            rc = binding.fa_fwd_kpad(*ptrs, kv_len.data_ptr(), B, H, H_kv, N, d, c, sc, st)
        elif H_kv != H:
            rc = binding.fa_fwd_gqa(*ptrs, B, H, H_kv, N, d, c, sc, st)
        elif q.dtype == torch.bfloat16:
            rc = binding.fa_fwd(*ptrs, B, H, N, d, c, sc, st)
        else:
            rc = binding.fa_fwd_f32(*ptrs, B, H, N, d, c, sc, st)
    if rc != binding.FA_OK:
        raise RuntimeError(f"fa_fwd failed ({rc}): {binding.fa_strerror(rc)}")
    _record(foreign, out, lse)
    return out, lse


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
             dout: torch.Tensor, causal: bool = False, scale: float | None = None, stream: int | None = None,
             kv_len: torch.Tensor | None = None):
    """Gradients (dq, dk, dv) of forward(q, k, v, causal, scale, kv_len=kv_len) -> (o, lse) for an upstream
    gradient dout of o.

    bf16 tensors: q, o, dout [B, H, N, d]; k, v [B, H_kv, N, d]; lse [B, H, N] fp32 from the same forward call;
    kv_len: None or the forward's device int32 [B] key-padding lengths. Allocates dq, dk, dv and the workspace with
    torch and calls fa_bwd (fa_bwd_kpad with kv_len) on torch's current stream (or `stream`).
    """
    _check(q, k, v)
    if q.dtype != torch.bfloat16:
        raise TypeError("the backward pass takes bfloat16 tensors")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    for name, t in (("o", o), ("dout", dout)):
        if (not isinstance(t, torch.Tensor) or t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous()
                or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous tensor of q's shape, dtype and device")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    if kv_len is not None and (not isinstance(kv_len, torch.Tensor) or kv_len.dtype != torch.int32
                               or kv_len.shape != (B,) or not kv_len.is_contiguous() or kv_len.device != q.device):
        raise ValueError("kv_len must be a contiguous int32 [B] tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws = torch.empty((max(binding.fa_bwd_workspace_bytes(B, H, H_kv, N, d), 16),), dtype=torch.uint8,
                     device=q.device)
    stream, foreign = _resolve_stream(stream, q.device)
    with torch.cuda.device(q.device):
        ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr())
        tail = (B, H, H_kv, N, d, int(bool(causal)), float(scale), int(stream))
        if kv_len is not None:
            rc = binding.fa_bwd_kpad(*ptrs, kv_len.data_ptr(), *tail)
        else:
            rc = binding.fa_bwd(*ptrs, *tail)
    if rc != binding.FA_OK:
        raise RuntimeError(f"fa_bwd failed ({rc}): {binding.fa_strerror(rc)}")
    _record(foreign, dq, dk, dv, ws)
    return dq, dk, dv


def forward_fp8(q: torch.Tensor, k: torch.Tensor, vt: torch.Tensor, q_scale: float, k_scale: float, v_scale: float,
                causal: bool = False, scale: float | None = None, stream: int | None = None):
    """Attention of fp8 inputs: q, k [B, H, N, d] and vt = v transposed [B, H, d, N], all float8_e4m3fn, with
    per-tensor scales (real inputs q*q_scale, ...). Returns o (bf16 [B, H, N, d]) and lse (fp32 [B, H, N])."""
    for name, t in (("q", q), ("k", k), ("vt", vt)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-d GPU tensor")
        if t.dtype != torch.float8_e4m3fn:
            raise TypeError(f"{name} must be float8_e4m3fn, got {t.dtype}")
    B, H, N, d = q.shape
    if k.shape != q.shape or vt.shape != (B, H, d, N) or not (q.device == k.device == vt.device):
        raise ValueError(f"q, k [B,H,N,d] and vt [B,H,d,N] disagree: {tuple(q.shape)} {tuple(k.shape)} "
                         f"{tuple(vt.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    stream, foreign = _resolve_stream(stream, q.device)
    with torch.cuda.device(q.device):
        rc = binding.fa_fwd_fp8(q.data_ptr(), k.data_ptr(), vt.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                float(q_scale), float(k_scale), float(v_scale), B, H, N, d, int(bool(causal)),
                                float(scale), int(stream))
    if rc != binding.FA_OK:
        raise RuntimeError(f"fa_fwd_fp8 failed ({rc}): {binding.fa_strerror(rc)}")
    _record(foreign, o, lse)
    return o, lse


def forward_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                   causal: bool = False, scale: float | None = None, stream: int | None = None):
    """Attention over packed variable-length sequences: q [total, H, d], k and v [total, H_kv, d] (bf16, contiguous,
    on the GPU), cu_seqlens a device int32 [B+1] tensor of sequence offsets (0 .. total), max_seqlen >= the longest
    sequence. Every sequence is its own attention problem. Returns o (bf16 [total, H, d]) and lse (fp32 [H, total]).
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous 3-d GPU tensor [total, heads, d]")
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    total, H, d = q.shape
    if k.shape != v.shape or k.shape[0] != total or k.shape[2] != d or k.shape[1] < 1 or H % k.shape[1] != 0 \
            or not (q.device == k.device == v.device):
        raise ValueError(f"q [total,H,d] and k, v [total,H_kv,d] disagree: {tuple(q.shape)} {tuple(k.shape)}")
    if (not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
            or not cu_seqlens.is_contiguous() or cu_seqlens.device != q.device):
        raise ValueError("cu_seqlens must be a contiguous int32 [B+1] tensor on q's device")
    B = cu_seqlens.shape[0] - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    stream, foreign = _resolve_stream(stream, q.device)
    with torch.cuda.device(q.device):
        rc = binding.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   cu_seqlens.data_ptr(), B, H, k.shape[1], total, int(max_seqlen), d,
                                   int(bool(causal)), float(scale), int(stream))
    if rc != binding.FA_OK:
        raise RuntimeError(f"fa_fwd_varlen failed ({rc}): {binding.fa_strerror(rc)}")
    _record(foreign, o, lse)
    return o, lse


def backward_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                    dout: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int, causal: bool = False,
                    scale: float | None = None, stream: int | None = None):
    """Gradients (dq, dk, dv) of forward_varlen(q, k, v, cu_seqlens, max_seqlen, causal, scale) -> (o, lse) for an
    upstream gradient dout [total, H, d] of o. Allocates the outputs and the workspace with torch."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous() or t.dim() != 3 \
                or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bf16 3-d GPU tensor")
    total, H, d = q.shape
    if o.shape != q.shape or dout.shape != q.shape or k.shape != v.shape or k.shape[0] != total \
            or k.shape[2] != d or k.shape[1] < 1 or H % k.shape[1] != 0:
        raise ValueError("q, o, dout [total,H,d] and k, v [total,H_kv,d] disagree")
    if any(t.device != q.device for t in (k, v, o, dout)):
        raise ValueError("q, k, v, o, dout must be on the same device")
    if lse.shape != (H, total) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [H, total] tensor on q's device")
    if (not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
            or not cu_seqlens.is_contiguous() or cu_seqlens.device != q.device):
        raise ValueError("cu_seqlens must be a contiguous int32 [B+1] tensor on q's device")
    B = cu_seqlens.shape[0] - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = binding.fa_bwd_workspace_bytes(B, H, k.shape[1], int(max_seqlen), d)
    ws = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device=q.device)
    stream, foreign = _resolve_stream(stream, q.device)
    with torch.cuda.device(q.device):
        rc = binding.fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                                   cu_seqlens.data_ptr(), B, H, k.shape[1], total, int(max_seqlen), d,
                                   int(bool(causal)), float(scale), int(stream))
    if rc != binding.FA_OK:
        raise RuntimeError(f"fa_bwd_varlen failed ({rc}): {binding.fa_strerror(rc)}")
    _record(foreign, dq, dk, dv, ws)
    return dq, dk, dv


class _Attention(torch.autograd.Function):
    """o = attention(q, k, v) with the library's gradient kernels as its backward (bf16 only)."""

    @staticmethod
    def forward(ctx, q, k, v, causal, scale, kv_len):
        o, lse = forward(q, k, v, causal=causal, scale=scale, kv_len=kv_len)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale, ctx.kv_len = causal, scale, kv_len
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = backward(q, k, v, o, lse, dout.contiguous(), causal=ctx.causal, scale=ctx.scale,
                              kv_len=ctx.kv_len)
        return dq, dk, dv, None, None, None


class _AttentionVarlen(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens, max_seqlen, causal, scale):
        o, lse = forward_varlen(q, k, v, cu_seqlens, max_seqlen, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse, cu_seqlens)
        ctx.max_seqlen, ctx.causal, ctx.scale = max_seqlen, causal, scale
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, o, lse, cu_seqlens = ctx.saved_tensors
        dq, dk, dv = backward_varlen(q, k, v, o, lse, dout.contiguous(), cu_seqlens, ctx.max_seqlen,
                                     causal=ctx.causal, scale=ctx.scale)
        return dq, dk, dv, None, None, None, None


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, scale: float | None = None,
              kv_len: torch.Tensor | None = None) -> torch.Tensor:
    """o of forward(q, k, v, causal, scale, kv_len) as a differentiable torch op: with q, k or v requiring grad,
    o.backward(...) runs fa_bwd (fa_bwd_kpad with kv_len) and accumulates dq, dk, dv. Gradients need bf16 inputs;
    fp32 inputs give a forward-only result."""
    if q.dtype != torch.bfloat16 or not torch.is_grad_enabled() or not (q.requires_grad or k.requires_grad
                                                                          or v.requires_grad):
        return forward(q, k, v, causal=causal, scale=scale, kv_len=kv_len)[0]
    return _Attention.apply(q, k, v, causal, scale, kv_len)


def attention_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                     causal: bool = False, scale: float | None = None) -> torch.Tensor:
    """o of forward_varlen(...) as a differentiable torch op (backward: fa_bwd_varlen)."""
    if not torch.is_grad_enabled() or not (q.requires_grad or k.requires_grad or v.requires_grad):
        return forward_varlen(q, k, v, cu_seqlens, max_seqlen, causal=causal, scale=scale)[0]
    return _AttentionVarlen.apply(q, k, v, cu_seqlens, max_seqlen, causal, scale)
