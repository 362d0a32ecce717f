"""Tensor-level call of the attention forward: checks shapes, allocates o and lse with torch, calls fa_fwd.

    o, lse = forward(q, k, v, causal=False, scale=None)

q, k, v: [B, H, N, d] contiguous CUDA (ROCm) tensors, all bf16 (-> fa_fwd) or all fp32 (-> fa_fwd_f32),
d in {64, 128}. scale defaults to 1/sqrt(d). Returns o (same dtype and shape as q) and lse ([B, H, N] fp32,
natural log). The kernel is enqueued on torch's current stream (or `stream`, a raw hipStream_t int).
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
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"q, k, v must all be bfloat16 or all float32, got {q.dtype} {k.dtype} {v.dtype}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, scale: float | None = None,
            out: torch.Tensor | None = None, lse: torch.Tensor | None = None, stream: int | None = None):
    _check(q, k, v)
    B, H, N, d = q.shape
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
    if stream is None:
        with torch.cuda.device(q.device):
            stream = torch.cuda.current_stream().cuda_stream
    fn = binding.fa_fwd if q.dtype == torch.bfloat16 else binding.fa_fwd_f32
    with torch.cuda.device(q.device):
        rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d, int(bool(causal)),
                float(scale), int(stream))
    if rc != binding.FA_OK:
        raise RuntimeError(f"fa_fwd failed ({rc}): {binding.fa_strerror(rc)}")
    return out, lse
