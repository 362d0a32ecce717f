"""fp64 CPU oracle for the exact attention forward and its gradients.

TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the benchmark's
CPU-baseline leg may import or call this package; the GPU path never does, and
this package imports nothing from it.

The arithmetic lives in attn_oracle.c (forward) and attn_bwd_oracle.c
(gradients): plain C, fp64, one materialised score row per query, sequential
sums. This module only builds them with gcc, loads them with ctypes and widens
the inputs to fp32 (exact for bf16 and fp32 inputs).

Definition followed (unite.ai page "Flash Attention: revolutionizing transformer
efficiency", opening code block and "The Math Behind Flash Attention" item 1):
    o_i = softmax_j(scale * q_i . k_j) v_j,   lse_i = ln sum_j exp(scale * q_i . k_j)
over the visible keys (all j, or j <= i when causal -- a reading of "causal"
in the triton-transformer README). Parity pins: tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRCS = (_HERE / "attn_oracle.c", _HERE / "attn_bwd_oracle.c")
_LIB = _HERE / "liboracle.so"
_lib = None


def build(force: bool = True) -> Path:
    """Compile the oracle sources with gcc into liboracle.so (no -ffast-math: IEEE fp64 semantics)."""
    if force or not _LIB.exists() or any(_LIB.stat().st_mtime < f.stat().st_mtime for f in _SRCS):
        tmp = _LIB.with_suffix(".so.tmp")
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", *map(str, _SRCS), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # FA_ORACLE_LIB: the same sources built another way (the sanitizer tier of the CPU tests builds them with
        # AddressSanitizer and UndefinedBehaviorSanitizer and runs the pins against that build)
        alt = os.environ.get("FA_ORACLE_LIB")
        if not alt and not _LIB.exists():
            build(force=False)
        lib = ctypes.CDLL(alt or str(_LIB))
        f = lib.oracle_attn_rows_ex
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                      ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long,
                      ctypes.c_int, ctypes.c_double, ctypes.c_void_p,
                      ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        g = lib.oracle_attn_bwd_rows
        g.restype = ctypes.c_int
        g.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_long] * 5 + [ctypes.c_int, ctypes.c_double,
                                                                     ctypes.c_void_p,
                                                                     ctypes.c_void_p, ctypes.c_long,
                                                                     ctypes.c_void_p, ctypes.c_long,
                                                                     ctypes.c_void_p, ctypes.c_void_p,
                                                                     ctypes.c_void_p, ctypes.c_int]
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _as_f32(x) -> np.ndarray:
    """Widen a CPU torch tensor (fp8 e4m3fn, bf16 or fp32) or array to a contiguous fp32 ndarray, exactly."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu")
            if x.dtype not in (torch.float8_e4m3fn, torch.bfloat16, torch.float32):
                raise TypeError(f"oracle takes fp8 e4m3fn, bf16 or fp32 inputs, got {x.dtype}")
            return np.ascontiguousarray(x.to(torch.float32).numpy())
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(x)
    if a.dtype != np.float32:
        raise TypeError(f"oracle takes fp32 arrays, got {a.dtype}")
    return np.ascontiguousarray(a)


def attention_rows(q, k, v, causal: bool, scale: float, rows=None, threads: int | None = None, kv_len=None):
    """Oracle output for the listed flat rows (b*H + h)*Nq + i (None: every row, in order).

    q: [B, H, Nq, d], k and v: [B, Hkv, Nk, d], bf16/fp32 (torch CPU tensors or fp32 arrays).
    Hkv divides H; query head h reads key/value head h // (H // Hkv) (grouped/multi-query attention).
    The attention problems have Nq == Nk; key blocks (Nk < Nq) serve the merge pins.
    scale: the fp32 scale handed to the GPU; the oracle uses exactly that value.
    kv_len: None, or B valid-key counts in [0, Nk] (key-padding mask: keys j >= kv_len[b] are masked).
    Returns (o [n_rows, d] float64, lse [n_rows] float64); a row with no visible key has o = 0, lse = -inf.
    """
    qa, ka, va = _as_f32(q), _as_f32(k), _as_f32(v)
    if (qa.ndim != 4 or ka.ndim != 4 or ka.shape != va.shape or qa.shape[0] != ka.shape[0]
            or qa.shape[3] != ka.shape[3] or ka.shape[1] < 1 or qa.shape[1] % ka.shape[1] != 0):
        raise ValueError(f"q [B,H,Nq,d] and k, v [B,Hkv,Nk,d] shapes disagree: {qa.shape} {ka.shape} {va.shape}")
    B, H, N, d = qa.shape
    Hkv, Nk = ka.shape[1], ka.shape[2]
    if kv_len is None:
        len_arr = None
    else:
        len_arr = np.ascontiguousarray(np.asarray(kv_len, dtype=np.int64).reshape(-1))
        if len_arr.size != B or (len_arr < 0).any() or (len_arr > Nk).any():
            raise ValueError(f"kv_len must hold {B} counts in [0, {Nk}], got {len_arr}")
    return _rows_exact_scale(qa, ka, va, causal, float(np.float32(scale)), rows, threads, len_arr)


def _rows_exact_scale(qa, ka, va, causal, sc: float, rows, threads, len_arr):
    """attention_rows on fp32 arrays with the score scale sc used as the given fp64 value."""
    B, H, N, d = qa.shape
    Hkv, Nk = ka.shape[1], ka.shape[2]
    if rows is None:
        n = B * H * N
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = int(rows_arr.size)
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    if n == 0:
        return o, lse
    rc = _load().oracle_attn_rows_ex(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, B, H, Hkv, N, Nk, d,
                                     int(bool(causal)), sc, None if len_arr is None else len_arr.ctypes.data,
                                     None if rows_arr is None else rows_arr.ctypes.data, n, o.ctypes.data,
                                     lse.ctypes.data, int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_rows failed with code {rc}")
    return o, lse


def attention(q, k, v, causal: bool, scale: float, threads: int | None = None, kv_len=None):
    """Oracle output for every row: (o [B,H,N,d] float64, lse [B,H,N] float64)."""
    B, H, N, d = tuple(q.shape)
    o, lse = attention_rows(q, k, v, causal, scale, None, threads, kv_len)
    return o.reshape(B, H, N, d), lse.reshape(B, H, N)


def attention_varlen(q, k, v, cu_seqlens, causal: bool, scale: float, rows=None, threads: int | None = None):
    """Attention of packed variable-length sequences: every sequence is its own attention problem.

    q: [T, H, d], k and v: [T, Hkv, d] (tokens of all sequences back to back; Hkv divides H); cu_seqlens: B+1
    offsets, sequence b holds tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 (batches of sequences of different
    lengths, read as FlashAttention-style packing of the padded batches the key-padding mask of the
    triton-transformer README's usage example describes). Queries of sequence b see only the keys of
    sequence b (and, when causal, only those at or before their own position in it). rows: flat ids t*H + h
    (token t, query head h), or None for all T*H in that order. Each sequence is handed to attention_rows as a
    [1, H, L, d] problem. Returns (o [n, d] float64, lse [n] float64).
    """
    qa, ka, va = _as_f32(q), _as_f32(k), _as_f32(v)
    if qa.ndim != 3 or ka.shape != va.shape or ka.ndim != 3 or ka.shape[0] != qa.shape[0] or \
            ka.shape[2] != qa.shape[2] or qa.shape[1] % ka.shape[1] != 0:
        raise ValueError(f"q [T,H,d] and k, v [T,Hkv,d] disagree: {qa.shape} {ka.shape} {va.shape}")
    T, H, d = qa.shape
    cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
    if cu.size < 1 or cu[0] != 0 or cu[-1] != T or (np.diff(cu) < 0).any():
        raise ValueError(f"cu_seqlens must rise from 0 to {T}: {cu}")
    ids = np.arange(T * H, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    if ids.size and (ids.min() < 0 or ids.max() >= T * H):
        raise ValueError("row ids out of range")
    tok, head = ids // H, ids % H
    seq = np.searchsorted(cu, tok, side="right") - 1  # the sequence holding each token
    o = np.zeros((ids.size, d), dtype=np.float64)
    lse = np.zeros((ids.size,), dtype=np.float64)
    for b in np.unique(seq):
        lo, hi = int(cu[b]), int(cu[b + 1])
        sel = np.nonzero(seq == b)[0]
        per = lambda x: np.ascontiguousarray(x[lo:hi].transpose(1, 0, 2)[None])  # [1, heads, L, d]
        flat = head[sel] * (hi - lo) + (tok[sel] - lo)
        o[sel], lse[sel] = attention_rows(per(qa), per(ka), per(va), causal, scale, rows=flat, threads=threads)
    return o, lse


def attention_bwd_rows(q, k, v, dout, causal: bool, scale: float, q_rows=None, kv_rows=None,
                       threads: int | None = None, kv_len=None):
    """Gradients of the attention forward for an upstream gradient dout of o (none for lse).

    q, dout: [B, H, N, d]; k, v: [B, Hkv, N, d] (Hkv divides H); bf16/fp32 CPU tensors or fp32 arrays.
    q_rows: flat query rows (b*H + h)*N + i for dq, or None for every row; kv_rows: flat key rows
    (b*Hkv + g)*N + j for dk and dv, or None for every row (an empty list skips that part).
    kv_len: None, or B valid-key counts (the key-padding lengths of the forward, clamped to [0, N]).
    Returns (dq [n_q, d], dk [n_kv, d], dv [n_kv, d]) as float64 arrays.
    """
    qa, ka, va, da = _as_f32(q), _as_f32(k), _as_f32(v), _as_f32(dout)
    if (qa.ndim != 4 or da.shape != qa.shape or ka.shape != va.shape or ka.ndim != 4 or ka.shape[0] != qa.shape[0]
            or ka.shape[2:] != qa.shape[2:] or qa.shape[1] % ka.shape[1] != 0):
        raise ValueError(f"shapes disagree: q {qa.shape} k {ka.shape} v {va.shape} dout {da.shape}")
    B, H, N, d = qa.shape
    Hkv = ka.shape[1]

    def rows_arg(rows, total):
        if rows is None:
            return None, total
        arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
        return arr, int(arr.size)

    lens = None
    if kv_len is not None:
        lens = np.ascontiguousarray(np.asarray(kv_len, dtype=np.int32).reshape(-1))
        if lens.size != B:
            raise ValueError(f"kv_len needs {B} entries, got {lens.size}")
    qr, n_q = rows_arg(q_rows, B * H * N)
    kr, n_kv = rows_arg(kv_rows, B * Hkv * N)
    dq = np.zeros((n_q, d), dtype=np.float64)
    dk = np.zeros((n_kv, d), dtype=np.float64)
    dv = np.zeros((n_kv, d), dtype=np.float64)
    if n_q == 0 and n_kv == 0:
        return dq, dk, dv
    rc = _load().oracle_attn_bwd_rows(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, da.ctypes.data, B, H, Hkv, N, d,
                                      int(bool(causal)), float(np.float32(scale)),
                                      None if lens is None else lens.ctypes.data,
                                      None if qr is None else qr.ctypes.data, n_q,
                                      None if kr is None else kr.ctypes.data, n_kv,
                                      dq.ctypes.data, dk.ctypes.data, dv.ctypes.data,
                                      int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_bwd_rows failed with code {rc}")
    return dq, dk, dv


def attention_bwd(q, k, v, dout, causal: bool, scale: float, threads: int | None = None, kv_len=None):
    """Every gradient row: (dq [B,H,N,d], dk [B,Hkv,N,d], dv [B,Hkv,N,d]) as float64 arrays."""
    B, H, N, d = tuple(q.shape)
    Hkv = tuple(k.shape)[1]
    dq, dk, dv = attention_bwd_rows(q, k, v, dout, causal, scale, None, None, threads, kv_len)
    return dq.reshape(B, H, N, d), dk.reshape(B, Hkv, N, d), dv.reshape(B, Hkv, N, d)


def attention_bwd_varlen(q, k, v, dout, cu_seqlens, causal: bool, scale: float, threads: int | None = None):
    """Gradients of attention_varlen for an upstream gradient dout [T, H, d] of o: every sequence's gradients are
    those of its own attention problem (attention_bwd on its [1, H, L, d] slice); sequences share nothing.
    Returns (dq [T, H, d], dk [T, Hkv, d], dv [T, Hkv, d]) as float64 arrays."""
    qa, ka, va, da = _as_f32(q), _as_f32(k), _as_f32(v), _as_f32(dout)
    if qa.ndim != 3 or da.shape != qa.shape or ka.shape != va.shape or ka.ndim != 3 or ka.shape[0] != qa.shape[0] \
            or ka.shape[2] != qa.shape[2] or qa.shape[1] % ka.shape[1] != 0:
        raise ValueError(f"q, dout [T,H,d] and k, v [T,Hkv,d] disagree: {qa.shape} {ka.shape} {da.shape}")
    T = qa.shape[0]
    cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
    if cu.size < 1 or cu[0] != 0 or cu[-1] != T or (np.diff(cu) < 0).any():
        raise ValueError(f"cu_seqlens must rise from 0 to {T}: {cu}")
    dq, dk, dv = np.zeros(qa.shape), np.zeros(ka.shape), np.zeros(ka.shape)
    for b in range(cu.size - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi == lo:
            continue
        per = lambda x: np.ascontiguousarray(x[lo:hi].transpose(1, 0, 2)[None])  # [1, heads, L, d]
        gq, gk, gv = attention_bwd(per(qa), per(ka), per(va), per(da), causal, scale, threads)
        dq[lo:hi], dk[lo:hi], dv[lo:hi] = (g[0].transpose(1, 0, 2) for g in (gq, gk, gv))
    return dq, dk, dv


def attention_fp8_rows(q8, k8, v8, q_scale: float, k_scale: float, v_scale: float, causal: bool, scale: float,
                       rows=None, threads: int | None = None):
    """Attention of per-tensor-scaled fp8 inputs: the real inputs are q8 * q_scale, k8 * k_scale, v8 * v_scale.

    q8, k8, v8: [B, H, N, d] torch float8_e4m3fn CPU tensors (v not transposed). Every fp8 value is exact in
    fp32; the score scale scale * q_scale * k_scale (the fp32 values handed to the GPU, multiplied in fp64) is
    applied to the raw fp8 dot products, and o is multiplied by v_scale (attention is linear in v).
    Returns (o [n_rows, d] float64, lse [n_rows] float64).
    """
    qa, ka, va = _as_f32(q8), _as_f32(k8), _as_f32(v8)
    if qa.ndim != 4 or qa.shape != ka.shape or ka.shape != va.shape:
        raise ValueError(f"q, k, v must all be [B,H,N,d]: {qa.shape} {ka.shape} {va.shape}")
    f32 = lambda x: float(np.float32(x))
    sc = f32(scale) * f32(q_scale) * f32(k_scale)
    o, lse = _rows_exact_scale(qa, ka, va, causal, sc, rows, threads, None)
    return o * f32(v_scale), lse
