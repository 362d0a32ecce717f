"""ctypes binding of libfa.so: the same entry points as include/fa.h, argument marshalling only.

Every step of the attention forward runs in the library's HIP kernel. PyTorch only provides device
buffers and the current stream. If libfa.so is missing this module raises at import time: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

# PyTorch ships its own HIP runtime (libamdhip64.so, soname libamdhip64.so.7). Importing torch first makes
# libfa.so's libamdhip64.so.7 dependency resolve to that same copy; loading libfa.so first would map a second
# HIP runtime into the process, and torch's streams and device pointers would then be handed to the wrong one.
import torch  # noqa: F401  (load order matters, see above)

_LIB_PATH = Path(__file__).resolve().parent / "libfa.so"

FA_OK = 0
FA_ERR_NULL = 1
FA_ERR_SHAPE = 2
FA_ERR_HEADDIM = 3
FA_ERR_ALIGN = 4
FA_ERR_ARG = 5
FA_ERR_ALIAS = 6
FA_ERR_HIP = 7
FA_ERR_SCRATCH = 8

EXPORTS = ("fa_fwd", "fa_fwd_gqa", "fa_fwd_kpad", "fa_fwd_varlen", "fa_fwd_fp8", "fa_bwd", "fa_bwd_noalloc", "fa_bwd_kpad",
           "fa_bwd_varlen", "fa_bwd_workspace_bytes", "fa_fwd_f32", "fa_fwd_instance", "fa_strerror", "fa_version")

if not _LIB_PATH.exists():
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python exact_attention_13_amd/build.py` "
                      "(the attention forward has no other implementation)")
_lib = ctypes.CDLL(str(_LIB_PATH))

_P = ctypes.c_void_p
_I = ctypes.c_int
_lib.fa_fwd.restype = _I
_lib.fa_fwd.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float, _P]
_lib.fa_fwd_gqa.restype = _I
_lib.fa_fwd_gqa.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P]
_lib.fa_fwd_kpad.restype = _I
_lib.fa_fwd_kpad.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P]
_lib.fa_fwd_varlen.restype = _I
_lib.fa_fwd_varlen.argtypes = [_P] * 6 + [_I] * 7 + [ctypes.c_float, _P]
_lib.fa_fwd_fp8.restype = _I
_lib.fa_fwd_fp8.argtypes = [_P] * 5 + [ctypes.c_float] * 3 + [_I] * 5 + [ctypes.c_float, _P]
_lib.fa_bwd.restype = _I
_lib.fa_bwd.argtypes = [_P] * 10 + [_I] * 6 + [ctypes.c_float, _P]
_lib.fa_bwd_noalloc.restype = _I
_lib.fa_bwd_noalloc.argtypes = [_P] * 9 + [_I] * 6 + [ctypes.c_float, _P]
_lib.fa_bwd_kpad.restype = _I
_lib.fa_bwd_kpad.argtypes = [_P] * 11 + [_I] * 6 + [ctypes.c_float, _P]
_lib.fa_bwd_varlen.restype = _I
_lib.fa_bwd_varlen.argtypes = [_P] * 11 + [_I] * 7 + [ctypes.c_float, _P]
_lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
_lib.fa_bwd_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
_lib.fa_fwd_f32.restype = _I
_lib.fa_fwd_f32.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float, _P]
_lib.fa_fwd_instance.restype = ctypes.c_char_p
_lib.fa_fwd_instance.argtypes = [_I] * 6
_lib.fa_strerror.restype = ctypes.c_char_p
_lib.fa_strerror.argtypes = [_I]
_lib.fa_version.restype = _I
_lib.fa_version.argtypes = []


def library_path() -> str:
    return str(_LIB_PATH)


def fa_fwd(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, d: int, causal: int, scale: float,
           stream: int) -> int:
    """Raw entry point: device pointers as ints, bf16 q/k/v/o, fp32 lse. Returns the FA_* code."""
    return _lib.fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, stream)


def fa_fwd_gqa(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, H_kv: int, N: int, d: int, causal: int,
               scale: float, stream: int) -> int:
    """Raw entry point: bf16 q/o [B,H,N,d], k/v [B,H_kv,N,d]; query head h reads key/value head h // (H // H_kv)."""
    return _lib.fa_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, causal, scale, stream)


def fa_fwd_kpad(q: int, k: int, v: int, o: int, lse: int, kv_len: int, B: int, H: int, H_kv: int, N: int, d: int,
                causal: int, scale: float, stream: int) -> int:
    """Raw entry point: fa_fwd_gqa plus kv_len, a device int32 [B] array of valid-key counts (key padding)."""
    return _lib.fa_fwd_kpad(q, k, v, o, lse, kv_len, B, H, H_kv, N, d, causal, scale, stream)


def fa_fwd_varlen(q: int, k: int, v: int, o: int, lse: int, cu_seqlens: int, B: int, H: int, H_kv: int, total: int,
                  max_seqlen: int, d: int, causal: int, scale: float, stream: int) -> int:
    """Raw entry point: packed sequences, bf16 q/o [total,H,d], k/v [total,H_kv,d], lse [H,total], cu_seqlens
    int32 [B+1] on the device."""
    return _lib.fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, H, H_kv, total, max_seqlen, d, causal, scale, stream)


def fa_fwd_fp8(q: int, k: int, vt: int, o: int, lse: int, q_scale: float, k_scale: float, v_scale: float, B: int,
               H: int, N: int, d: int, causal: int, scale: float, stream: int) -> int:
    """Raw entry point: float8_e4m3fn q, k [B,H,N,d] and vt [B,H,d,N] with per-tensor scales; bf16 o."""
    return _lib.fa_fwd_fp8(q, k, vt, o, lse, q_scale, k_scale, v_scale, B, H, N, d, causal, scale, stream)


def fa_bwd(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int, workspace: int, B: int,
           H: int, H_kv: int, N: int, d: int, causal: int, scale: float, stream: int) -> int:
    """Raw entry point: gradients dq [B,H,N,d], dk, dv [B,H_kv,N,d] (bf16) of the forward for upstream dout;
    workspace: fa_bwd_workspace_bytes(B, H, H_kv, N, d) bytes of device memory."""
    return _lib.fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, H_kv, N, d, causal, scale, stream)


def fa_bwd_noalloc(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int, B: int, H: int,
                   H_kv: int, N: int, d: int, causal: int, scale: float, stream: int) -> int:
    """Raw entry point: fa_bwd with the library's own scratch buffer as the workspace. Returns the FA_* code."""
    return _lib.fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, N, d, causal, scale, stream)


def fa_bwd_kpad(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int, workspace: int,
                kv_len: int, B: int, H: int, H_kv: int, N: int, d: int, causal: int, scale: float, stream: int) -> int:
    """Raw entry point: fa_bwd for a forward made with fa_fwd_kpad; kv_len is the same device int32 [B] array."""
    return _lib.fa_bwd_kpad(q, k, v, o, lse, dout, dq, dk, dv, workspace, kv_len, B, H, H_kv, N, d, causal, scale,
                            stream)


def fa_bwd_varlen(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int, workspace: int,
                  cu_seqlens: int, B: int, H: int, H_kv: int, total: int, max_seqlen: int, d: int, causal: int,
                  scale: float, stream: int) -> int:
    """Raw entry point: gradients of fa_fwd_varlen; workspace of fa_bwd_workspace_bytes(B, H, H_kv, max_seqlen,
    d) bytes."""
    return _lib.fa_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_seqlens, B, H, H_kv, total,
                              max_seqlen, d, causal, scale, stream)


def fa_bwd_workspace_bytes(B: int, H: int, H_kv: int, N: int, d: int) -> int:
    return int(_lib.fa_bwd_workspace_bytes(B, H, H_kv, N, d))


def fa_fwd_f32(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, d: int, causal: int,
               scale: float, stream: int) -> int:
    """Raw entry point: device pointers as ints, fp32 q/k/v/o and lse. Returns the FA_* code."""
    return _lib.fa_fwd_f32(q, k, v, o, lse, B, H, N, d, causal, scale, stream)


def fa_fwd_instance(B: int, H: int, N: int, d: int, causal: int, packed: int = 0) -> str | None:
    """Name of the bf16 forward kernel instance the library launches for these sizes (None if they are invalid)."""
    r = _lib.fa_fwd_instance(B, H, N, d, causal, packed)
    return None if r is None else r.decode()


def fa_strerror(code: int) -> str:
    return _lib.fa_strerror(code).decode()


def fa_version() -> int:
    return _lib.fa_version()
