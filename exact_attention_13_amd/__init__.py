"""Exact fused attention for AMD MI355X (gfx950): a C-ABI HIP library and its Python binding.

    from exact_attention_13_amd import attention, backward, forward
    o, lse = forward(q, k, v, causal=True)
    dq, dk, dv = backward(q, k, v, o, lse, dout, causal=True)
    o = attention(q, k, v, causal=True)   # differentiable: o.backward(dout) fills q.grad, k.grad, v.grad

The library (libfa.so, built from csrc/ by `python exact_attention_13_amd/build.py`) exports fa_fwd,
fa_fwd_gqa, fa_fwd_kpad, fa_fwd_varlen, fa_fwd_fp8, fa_bwd, fa_bwd_noalloc, fa_bwd_kpad, fa_bwd_varlen,
fa_bwd_workspace_bytes, fa_fwd_f32, fa_fwd_instance, fa_strerror and fa_version (include/fa.h). Importing this package fails if it is not built.
"""
from .binding import (EXPORTS, FA_ERR_ALIAS, FA_ERR_ALIGN, FA_ERR_ARG, FA_ERR_HEADDIM, FA_ERR_HIP, FA_ERR_NULL,
                      FA_ERR_SCRATCH, FA_ERR_SHAPE, FA_OK, fa_bwd, fa_bwd_kpad, fa_bwd_noalloc, fa_bwd_varlen,
                      fa_bwd_workspace_bytes, fa_fwd, fa_fwd_f32, fa_fwd_fp8, fa_fwd_gqa, fa_fwd_instance, fa_fwd_kpad,
                      fa_fwd_varlen, fa_strerror, fa_version, library_path)
from .attention import (attention, attention_varlen, backward, backward_varlen, forward, forward_fp8,
                        forward_varlen)

__all__ = ["attention", "attention_varlen", "forward", "forward_fp8", "forward_varlen", "backward", "backward_varlen",
           "fa_fwd", "fa_fwd_gqa", "fa_fwd_kpad", "fa_fwd_varlen", "fa_fwd_fp8", "fa_fwd_f32", "fa_bwd",
           "fa_bwd_noalloc", "fa_bwd_kpad", "fa_bwd_varlen", "fa_bwd_workspace_bytes", "fa_fwd_instance",
           "fa_strerror", "fa_version", "library_path", "EXPORTS", "FA_OK", "FA_ERR_NULL", "FA_ERR_SHAPE",
           "FA_ERR_HEADDIM", "FA_ERR_ALIGN", "FA_ERR_ARG", "FA_ERR_ALIAS", "FA_ERR_HIP", "FA_ERR_SCRATCH"]
