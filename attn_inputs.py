"""Seeded synthetic inputs for the exact attention forward.

This module is shared by both sides of every parity check (the fp64 CPU oracle
and the HIP path). It only draws Q, K, V and picks which query rows a check
samples; it contains none of the attention arithmetic.

Recipe (one workload = B, H, N, d, causal, dtype, seed):
  g = torch.Generator('cpu').manual_seed(seed)
  q = torch.randn((B, H, N, d), generator=g, dtype=float32), then k and v likewise with shape
  (B, Hkv, N, d) (Hkv = H unless the workload has grouped key/value heads), in that order
  k *= k_scale        (3.0 for the peaked-softmax workload, in fp32, before rounding)
  round to bf16 with round-to-nearest-even (fp32 workloads stay fp32)
Layout is [B, H, N, d], contiguous, row-major. The default softmax scale is
1/sqrt(d) rounded to fp32: the standard attention code on the unite.ai page
("Flash Attention: revolutionizing transformer efficiency", opening code block)
divides the scores by the square root of the head width.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    dtype: str          # "bf16", "f32" or "fp8" (float8_e4m3fn q, k, v with per-tensor scales)
    seed: int
    k_scale: float = 1.0
    sampled_rows: int = 0   # 0: every row is checked; else rows sampled per check
    Hkv: int = 0            # key/value heads (grouped-query attention); 0: same as H
    kv_len: tuple = ()      # per-batch valid-key counts (key padding); (): every key valid

    @property
    def Hk(self) -> int:
        return self.Hkv or self.H

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    def _pairs(self, L: int) -> float:
        """Visible (query, key) pairs of one head with L valid keys, in the metric's convention: N*L, or for
        causal L^2/2 (the triangle, counted as the metric counts N^2/2) plus (N - L)*L (the rows past it)."""
        return L * L / 2 + (self.N - L) * L if self.causal else float(self.N * L)

    @property
    def flops(self) -> float:
        """Attention-forward FLOPs as the metric counts them: 4*B*H*N^2*d, halved when causal; with key padding
        4*H*d times the visible pairs of every batch."""
        lens = self.kv_len or (self.N,) * self.B
        return 4.0 * self.H * self.d * sum(self._pairs(L) for L in lens)

    @property
    def elt_bytes(self) -> int:
        return {"bf16": 2, "f32": 4, "fp8": 1}[self.dtype]

    @property
    def kv_rows(self) -> int:
        """Key/value rows the kernel must read: B*Hkv*N, or only the valid ones with key padding."""
        return self.Hk * (sum(self.kv_len) if self.kv_len else self.B * self.N)

    @property
    def algorithmic_bytes(self) -> int:
        """Q read once, valid K and V rows read once, O written once (input dtype; bf16 for fp8 inputs); lse
        written once (fp32)."""
        n = self.B * self.H * self.N
        out = 2 if self.dtype == "fp8" else self.elt_bytes
        return (n + 2 * self.kv_rows) * self.d * self.elt_bytes + n * self.d * out + 4 * n


# The workloads: seed = workload number; C2 has a causal and a non-causal variant.
WORKLOADS = {
    "c1_f32_b1h1n128d64": Workload("c1_f32_b1h1n128d64", 1, 1, 128, 64, False, "f32", 1),
    "c2n_bf16_b4h8n1024d64": Workload("c2n_bf16_b4h8n1024d64", 4, 8, 1024, 64, False, "bf16", 2),
    "c2c_bf16_b4h8n1024d64_causal": Workload("c2c_bf16_b4h8n1024d64_causal", 4, 8, 1024, 64, True, "bf16", 2),
    "c3_bf16_b2h16n4096d128": Workload("c3_bf16_b2h16n4096d128", 2, 16, 4096, 128, False, "bf16", 3),
    "c4_bf16_b1h32n16384d128_causal": Workload("c4_bf16_b1h32n16384d128_causal", 1, 32, 16384, 128, True, "bf16", 4,
                                               sampled_rows=256),
    "c5_bf16_b1h8n32768d64_causal_k3": Workload("c5_bf16_b1h8n32768d64_causal_k3", 1, 8, 32768, 64, True, "bf16", 5,
                                                k_scale=3.0, sampled_rows=256),
    # Grouped-query attention (8 key/value heads for 32 query heads) at the headline sequence length, and
    # multi-query attention (1 for 32) at the long causal one.
    "gqa_bf16_b2h32kv8n4096d128": Workload("gqa_bf16_b2h32kv8n4096d128", 2, 32, 4096, 128, False, "bf16", 6,
                                           sampled_rows=256, Hkv=8),
    "mqa_bf16_b1h32kv1n16384d128_causal": Workload("mqa_bf16_b1h32kv1n16384d128_causal", 1, 32, 16384, 128, True,
                                                   "bf16", 7, sampled_rows=256, Hkv=1),
    # Key padding: 8 right-padded sequences of mixed lengths in a batch padded to N = 4096 (encoder-style,
    # non-causal, as in the boolean-mask usage example of the triton-transformer README).
    "kpad_bf16_b8h16n4096d128": Workload("kpad_bf16_b8h16n4096d128", 8, 16, 4096, 128, False, "bf16", 8,
                                         sampled_rows=256, kv_len=(4096, 3001, 2500, 4000, 1234, 777, 3333, 2048)),
}


@dataclass(frozen=True)
class VarlenWorkload:
    """Packed variable-length batch: B = len(lens) sequences back to back, q [T, H, d], k and v [T, Hkv, d]."""
    name: str
    lens: tuple
    H: int
    d: int
    causal: bool
    seed: int
    Hkv: int = 0
    sampled_rows: int = 256

    @property
    def B(self) -> int:
        return len(self.lens)

    @property
    def T(self) -> int:
        return sum(self.lens)

    @property
    def max_len(self) -> int:
        return max(self.lens)

    @property
    def Hk(self) -> int:
        return self.Hkv or self.H

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    @property
    def cu_seqlens(self) -> list:
        return [0] + list(np.cumsum(self.lens).tolist())

    @property
    def flops(self) -> float:
        """4*H*d per visible (query, key) pair of every sequence; causal triangles counted as L^2/2."""
        return 4.0 * self.H * self.d * sum(L * L / 2 if self.causal else float(L * L) for L in self.lens)

    @property
    def algorithmic_bytes(self) -> int:
        """q, k, v read once, o written once (bf16), lse written once (fp32)."""
        return 2 * self.T * self.d * (2 * self.H + 2 * self.Hk) + 4 * self.T * self.H


# Packed batches: the key-padding lengths without the padding (encoder-style), and a causal mix of short and
# long sequences with grouped heads (decoder-style).
VARLEN_WORKLOADS = {
    "varlen_bf16_b8h16d128": VarlenWorkload("varlen_bf16_b8h16d128", (4096, 3001, 2500, 4000, 1234, 777, 3333, 2048),
                                           16, 128, False, 9),
    "varlen_bf16_b12h32kv8d128_causal": VarlenWorkload(
        "varlen_bf16_b12h32kv8d128_causal", (8192, 512, 3000, 1, 6000, 4096, 777, 2048, 5555, 64, 100, 1900),
        32, 128, True, 10, Hkv=8),
}


def make_qkv_varlen(lens, H: int, d: int, seed: int, Hkv: int | None = None):
    """Packed inputs of sum(lens) tokens: q [T, H, d] and k, v [T, Hkv, d] ~ N(0, 1) in fp32 (CPU generator, drawn
    in that order), rounded to bf16. Returns CPU tensors."""
    T = int(sum(lens))
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn((T, H, d), generator=g, dtype=torch.float32)
    k = torch.randn((T, Hkv or H, d), generator=g, dtype=torch.float32)
    v = torch.randn((T, Hkv or H, d), generator=g, dtype=torch.float32)
    return tuple(x.to(torch.bfloat16).contiguous() for x in (q, k, v))


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded to fp32 (the value handed to both sides)."""
    return float(np.float32(1.0 / math.sqrt(d)))


def make_qkv(B: int, H: int, N: int, d: int, seed: int, dtype: str = "bf16", k_scale: float = 1.0,
             Hkv: int | None = None):
    """Draw q [B,H,N,d] and k, v [B,Hkv,N,d] ~ N(0, 1) in fp32 (CPU generator), scale k, round to dtype.
    Returns CPU tensors. Hkv defaults to H."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    kv_shape = (B, Hkv or H, N, d)
    q = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
    k = torch.randn(kv_shape, generator=g, dtype=torch.float32)
    v = torch.randn(kv_shape, generator=g, dtype=torch.float32)
    if k_scale != 1.0:
        k = k * float(k_scale)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    return q.to(tdt).contiguous(), k.to(tdt).contiguous(), v.to(tdt).contiguous()


FP8_MAX = 448.0  # largest finite float8_e4m3fn value


def make_qkv_fp8(B: int, H: int, N: int, d: int, seed: int, k_scale: float = 1.0):
    """The same fp32 draws as make_qkv, quantized per tensor to float8_e4m3fn (round-to-nearest-even):
    s_x = max|x| / 448 rounded to fp32, x8 = x / s_x. Returns (q8, k8, v8, s_q, s_k, s_v); the real inputs the
    fp8 path is given are x8 * s_x."""
    q, k, v = make_qkv(B, H, N, d, seed, "f32", k_scale)
    out, scales = [], []
    for x in (q, k, v):
        s = float(np.float32(float(x.abs().max()) / FP8_MAX))
        out.append((x / s).to(torch.float8_e4m3fn).contiguous())
        scales.append(s)
    return (*out, *scales)


def make_workload(w: Workload):
    return make_qkv(w.B, w.H, w.N, w.d, w.seed, w.dtype, w.k_scale, w.Hkv or None)


def kv_len_of(w: Workload):
    """The workload's per-batch valid-key counts as a list, or None without key padding."""
    return list(w.kv_len) if w.kv_len else None


def sample_rows(B: int, H: int, N: int, n: int, seed: int) -> np.ndarray:
    """n distinct flat row ids (b*H + h)*N + i, uniform without replacement, seeded with seed+1000."""
    total = B * H * N
    n = min(n, total)
    g = torch.Generator("cpu").manual_seed(int(seed) + 1000)
    return torch.randperm(total, generator=g)[:n].numpy().astype(np.int64)


def edge_rows(N: int, Br: int = 128, Bc: int = 64) -> np.ndarray:
    """Fixed rows of head 0 at tile edges: first, last, and around one Q block and one KV tile."""
    cand = [0, 1, Br - 1, Br, N // 2, N - Bc, N - 2, N - 1]
    return np.array(sorted({i for i in cand if 0 <= i < N}), dtype=np.int64)


def check_rows(w: Workload) -> np.ndarray | None:
    """Rows a parity check compares: None (all rows) or the sampled set plus the edge rows."""
    if not w.sampled_rows:
        return None
    r = np.concatenate([sample_rows(w.B, w.H, w.N, w.sampled_rows, w.seed), edge_rows(w.N)])
    return np.unique(r)


def sha256(*tensors: torch.Tensor) -> str:
    h = hashlib.sha256()
    for t in tensors:
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()
