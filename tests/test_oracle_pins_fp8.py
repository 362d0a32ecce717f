"""Pins for the oracle of the fp8 attention forward (oracle.attention_fp8_rows).

The unite.ai page "Flash Attention: revolutionizing transformer efficiency" lists FP8 among the
FlashAttention-3 techniques (section "FlashAttention-3", items 2-3) without a method or a tolerance. The reading
pinned here: q, k, v arrive as float8_e4m3fn values with one fp32 scale per tensor, and the operation is exact
attention of the real inputs x8 * s_x. The oracle decodes fp8 exactly, applies scale * s_q * s_k to the raw dot
products and multiplies o by s_v. The pins: the e4m3fn decode written out from the format's definition, torch
SDPA in fp64 on the dequantized inputs, and the scale identities.
"""
import math

import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle


def _decode_e4m3fn(byte: int) -> float:
    """The float8_e4m3fn format: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is subnormal
    (mantissa * 2^-9); S.1111.111 is NaN; there is no infinity."""
    sign = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def test_fp8_decode_matches_the_format_definition():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    got = oracle._as_f32(codes.view(torch.float8_e4m3fn))
    ref = np.array([_decode_e4m3fn(c) for c in range(256)], dtype=np.float64)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok].astype(np.float64), ref[ok])
    assert np.nanmax(np.abs(ref)) == ai.FP8_MAX


def test_quantized_inputs_round_to_nearest_even_and_use_the_range():
    q, k, v = ai.make_qkv(1, 2, 64, 64, seed=9, dtype="f32")
    q8, k8, v8, sq, sk, sv = ai.make_qkv_fp8(1, 2, 64, 64, seed=9)
    for x, x8, s in ((q, q8, sq), (k, k8, sk), (v, v8, sv)):
        assert s == float(np.float32(s)) and s > 0
        dec = x8.float().numpy().astype(np.float64)
        assert np.abs(dec).max() <= ai.FP8_MAX and np.abs(dec).max() >= ai.FP8_MAX / 2
        # round to nearest: the decoded value is within half a step (2^-4 relative, 2^-10 absolute) of x / s
        t = (x / s).numpy().astype(np.float64)
        assert np.all(np.abs(dec - t) <= np.maximum(np.abs(t) * 2.0 ** -4, 2.0 ** -10) + 1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_oracle_matches_sdpa_on_dequantized_inputs(causal):
    B, H, N, d = 1, 2, 150, 64
    q8, k8, v8, sq, sk, sv = ai.make_qkv_fp8(B, H, N, d, seed=13)
    scale = ai.default_scale(d)
    o, lse = oracle.attention_fp8_rows(q8, k8, v8, sq, sk, sv, causal, scale)
    deq = [x.to(torch.float64) * s for x, s in ((q8, sq), (k8, sk), (v8, sv))]
    ref = torch.nn.functional.scaled_dot_product_attention(*deq, is_causal=causal, scale=scale).numpy()
    np.testing.assert_allclose(o.reshape(ref.shape), ref, rtol=0, atol=1e-12)
    from scipy.special import logsumexp
    s = np.einsum("bhic,bhjc->bhij", deq[0].numpy(), deq[1].numpy()) * scale
    if causal:
        s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
    np.testing.assert_allclose(lse.reshape(B, H, N), logsumexp(s, axis=-1), rtol=0, atol=1e-11)


def test_fp8_scale_identities():
    """o is linear in the v scale; only the product of the q and k scales matters."""
    q8, k8, v8, sq, sk, sv = ai.make_qkv_fp8(1, 1, 60, 64, seed=15)
    o1, l1 = oracle.attention_fp8_rows(q8, k8, v8, sq, sk, sv, True, 0.125)
    o2, l2 = oracle.attention_fp8_rows(q8, k8, v8, sq * 2, sk / 2, sv * 4, True, 0.125)
    np.testing.assert_allclose(o2, 4 * o1, rtol=1e-15, atol=0)
    np.testing.assert_allclose(l2, l1, rtol=1e-15, atol=0)
