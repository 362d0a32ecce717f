"""Pins for the oracle of packed variable-length batches (oracle.attention_varlen).

Batches of sequences with different lengths: the pages show only a boolean (batch, seq) mask in the
triton-transformer README's usage example ("ex. BERT"), i.e. padded batches. The reading
pinned here is FlashAttention-style packing: the tokens of B sequences lie back to back ([T, H, d]), sequence b
holds tokens cu[b] .. cu[b+1]-1, and its queries attend only to its own keys (causal: to those at or before their
own position in the sequence). The pins: torch SDPA in fp64 on the whole packed problem with a block-diagonal
boolean mask (no slicing involved), the plain oracle for one sequence, invariance to the order of the sequences,
and empty sequences.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import attn_inputs as ai
import oracle


def _packed(T, H, Hkv, d, seed):
    q, _, _ = ai.make_qkv(1, H, T, d, seed, "bf16")
    _, k, v = ai.make_qkv(1, Hkv, T, d, seed + 1, "bf16")
    # [1, H, T, d] -> [T, H, d]
    return tuple(x[0].transpose(0, 1).contiguous() for x in (q, k, v))


def _block_mask(cu, causal):
    T = int(cu[-1])
    seq = np.searchsorted(cu, np.arange(T), side="right") - 1
    keep = seq[:, None] == seq[None, :]
    if causal:
        keep &= np.tril(np.ones((T, T), dtype=bool))
    return keep


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 1)])
def test_varlen_matches_sdpa_with_a_block_diagonal_mask(H, Hkv, causal):
    cu = np.array([0, 37, 38, 100, 100, 163])  # lengths 37, 1, 62, 0, 63
    T, d = int(cu[-1]), 64
    q, k, v = _packed(T, H, Hkv, d, seed=31)
    scale = ai.default_scale(d)
    o, lse = oracle.attention_varlen(q, k, v, cu, causal, scale)
    keep = torch.from_numpy(_block_mask(cu, causal))
    qd, kd, vd = (x.to(torch.float64).transpose(0, 1)[None] for x in (q, k, v))  # [1, heads, T, d]
    ref = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, attn_mask=keep, scale=float(np.float32(scale)),
                                                           enable_gqa=(H != Hkv))
    np.testing.assert_allclose(o.reshape(T, H, d), ref[0].transpose(0, 1).numpy(), rtol=0, atol=1e-12)
    kr = kd.repeat_interleave(H // Hkv, dim=1)
    s = (qd @ kr.transpose(-1, -2))[0].numpy() * float(np.float32(scale))
    s = np.where(keep.numpy()[None], s, -np.inf)
    np.testing.assert_allclose(lse.reshape(T, H), logsumexp(s, axis=-1).T, rtol=0, atol=1e-11)


def test_one_sequence_is_the_plain_forward():
    T, H, d = 90, 2, 64
    q, k, v = _packed(T, H, H, d, seed=33)
    for causal in (False, True):
        o, lse = oracle.attention_varlen(q, k, v, [0, T], causal, 0.125)
        o2, l2 = oracle.attention(q.transpose(0, 1)[None].contiguous(), k.transpose(0, 1)[None].contiguous(),
                                  v.transpose(0, 1)[None].contiguous(), causal, 0.125)
        np.testing.assert_array_equal(o.reshape(T, H, d), o2[0].transpose(1, 0, 2))
        np.testing.assert_array_equal(lse.reshape(T, H), l2[0].T)


def test_sequence_order_and_empty_sequences_do_not_matter():
    """Swapping two sequences in the packing moves their rows and changes nothing else; empty ones add nothing."""
    H, d = 2, 64
    la, lb = 41, 23
    q, k, v = _packed(la + lb, H, H, d, seed=35)
    o, lse = oracle.attention_varlen(q, k, v, [0, la, la + lb], True, 0.1)
    perm = torch.cat([torch.arange(la, la + lb), torch.arange(0, la)])
    o2, l2 = oracle.attention_varlen(q[perm], k[perm], v[perm], [0, 0, lb, lb, la + lb], True, 0.1)
    np.testing.assert_array_equal(o2.reshape(la + lb, H, d), o.reshape(la + lb, H, d)[perm.numpy()])
    np.testing.assert_array_equal(l2.reshape(la + lb, H), lse.reshape(la + lb, H)[perm.numpy()])


def test_row_lists_and_bad_offsets():
    T, H, d = 50, 2, 64
    q, k, v = _packed(T, H, H, d, seed=37)
    cu = [0, 20, 50]
    o, lse = oracle.attention_varlen(q, k, v, cu, False, 0.2)
    rows = np.array([0, 1, 39, 40, 99])
    o_s, l_s = oracle.attention_varlen(q, k, v, cu, False, 0.2, rows=rows)
    np.testing.assert_array_equal(o_s, o[rows])
    np.testing.assert_array_equal(l_s, lse[rows])
    for bad in ([1, 50], [0, 30, 20, 50], [0, 49]):
        with pytest.raises(ValueError):
            oracle.attention_varlen(q, k, v, bad, False, 0.2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 1)])
def test_varlen_gradients_match_autograd_with_a_block_diagonal_mask(H, Hkv, causal):
    """fp64 autograd of SDPA on the whole packed problem with the block-diagonal mask (every row of a non-empty
    sequence sees at least its first key, so no row of the masked softmax is empty)."""
    cu = np.array([0, 37, 38, 100, 100, 163])
    T, d = int(cu[-1]), 64
    q, k, v = _packed(T, H, Hkv, d, seed=41)
    g = torch.Generator("cpu").manual_seed(42)
    dout = torch.randn((T, H, d), generator=g).to(torch.bfloat16)
    scale = ai.default_scale(d)
    dq, dk, dv = oracle.attention_bwd_varlen(q, k, v, dout, cu, causal, scale)
    keep = torch.from_numpy(_block_mask(cu, causal))
    qd, kd, vd = (x.to(torch.float64).transpose(0, 1)[None].clone().requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, attn_mask=keep, scale=float(np.float32(scale)),
                                                         enable_gqa=(H != Hkv))
    o.backward(dout.to(torch.float64).transpose(0, 1)[None])
    for got, ref in ((dq, qd), (dk, kd), (dv, vd)):
        np.testing.assert_allclose(got, ref.grad[0].transpose(0, 1).numpy(), rtol=0, atol=1e-12)
