"""Pins for the oracle's grouped/multi-query heads and key-padding lengths.

Grouped-query and multi-query attention are named on the unite.ai page "Flash
Attention: revolutionizing transformer efficiency" (section "FlashAttention-2",
item 3) without a definition; the reading pinned here is that the H/Hkv
consecutive query heads of a group share one key/value head. The key-padding
mask appears as a boolean (batch, seq) mask in the triton-transformer README's
usage example ("ex. BERT"); the reading pinned here is a prefix of valid keys
per batch (right padding). Each pin below fails for a plausible slip: the
grouping taken modulo Hkv instead of by division, the length applied per head
instead of per batch, an off-by-one at the length, a length that also hides
query rows, or an empty softmax that turns into NaN.
"""
import math

import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle


def _brute(q, k, v, causal, scale, kv_len=None):
    """Pure-Python definition with exactly rounded sums; k, v may have fewer heads than q."""
    B, H, N, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    qd, kd, vd = (x.to(torch.float64).numpy() for x in (q, k, v))
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        L = Nk if kv_len is None else int(kv_len[b])
        for h in range(H):
            g = (h * Hkv) // H  # the group of h: H/Hkv consecutive query heads per key/value head
            for i in range(N):
                js = [j for j in range(L) if (not causal or j <= i)]
                if not js:
                    lse[b, h, i] = -math.inf
                    continue
                s = [scale * math.fsum(float(qd[b, h, i, c]) * float(kd[b, g, j, c]) for c in range(d)) for j in js]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                tot = math.fsum(w)
                for c in range(d):
                    o[b, h, i, c] = math.fsum(wj * float(vd[b, g, j, c]) for wj, j in zip(w, js)) / tot
                lse[b, h, i] = m + math.log(tot)
    return o, lse


def _qkv(B, H, Hkv, N, d, seed, dtype="f32"):
    q, _, _ = ai.make_qkv(B, H, N, d, seed, dtype)
    _, k, v = ai.make_qkv(B, Hkv, N, d, seed + 1, dtype)
    return q, k, v


@pytest.mark.parametrize("B,H,Hkv,N,d", [(1, 4, 2, 6, 3), (2, 3, 1, 5, 4), (2, 6, 3, 7, 2), (1, 2, 2, 4, 5)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_brute_force_tiny(B, H, Hkv, N, d, causal):
    q, k, v = _qkv(B, H, Hkv, N, d, seed=21)
    o, lse = oracle.attention(q, k, v, causal, 0.41, threads=3)
    ob, lb = _brute(q, k, v, causal, float(np.float32(0.41)))
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)


@pytest.mark.parametrize("kv_len", [[0, 3], [5, 1], [2, 5], [4, 4]])
@pytest.mark.parametrize("causal", [False, True])
def test_kpad_brute_force_tiny(kv_len, causal):
    q, k, v = _qkv(2, 4, 2, 5, 3, seed=23)
    o, lse = oracle.attention(q, k, v, causal, 0.7, threads=2, kv_len=kv_len)
    ob, lb = _brute(q, k, v, causal, float(np.float32(0.7)), kv_len)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-13)


@pytest.mark.parametrize("H,Hkv", [(8, 2), (8, 1), (6, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_matches_sdpa_fp64(H, Hkv, causal):
    """torch's own grouped attention (enable_gqa) on the CPU in fp64 is an independent opinion of the grouping."""
    N, d = 150, 64
    q, k, v = _qkv(2, H, Hkv, N, d, seed=31, dtype="bf16")
    scale = ai.default_scale(d)
    o, lse = oracle.attention(q, k, v, causal, scale)
    qd, kd, vd = (x.to(torch.float64) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, is_causal=causal, scale=scale,
                                                           enable_gqa=True).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_kpad_matches_sdpa_with_boolean_mask(causal):
    """A boolean key mask (True = attend) in torch's SDPA, fp64 on the CPU, with the scores' logsumexp by scipy."""
    from scipy.special import logsumexp

    B, H, N, d = 3, 2, 97, 64
    lens = [97, 40, 1]
    q, k, v = ai.make_qkv(B, H, N, d, seed=33, dtype="bf16")
    scale = ai.default_scale(d)
    o, lse = oracle.attention(q, k, v, causal, scale, kv_len=lens)
    keep = torch.zeros((B, 1, N, N), dtype=torch.bool)
    for b, L in enumerate(lens):
        keep[b, :, :, :L] = True
    if causal:
        keep &= torch.tril(torch.ones((N, N), dtype=torch.bool))
    qd, kd, vd = (x.to(torch.float64) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, attn_mask=keep, scale=scale).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    scores = np.where(keep.numpy(), np.einsum("bhic,bhjc->bhij", qd.numpy(), kd.numpy()) * scale, -np.inf)
    np.testing.assert_allclose(lse, logsumexp(scores, axis=-1), rtol=0, atol=1e-12)


def test_gqa_equals_attention_with_repeated_heads():
    """Each query head of a group attends exactly as it would to its own copy of the group's key/value head."""
    B, H, Hkv, N, d = 2, 8, 2, 70, 64
    q, k, v = _qkv(B, H, Hkv, N, d, seed=35, dtype="bf16")
    scale = ai.default_scale(d)
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, causal, scale)
        rep = H // Hkv
        kr = torch.cat([k[:, g:g + 1].expand(B, rep, N, d) for g in range(Hkv)], dim=1).contiguous()
        vr = torch.cat([v[:, g:g + 1].expand(B, rep, N, d) for g in range(Hkv)], dim=1).contiguous()
        o2, lse2 = oracle.attention(q, kr, vr, causal, scale)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_kpad_equals_attention_over_the_valid_prefix():
    """A batch with L valid keys gives exactly the attention over k[:L], v[:L] (non-causal)."""
    B, H, N, d = 3, 2, 90, 64
    lens = [90, 33, 64]
    q, k, v = ai.make_qkv(B, H, N, d, seed=37, dtype="bf16")
    scale = ai.default_scale(d)
    o, lse = oracle.attention(q, k, v, False, scale, kv_len=lens)
    for b, L in enumerate(lens):
        ob, lb = oracle.attention(q[b:b + 1], k[b:b + 1, :, :L].contiguous(), v[b:b + 1, :, :L].contiguous(),
                                  False, scale)
        assert np.array_equal(o[b:b + 1], ob) and np.array_equal(lse[b:b + 1], lb)


@pytest.mark.parametrize("causal", [False, True])
def test_padded_keys_do_not_matter(causal):
    B, H, N, d = 2, 2, 80, 64
    lens = [50, 7]
    q, k, v = ai.make_qkv(B, H, N, d, seed=39, dtype="bf16")
    scale = ai.default_scale(d)
    o, lse = oracle.attention(q, k, v, causal, scale, kv_len=lens)
    k2, v2 = k.clone(), v.clone()
    for b, L in enumerate(lens):
        k2[b, :, L:] = 1e3
        v2[b, :, L:] = -7.0
    o2, lse2 = oracle.attention(q, k2, v2, causal, scale, kv_len=lens)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_length_batch_is_empty_softmax(causal):
    """No visible key: the sum of weights is empty, so o = 0 and lse = ln 0 = -inf; other batches unaffected."""
    B, H, N, d = 2, 2, 33, 64
    q, k, v = ai.make_qkv(B, H, N, d, seed=41, dtype="bf16")
    scale = ai.default_scale(d)
    o, lse = oracle.attention(q, k, v, causal, scale, kv_len=[0, N])
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    o_full, lse_full = oracle.attention(q, k, v, causal, scale)
    assert np.array_equal(o[1], o_full[1]) and np.array_equal(lse[1], lse_full[1])


def test_zero_query_with_padding_is_prefix_mean():
    """q = 0: every visible key has the same score, so o is the mean of the visible values, lse = ln(count)."""
    B, H, N, d = 2, 4, 40, 64
    lens = [25, 40]
    _, k, v = _qkv(B, H, 2, N, d, seed=43, dtype="bf16")
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
    o, lse = oracle.attention(q, k, v, True, ai.default_scale(d), kv_len=lens)
    vd = v.to(torch.float64).numpy()
    for b, L in enumerate(lens):
        for h in range(H):
            g = h // 2
            for i in range(N):
                n = min(i + 1, L)
                np.testing.assert_allclose(o[b, h, i], vd[b, g, :n].mean(axis=0), rtol=0, atol=1e-13)
                assert abs(lse[b, h, i] - math.log(n)) <= 1e-13


def test_bad_grouping_and_lengths_rejected():
    q, k, v = _qkv(1, 4, 3, 8, 4, seed=45)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, False, 1.0)  # 3 does not divide 4
    q, k, v = _qkv(2, 4, 2, 8, 4, seed=45)
    for bad in ([9, 1], [-1, 2], [1, 2, 3]):
        with pytest.raises(ValueError):
            oracle.attention(q, k, v, False, 1.0, kv_len=bad)
