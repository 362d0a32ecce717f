"""Pins for the fp64 oracle of the attention gradients (oracle/attn_bwd_oracle.c).

The pages name the faster backward pass and the recomputation of attention from
stored statistics (unite.ai page "Flash Attention: revolutionizing transformer
efficiency": key ideas after "Enter Flash Attention", item 2; "FlashAttention-2",
item 2) but print no formula, so the gradient oracle is pinned to facts outside
its own code: finite differences of the (separately pinned) forward oracle,
torch autograd in fp64, closed forms at q = 0 and with a single key, the zero
sum of dk over the keys, and the reduction of grouped heads to repeated heads.
Each catches a plausible slip: a dropped scale, dS without the D_i term, D_i
from the wrong row, a transposed product, the causal side, the group sum.
"""
import math

import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle


def _dout(B, H, N, d, seed, dtype="bf16"):
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
    return x.to({"bf16": torch.bfloat16, "f32": torch.float32}[dtype])


def _loss(q, k, v, dout, causal, scale):
    """L = sum dO * o with the forward oracle (fp64)."""
    o, _ = oracle.attention(q, k, v, causal, scale, threads=1)
    return float(np.sum(o * dout.to(torch.float64).numpy()))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Hkv,N,d", [(1, 2, 2, 5, 4), (1, 4, 2, 4, 3), (2, 2, 1, 3, 2)])
def test_matches_richardson_finite_differences_of_the_forward_oracle(B, H, Hkv, N, d, causal):
    """Every gradient entry against central differences of L = sum dO*o, Richardson-extrapolated (error O(h^4)).
    Inputs are bf16 values, so x +- 2^-8 and x +- 2^-9 are exact in the fp32 the forward oracle takes."""
    q, _, _ = ai.make_qkv(B, H, N, d, seed=51, dtype="bf16")
    _, k, v = ai.make_qkv(B, Hkv, N, d, seed=52, dtype="bf16")
    q, k, v = q.float(), k.float(), v.float()
    dout = _dout(B, H, N, d, seed=53, dtype="f32")
    scale = 0.6
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, causal, scale)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        flat = x.view(-1)
        fd = np.zeros(flat.numel())
        for e in range(flat.numel()):
            def central(h):
                x0 = float(flat[e])
                flat[e] = x0 + h
                up = _loss(q, k, v, dout, causal, scale)
                flat[e] = x0 - h
                dn = _loss(q, k, v, dout, causal, scale)
                flat[e] = x0
                return (up - dn) / (2 * h)
            fd[e] = (4 * central(2.0 ** -9) - central(2.0 ** -8)) / 3
        np.testing.assert_allclose(g.reshape(-1), fd, rtol=0, atol=2e-8, err_msg=f"d{name}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 1), (6, 3)])
def test_matches_torch_autograd_fp64(H, Hkv, causal):
    B, N, d = 2, 70, 64
    q, _, _ = ai.make_qkv(B, H, N, d, seed=55)
    _, k, v = ai.make_qkv(B, Hkv, N, d, seed=56)
    dout = _dout(B, H, N, d, seed=57)
    scale = ai.default_scale(d)
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, causal, scale)
    qd, kd, vd = (x.to(torch.float64).requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, is_causal=causal, scale=scale,
                                                         enable_gqa=(H != Hkv))
    o.backward(dout.to(torch.float64))
    np.testing.assert_allclose(dq, qd.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, kd.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, vd.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_closed_forms(causal):
    """q = 0: all visible scores equal, p_ij = 1/|J_i|. Then dk = scale*sum_i dS_ij q_i = 0 exactly, and
    dv_j = sum over the queries i that see j of dO_i / |J_i|."""
    B, H, N, d = 1, 2, 37, 64
    _, k, v = ai.make_qkv(B, H, N, d, seed=59)
    q = torch.zeros_like(k)
    dout = _dout(B, H, N, d, seed=60)
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, causal, ai.default_scale(d))
    assert np.all(dk == 0.0)
    do = dout.to(torch.float64).numpy()
    cnt = np.arange(1, N + 1) if causal else np.full(N, N)
    w = do / cnt[None, None, :, None]
    ref = np.flip(np.cumsum(np.flip(w, axis=2), axis=2), axis=2) if causal else np.broadcast_to(
        w.sum(axis=2, keepdims=True), w.shape)
    np.testing.assert_allclose(dv, ref, rtol=0, atol=1e-13)


def test_single_key_closed_form():
    """N = 1: p = 1, so dS = dP - D = dO.v - dO.v = 0 (dq = dk = 0) and dv = dO."""
    q, k, v = ai.make_qkv(2, 3, 1, 64, seed=61)
    dout = _dout(2, 3, 1, 64, seed=62)
    for causal in (False, True):
        dq, dk, dv = oracle.attention_bwd(q, k, v, dout, causal, 0.3)
        assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
        np.testing.assert_array_equal(dv, dout.to(torch.float64).numpy())


@pytest.mark.parametrize("causal", [False, True])
def test_dk_sums_to_zero_over_the_keys(causal):
    """sum_j dS_ij = sum_j p_ij dP_ij - D_i sum_j p_ij = D_i - D_i = 0, so sum_j dk_j = 0 for every head."""
    B, H, N, d = 2, 2, 90, 64
    q, k, v = ai.make_qkv(B, H, N, d, seed=63)
    dout = _dout(B, H, N, d, seed=64)
    _, dk, _ = oracle.attention_bwd(q, k, v, dout, causal, ai.default_scale(d))
    scale_ref = np.abs(dk).max()
    assert np.abs(dk.sum(axis=2)).max() <= 1e-12 * N * scale_ref


def test_grouped_heads_sum_the_gradients_of_repeated_heads():
    B, H, Hkv, N, d = 2, 6, 2, 40, 64
    q, _, _ = ai.make_qkv(B, H, N, d, seed=65)
    _, k, v = ai.make_qkv(B, Hkv, N, d, seed=66)
    dout = _dout(B, H, N, d, seed=67)
    for causal in (False, True):
        dq, dk, dv = oracle.attention_bwd(q, k, v, dout, causal, 0.125)
        kr = k.repeat_interleave(H // Hkv, dim=1).contiguous()
        vr = v.repeat_interleave(H // Hkv, dim=1).contiguous()
        dq2, dk2, dv2 = oracle.attention_bwd(q, kr, vr, dout, causal, 0.125)
        np.testing.assert_array_equal(dq, dq2)
        np.testing.assert_allclose(dk, dk2.reshape(B, Hkv, H // Hkv, N, d).sum(axis=2), rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv, dv2.reshape(B, Hkv, H // Hkv, N, d).sum(axis=2), rtol=0, atol=1e-13)


def test_row_lists_match_the_full_computation():
    B, H, Hkv, N, d = 1, 4, 2, 50, 64
    q, _, _ = ai.make_qkv(B, H, N, d, seed=69)
    _, k, v = ai.make_qkv(B, Hkv, N, d, seed=70)
    dout = _dout(B, H, N, d, seed=71)
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, True, 0.2)
    qr = np.array([0, 7, 49, 120, 199])
    kr = np.array([3, 50, 99])
    dq_s, dk_s, dv_s = oracle.attention_bwd_rows(q, k, v, dout, True, 0.2, q_rows=qr, kv_rows=kr)
    np.testing.assert_array_equal(dq_s, dq.reshape(-1, d)[qr])
    np.testing.assert_array_equal(dk_s, dk.reshape(-1, d)[kr])
    np.testing.assert_array_equal(dv_s, dv.reshape(-1, d)[kr])
    e_q, e_k, e_v = oracle.attention_bwd_rows(q, k, v, dout, True, 0.2, q_rows=[], kv_rows=kr)
    assert e_q.shape == (0, d) and np.array_equal(e_k, dk_s)


def test_scale_and_query_trade_off():
    """Doubling q and halving the scale leaves every score, p and dS unchanged: dv and dk (= scale/2 * dS * 2q)
    stay, dq (= scale/2 * dS * k, the gradient with respect to the doubled input) halves."""
    B, H, N, d = 1, 2, 30, 64
    q, k, v = ai.make_qkv(B, H, N, d, seed=73, dtype="f32")
    dout = _dout(B, H, N, d, seed=74, dtype="f32")
    dq1, dk1, dv1 = oracle.attention_bwd(q, k, v, dout, True, 0.25)
    dq2, dk2, dv2 = oracle.attention_bwd(q * 2, k, v, dout, True, 0.125)
    np.testing.assert_allclose(dv2, dv1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk2, dk1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq2, dq1 / 2, rtol=0, atol=1e-13)


def test_bad_arguments_rejected():
    q, k, v = ai.make_qkv(1, 2, 8, 4, seed=75, dtype="f32")
    dout = _dout(1, 2, 8, 4, seed=76, dtype="f32")
    with pytest.raises(RuntimeError):
        oracle.attention_bwd_rows(q, k, v, dout, False, 1.0, q_rows=[16])
    with pytest.raises(RuntimeError):
        oracle.attention_bwd_rows(q, k, v, dout, False, 1.0, kv_rows=[-1])
    with pytest.raises(ValueError):
        oracle.attention_bwd_rows(q, k[:, :, :4].contiguous(), v[:, :, :4].contiguous(), dout, False, 1.0)
    assert math.isfinite(float(oracle.attention_bwd(q, k, v, dout, False, 1.0)[0].sum()))


# Key padding (per-batch valid-key counts L_b, the right-padding reading of the triton-transformer README's
# boolean (batch, seq) mask): keys j >= L_b are invisible to every query of batch b.

def _keep_mask(B, N, lens, causal):
    """Boolean [B, 1, N, N] mask of visible (i, j): j < L_b, and j <= i when causal."""
    j = torch.arange(N)
    keep = (j[None, :] < torch.tensor(lens)[:, None])[:, None, None, :].expand(B, 1, N, N).clone()
    if causal:
        keep &= torch.tril(torch.ones(N, N, dtype=torch.bool))
    return keep


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 1)])
def test_key_padding_matches_torch_autograd_fp64_with_a_boolean_mask(H, Hkv, causal):
    B, N, d = 3, 50, 64
    lens = [50, 17, 1]
    q, _, _ = ai.make_qkv(B, H, N, d, seed=81)
    _, k, v = ai.make_qkv(B, Hkv, N, d, seed=82)
    dout = _dout(B, H, N, d, seed=83)
    scale = ai.default_scale(d)
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, causal, scale, kv_len=lens)
    qd, kd, vd = (x.to(torch.float64).requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, attn_mask=_keep_mask(B, N, lens, causal),
                                                         scale=scale, enable_gqa=(H != Hkv))
    o.backward(dout.to(torch.float64))
    np.testing.assert_allclose(dq, qd.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, kd.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, vd.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_key_padding_matches_richardson_finite_differences(causal):
    """Central differences of L = sum dO*o through the forward oracle with the same lengths (itself pinned to
    brute force and SDPA with a mask), on a tiny grouped problem with a partly padded and a fully visible batch."""
    B, H, Hkv, N, d = 2, 2, 1, 5, 3
    lens = [3, 5]
    q, _, _ = ai.make_qkv(B, H, N, d, seed=84, dtype="bf16")
    _, k, v = ai.make_qkv(B, Hkv, N, d, seed=85, dtype="bf16")
    q, k, v = q.float(), k.float(), v.float()
    dout = _dout(B, H, N, d, seed=86, dtype="f32")
    scale = 0.7
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, causal, scale, kv_len=lens)

    def loss():
        o, _ = oracle.attention(q, k, v, causal, scale, threads=1, kv_len=lens)
        return float(np.sum(o * dout.to(torch.float64).numpy()))
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        flat = x.view(-1)
        fd = np.zeros(flat.numel())
        for e in range(flat.numel()):
            def central(h):
                x0 = float(flat[e])
                flat[e] = x0 + h
                up = loss()
                flat[e] = x0 - h
                dn = loss()
                flat[e] = x0
                return (up - dn) / (2 * h)
            fd[e] = (4 * central(2.0 ** -9) - central(2.0 ** -8)) / 3
        np.testing.assert_allclose(g.reshape(-1), fd, rtol=0, atol=2e-8, err_msg=f"d{name}")


def test_key_padding_ignores_padded_contents_and_zeroes_their_gradients():
    """Rewriting k and v past L_b changes nothing; dk and dv of padded keys are exactly 0."""
    B, H, N, d = 2, 2, 40, 64
    lens = [23, 40]
    q, k, v = ai.make_qkv(B, H, N, d, seed=87)
    dout = _dout(B, H, N, d, seed=88)
    k2, v2 = k.clone(), v.clone()
    k2[0, :, 23:] = 50.0
    v2[0, :, 23:] = -7.0
    for causal in (False, True):
        a = oracle.attention_bwd(q, k, v, dout, causal, 0.125, kv_len=lens)
        b = oracle.attention_bwd(q, k2, v2, dout, causal, 0.125, kv_len=lens)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)
        assert np.all(a[1][0, :, 23:] == 0.0) and np.all(a[2][0, :, 23:] == 0.0)
        assert np.abs(a[1][0, :, :23]).max() > 0 and np.abs(a[2][0, :, :23]).max() > 0


def test_key_padding_empty_batch_and_clamping():
    """L_b = 0: no query of the batch sees a key, every gradient of the batch is 0 (the other batch is untouched);
    lengths are clamped to [0, N], so L_b >= N is no padding and L_b < 0 is L_b = 0."""
    B, H, N, d = 2, 2, 30, 64
    q, k, v = ai.make_qkv(B, H, N, d, seed=89)
    dout = _dout(B, H, N, d, seed=90)
    full = oracle.attention_bwd(q, k, v, dout, True, 0.2)
    for lens in ([0, 30], [-5, 1000]):
        got = oracle.attention_bwd(q, k, v, dout, True, 0.2, kv_len=lens)
        for x, y in zip(got, full):
            assert np.all(x[0] == 0.0)
            np.testing.assert_array_equal(x[1], y[1])
