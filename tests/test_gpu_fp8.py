"""Parity of the fp8 forward (fa_fwd_fp8, through the C ABI) with the fp64 oracle of the dequantized inputs.

Tolerance, from the arithmetic (the pages give none for FP8). Scores are exact (products of e4m3 values are exact
in fp32, the sums' fp32 rounding is ~2^-24) and exp2 is within a few fp32 ulps; the one coarse step is rounding
the weights p' (the row's maximum weight is in [1, 2^8]) to e4m3: |p~ - p'| <= 2^-4 p' for p' >= 2^-6 and <= 2^-10
below. l sums the rounded weights, so o = sum w~_j v_j with w~ = p~ / sum p~, and
    |o - o_ref| <= sum_j |w~_j - w_j| max_j |v_j - o_ref| <= 2E / (1 - E) max_j |v_j - o_ref|,
    E = sum_j |p~_j - p'_j| / sum p' <= 2^-4 + 2^-10 n / Z,
with n the visible keys and Z = sum_j exp(s_j - max s) >= 1 of the row; o is then rounded to bf16 (2^-9 |o|,
2^-8 allowed). lse: |lse - lse_ref| <= E / (1 - E). The checks below apply that bound per element, plus two tight
ones where the weights are exact or read out one by one (q = 0, v = I).
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_13_amd as fa_mod
    return fa_mod


def _run(fa, q8, k8, v8, sq, sk, sv, causal, scale):
    vt = v8.transpose(2, 3).contiguous()
    o, lse = fa.forward_fp8(q8.to("cuda:0"), k8.to("cuda:0"), vt.to("cuda:0"), sq, sk, sv, causal=causal,
                            scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _bound_check(label, o_gpu, lse_gpu, q8, k8, v8, sq, sk, sv, causal, scale, rows=None):
    B, H, N, d = q8.shape
    o_ref, lse_ref = oracle.attention_fp8_rows(q8, k8, v8, sq, sk, sv, causal, scale, rows=rows)
    flat = np.arange(B * H * N) if rows is None else np.asarray(rows)
    og = o_gpu.reshape(-1, d)[flat]
    lg = lse_gpu.reshape(-1)[flat]
    qd = (q8.to(torch.float64) * float(np.float32(sq))).reshape(-1, N, d)
    kd = (k8.to(torch.float64) * float(np.float32(sk))).reshape(-1, N, d)
    vd = (v8.to(torch.float64) * float(np.float32(sv))).reshape(-1, N, d)
    worst_o = worst_l = 0.0
    for r, fr in enumerate(flat):
        bh, i = divmod(int(fr), N)
        n = i + 1 if causal else N
        s = (kd[bh, :n] @ qd[bh, i]).numpy() * float(np.float32(scale))
        Z = float(np.exp(s - s.max()).sum())
        E = 2.0 ** -4 + 2.0 ** -10 * n / Z
        spread = np.abs(vd[bh, :n].numpy() - o_ref[r][None, :]).max(axis=0)
        bound = 2 * E / (1 - E) * spread + 2.0 ** -8 * np.abs(o_ref[r])
        err = np.abs(og[r] - o_ref[r])
        assert np.all(err <= bound), f"{label} row {fr}: error {err.max()} above bound"
        worst_o = max(worst_o, float((err / bound).max()))
        el = abs(lg[r] - lse_ref[r])
        assert el <= E / (1 - E) + 1e-5, f"{label} row {fr}: lse error {el}"
        worst_l = max(worst_l, el / (E / (1 - E)))
    eo = float(np.abs(og - o_ref).max())
    print(f"[parity] {label} max|do|={eo:.3e} rms={float(np.sqrt(np.mean((og - o_ref) ** 2))):.3e} "
          f"max|dlse|={float(np.abs(lg - lse_ref).max()):.3e} worst error/bound o={worst_o:.3f} lse={worst_l:.3f}",
          flush=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [16, 48, 64, 80, 128, 336, 1008])
def test_fp8_ragged(fa, N, d, causal):
    label = f"fp8 B2 H2 N{N} d{d} causal={causal}"
    print(f"[case] {label}", flush=True)
    q8, k8, v8, sq, sk, sv = ai.make_qkv_fp8(2, 2, N, d, seed=600 + N)
    scale = ai.default_scale(d)
    o, lse = _run(fa, q8, k8, v8, sq, sk, sv, causal, scale)
    _bound_check(label, o, lse, q8, k8, v8, sq, sk, sv, causal, scale)


@pytest.mark.parametrize("B,H,N,d,causal", [(2, 16, 4096, 128, False), (1, 32, 4096, 128, True),
                                              (1, 8, 16384, 128, True), (2, 16, 4096, 64, False),
                                              (1, 32, 4096, 64, True), (1, 64, 2000, 64, True)])
def test_fp8_large_sampled_rows(fa, B, H, N, d, causal):
    """Grids of at least 512 blocks of 256 rows (ceil(N/256) B H >= 512): the 8-wave instances at d = 64 and 128,
    one of them with an 80-key last tile."""
    label = f"fp8 B{B} H{H} N{N} d{d} causal={causal}"
    print(f"[case] {label}", flush=True)
    q8, k8, v8, sq, sk, sv = ai.make_qkv_fp8(B, H, N, d, seed=650 + H)
    scale = ai.default_scale(d)
    o, lse = _run(fa, q8, k8, v8, sq, sk, sv, causal, scale)
    rows = np.unique(np.concatenate([ai.sample_rows(B, H, N, 96, 650 + H), ai.edge_rows(N, 256, 128),
                                     (B * H - 1) * N + ai.edge_rows(N, 256, 128)]))
    _bound_check(label, o, lse, q8, k8, v8, sq, sk, sv, causal, scale, rows=rows)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_extreme_scales(fa, causal):
    """1e-20 x and 8 x the default scale: near-uniform weights, and rows with one dominant key whose exponent
    reference moves on many tiles; every row within the derived bound."""
    N, d = 400, 128
    q8, k8, v8, sq, sk, sv = ai.make_qkv_fp8(2, 3, N, d, seed=690)
    for f in (1e-20, 8.0):
        scale = ai.default_scale(d) * f
        o, lse = _run(fa, q8, k8, v8, sq, sk, sv, causal, scale)
        _bound_check(f"fp8 scale x{f} causal={causal}", o, lse, q8, k8, v8, sq, sk, sv, causal, scale)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [2048, 1936])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_reference_steps_between_tiles_in_8_wave_workgroups(fa, causal, N, d):
    """Scores that step up and down from one 128-key tile to the next, on a grid large enough for the 8-wave
    workgroups (ceil(N/256) B H >= 512), which first take a tile's weights against the current exponent reference
    and form the row maximum only when some row's weights sum to 2^8 or more. With q_i = g_i (1, ..., 1) and
    k_j = b_t (1, ..., 1) on tile t, a row's score gap to its reference is 28 g_i (b_t - b_ref) in log2 units at the
    scale below: for g = 1 the steps give gaps of 7 (weights 2^7: the sum test fails, the maximum does not move
    the reference), 14 (the reference moves), 3.5 (sum test fails, no move), 0 and below (sum test passes); other
    g scale the gaps, g < 0 reverses them. N = 1936 ends in a tile of 16 keys. Sampled rows of every kind against
    the derived bound."""
    B, H = 1, 64
    steps = [1.0, 1.25, 1.5, 1.5, 1.625, 1.0, 2.0, 2.0, 2.5, 2.5, 2.25, 2.5, 1.5, 2.5, 2.5, 2.5]
    gains = [1.0, 0.5, -1.0, 0.75]
    kb = torch.tensor(steps, dtype=torch.float32).repeat_interleave(128)[:N]
    k8 = kb.reshape(1, 1, N, 1).expand(B, H, N, d).contiguous().to(torch.float8_e4m3fn)
    qg = torch.tensor(gains, dtype=torch.float32).repeat(N // len(gains))
    q8 = qg.reshape(1, 1, N, 1).expand(B, H, N, d).contiguous().to(torch.float8_e4m3fn)
    _, _, v8, _, _, sv = ai.make_qkv_fp8(B, H, N, d, seed=695)
    scale = float(np.float32(7.0 / (np.log2(np.e) * d * 0.25)))
    label = f"fp8 stepped scores B{B} H{H} N{N} d{d} causal={causal}"
    print(f"[case] {label}", flush=True)
    o, lse = _run(fa, q8, k8, v8, 1.0, 1.0, sv, causal, scale)
    tile_ends = (128 * np.arange((N + 127) // 128)[:, None] + np.arange(124, 128)[None, :]).ravel()
    tile_ends = tile_ends[tile_ends < N]
    cand = np.unique(np.concatenate([ai.sample_rows(B, H, N, 96, 695), np.arange(0, 8), tile_ends,
                                     (H - 1) * N + tile_ends]))
    # The derived bound needs E = 2^-4 + 2^-10 n / Z well below 1: a causal row that sees only the first keys of
    # its highest tile has one dominant weight among a thousand tiny ones (Z ~ 1) and no useful bound; such rows
    # (chosen from the inputs alone) are left out.
    i = cand % N
    n = i + 1 if causal else np.full_like(i, N)
    s_row = scale * d * np.asarray(gains)[i % 4][:, None] * np.asarray(kb)[None, :]
    s_row = np.where(np.arange(N)[None, :] < n[:, None], s_row, -np.inf)
    Z = np.exp(s_row - s_row.max(axis=1, keepdims=True)).sum(axis=1)
    rows = cand[n / Z <= 128]
    assert len(rows) >= 64, len(rows)
    _bound_check(label, o, lse, q8, k8, v8, 1.0, 1.0, sv, causal, scale, rows=rows)


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_zero_query_is_the_prefix_mean(fa, d):
    """q = 0: every visible score is 0, the weights are exactly 1 (no rounding), o_i = mean of v_0..v_i. Allowed:
    bf16 rounding of o (2^-8 |o|) and the matrix instruction's accumulation of the fp8 products, which is not
    exact fp32 (seen: ~2^-19 of sum |v_j|; allowed: 2^-16 of the mean |v_j|), visible where the mean cancels."""
    B, H, N = 1, 2, 400
    _, k8, v8, _, sk, sv = ai.make_qkv_fp8(B, H, N, d, seed=670)
    q8 = torch.zeros((B, H, N, d), dtype=torch.float8_e4m3fn)
    o, lse = _run(fa, q8, k8, v8, 1.0, sk, sv, True, ai.default_scale(d))
    vd = v8.to(torch.float64).numpy() * float(np.float32(sv))
    cnt = np.arange(1, N + 1)[None, None, :, None]
    mean = np.cumsum(vd, axis=2) / cnt
    mean_abs = np.cumsum(np.abs(vd), axis=2) / cnt
    err = np.abs(o - mean)
    assert np.all(err <= 2.0 ** -8 * np.abs(mean) + 2.0 ** -16 * mean_abs), float(err.max())
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, N + 1)), lse.shape), rtol=0, atol=2e-6)
    print(f"[parity] fp8 q=0 d{d} max|do|={float(err.max()):.3e}", flush=True)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_identity_values_read_out_every_weight(fa, causal):
    """v = I (N = d = 128): o[i, :N] is the row's normalised weights; each must be within its own rounding bound
    |w~_j - w_j| <= (|p~_j - p'_j| + w_j sum_k |p~_k - p'_k|) / sum p~ <= (2^-4 w_j + 2^-10 / Z + E w_j) / (1 - E),
    plus bf16 rounding of o (2^-8 w_j)."""
    N = d = 128
    q8, k8, _, sq, sk, _ = ai.make_qkv_fp8(1, 1, N, d, seed=680)
    v8 = torch.eye(N, dtype=torch.float32).reshape(1, 1, N, d).to(torch.float8_e4m3fn)
    scale = ai.default_scale(d)
    o, _ = _run(fa, q8, k8, v8, sq, sk, 1.0, causal, scale)
    w_ref, _ = oracle.attention_fp8_rows(q8, k8, v8, sq, sk, 1.0, causal, scale)
    w = o[0, 0]
    qd = q8.to(torch.float64)[0, 0] * float(np.float32(sq))
    kd = k8.to(torch.float64)[0, 0] * float(np.float32(sk))
    for i in range(N):
        n = i + 1 if causal else N
        s = (kd[:n] @ qd[i]).numpy() * float(np.float32(scale))
        Z = float(np.exp(s - s.max()).sum())
        E = 2.0 ** -4 + 2.0 ** -10 * n / Z
        # |w~_j - w_j| <= (|D_j| + w_j sum|D|)/sum p~ with |D_j| <= 2^-4 p'_j + 2^-10, sum p~ >= (1 - E) sum p'
        bound = (2.0 ** -4 * w_ref[i, :n] + 2.0 ** -10 / Z + w_ref[i, :n] * E) / (1 - E) + 2.0 ** -8 * w_ref[i, :n]
        err = np.abs(w[i, :n] - w_ref[i, :n])
        assert np.all(err <= bound + 1e-7), (i, float((err - bound).max()))
        if causal:
            assert np.all(w[i, n:] == 0.0)  # masked keys get exactly zero weight
    print(f"[parity] fp8 v=I causal={causal} max|dw|={float(np.abs(w - w_ref).max()):.3e}", flush=True)


def test_fp8_deterministic_and_raw_entry_point(fa):
    B, H, N, d = 2, 4, 1024, 128
    q8, k8, v8, sq, sk, sv = ai.make_qkv_fp8(B, H, N, d, seed=690)
    q, k, vt = q8.cuda(), k8.cuda(), v8.transpose(2, 3).contiguous().cuda()
    a = fa.forward_fp8(q, k, vt, sq, sk, sv, causal=True)
    b = fa.forward_fp8(q, k, vt, sq, sk, sv, causal=True)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    rc = fa.fa_fwd_fp8(q.data_ptr(), k.data_ptr(), vt.data_ptr(), o.data_ptr(), lse.data_ptr(), sq, sk, sv, B, H, N,
                       d, 1, ai.default_scale(d), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == fa.FA_OK
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(a[0], o) and torch.equal(a[1], lse)
    assert fa.fa_fwd_fp8(q.data_ptr(), k.data_ptr(), vt.data_ptr(), o.data_ptr(), lse.data_ptr(), sq, sk, sv, B, H,
                         N + 8, d, 1, 0.1, 0) == fa.FA_ERR_SHAPE
