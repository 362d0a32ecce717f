"""Parity of the grouped/multi-query (fa_fwd_gqa) and key-padding (fa_fwd_kpad) entry points with the fp64 oracle.

Same bar as the plain forward: max |o_gpu - o_oracle| and max |lse_gpu - lse_oracle| <= 2e-2 (bf16 inputs),
over every checked element. Rows without a visible key must give exactly o = 0 and lse = -inf. Structural checks
are bitwise: grouped heads equal the plain forward on repeated key/value heads, full lengths equal no mask, and
the content of padded keys never matters.
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_13_amd as fa_mod
    return fa_mod


def _qkv(B, H, Hkv, N, d, seed):
    q, _, _ = ai.make_qkv(B, H, N, d, seed, "bf16")
    _, k, v = ai.make_qkv(B, Hkv, N, d, seed + 1, "bf16")
    return q, k, v


def _run(fa, q, k, v, causal, kv_len=None):
    dev = [t.to("cuda:0") for t in (q, k, v)]
    lens = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device="cuda:0")
    o, lse = fa.forward(*dev, causal=causal, scale=ai.default_scale(q.shape[3]), kv_len=lens)
    torch.cuda.synchronize()
    return o, lse


def _compare(o, lse, q, k, v, causal, kv_len=None, rows=None, label=""):
    d = q.shape[3]
    og = o.float().cpu().numpy().astype(np.float64).reshape(-1, d)
    lg = lse.cpu().numpy().astype(np.float64).reshape(-1)
    # oracle lengths: the kernel clamps to [0, N]
    ol = None if kv_len is None else [min(max(int(x), 0), q.shape[2]) for x in kv_len]
    o_ref, lse_ref = oracle.attention_rows(q, k, v, causal, ai.default_scale(d), rows=rows, kv_len=ol)
    if rows is not None:
        og, lg = og[rows], lg[rows]
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lg), empty), f"{label}: rows without visible keys differ"
    assert np.all(og[empty] == 0.0), label
    live = ~empty
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg[live])), label
    eo = float(np.abs(og[live] - o_ref[live]).max()) if live.any() else 0.0
    el = float(np.abs(lg[live] - lse_ref[live]).max()) if live.any() else 0.0
    print(f"[parity] {label} max|do|={eo:.3e} max|dlse|={el:.3e} empty_rows={int(empty.sum())}", flush=True)
    assert eo <= TOL, f"{label}: o error {eo}"
    assert el <= TOL, f"{label}: lse error {el}"


# --- grouped / multi-query heads ------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [77, 1000])
@pytest.mark.parametrize("Hkv", [8, 4, 2, 1])
def test_gqa_parity(fa, Hkv, N, d, causal):
    label = f"gqa B2 H8 Hkv{Hkv} N{N} d{d} causal={causal}"
    print(f"[case] {label}", flush=True)
    q, k, v = _qkv(2, 8, Hkv, N, d, seed=200 + Hkv + N)
    o, lse = _run(fa, q, k, v, causal)
    _compare(o, lse, q, k, v, causal, label=label)


@pytest.mark.parametrize("Hkv,causal", [(8, False), (1, True), (4, True)])
def test_gqa_parity_wide_grid(fa, Hkv, causal):
    """A grid large enough for the 8-wave workgroups (32 query heads, N = 2048); sampled rows plus tile edges."""
    B, H, N, d = 2, 32, 2048, 128
    label = f"gqa B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}"
    print(f"[case] {label}", flush=True)
    q, k, v = _qkv(B, H, Hkv, N, d, seed=230 + Hkv)
    o, lse = _run(fa, q, k, v, causal)
    rows = np.unique(np.concatenate([ai.sample_rows(B, H, N, 384, 230 + Hkv), ai.edge_rows(N, 256, 128),
                                     (B * H - 1) * N + ai.edge_rows(N, 256, 128)]))
    _compare(o, lse, q, k, v, causal, rows=rows, label=label)


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [(2, 6, 2, 300, 64, False), (2, 6, 2, 300, 64, True),
                                                  (1, 12, 4, 1000, 128, True), (8, 6, 2, 200, 128, False),
                                                  (4, 24, 8, 300, 128, True)])
def test_gqa_groups_of_three(fa, B, H, Hkv, N, d, causal):
    """Groups that are not a power of two (3 query heads per key/value head), on grids whose B*H/group is a multiple
    of 8 (the XCD mapping then keeps a group's query heads on one XCD) and on grids where it is not; every row."""
    label = f"gqa B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}"
    print(f"[case] {label}", flush=True)
    q, k, v = _qkv(B, H, Hkv, N, d, seed=250 + B + H + N)
    o, lse = _run(fa, q, k, v, causal)
    _compare(o, lse, q, k, v, causal, label=label)


@pytest.mark.parametrize("N,H,causal", [(333, 16, True), (2048, 32, False), (2048, 32, True)])
def test_gqa_equals_plain_forward_on_repeated_heads(fa, N, H, causal):
    """Each query head reads exactly its group's key/value head: bitwise equal to fa_fwd on repeated heads."""
    B, Hkv, d = 2, 4, 128
    q, k, v = _qkv(B, H, Hkv, N, d, seed=240)
    o, lse = _run(fa, q, k, v, causal)
    kr = k.repeat_interleave(H // Hkv, dim=1).contiguous()
    vr = v.repeat_interleave(H // Hkv, dim=1).contiguous()
    o2, lse2 = _run(fa, q, kr, vr, causal)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


# --- key padding ----------------------------------------------------------------------------------------------------

LENS = {333: [333, 0, 1, 63, 64, 65, 129, 300], 1000: [1000, 999, 0, 1, 128, 511, 700, 17]}


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [333, 1000])
@pytest.mark.parametrize("Hkv", [4, 2])
def test_kpad_parity(fa, Hkv, N, d, causal):
    lens = LENS[N]
    label = f"kpad B{len(lens)} H4 Hkv{Hkv} N{N} d{d} causal={causal}"
    print(f"[case] {label}", flush=True)
    q, k, v = _qkv(len(lens), 4, Hkv, N, d, seed=300 + N + Hkv)
    o, lse = _run(fa, q, k, v, causal, lens)
    _compare(o, lse, q, k, v, causal, lens, label=label)


@pytest.mark.parametrize("causal", [False, True])
def test_kpad_parity_wide_grid(fa, causal):
    """8-wave workgroups (B8 H16 N2048 d128) with mixed lengths; sampled rows plus every batch's edges."""
    B, H, N, d = 8, 16, 2048, 128
    lens = [2048, 1, 0, 127, 128, 129, 1500, 2047]
    label = f"kpad B{B} H{H} N{N} d{d} causal={causal}"
    print(f"[case] {label}", flush=True)
    q, k, v = _qkv(B, H, H, N, d, seed=330)
    o, lse = _run(fa, q, k, v, causal, lens)
    edge = []
    for b, L in enumerate(lens):
        for i in sorted({0, 1, max(L - 1, 0), min(L, N - 1), N - 1, 255, 256}):
            edge.append((b * H + (b % H)) * N + i)
    rows = np.unique(np.concatenate([ai.sample_rows(B, H, N, 384, 330), np.array(edge, dtype=np.int64)]))
    _compare(o, lse, q, k, v, causal, lens, rows=rows, label=label)


@pytest.mark.parametrize("N,H,causal", [(333, 16, False), (2048, 32, True)])
def test_kpad_full_lengths_equal_plain_forward(fa, N, H, causal):
    B, d = 2, 128
    q, k, v = _qkv(B, H, H, N, d, seed=340)
    o, lse = _run(fa, q, k, v, causal, [N] * B)
    o2, lse2 = _run(fa, q, k, v, causal)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("causal", [False, True])
def test_kpad_padded_keys_are_never_read(fa, causal):
    """Garbage (huge values, inf, NaN) in the padded keys and values changes no output bit."""
    B, H, N, d = 4, 4, 1000, 64
    lens = [1000, 250, 1, 640]
    q, k, v = _qkv(B, H, 2, N, d, seed=350)
    o, lse = _run(fa, q, k, v, causal, lens)
    k2, v2 = k.clone(), v.clone()
    for b, L in enumerate(lens):
        k2[b, :, L:] = float("nan")
        v2[b, :, L:] = float("inf")
        if L + 1 < N:
            k2[b, :, L + 1:] = 3e38
    o2, lse2 = _run(fa, q, k2, v2, causal, lens)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_kpad_lengths_are_clamped(fa):
    B, H, N, d = 3, 2, 200, 128
    q, k, v = _qkv(B, H, H, N, d, seed=360)
    o, lse = _run(fa, q, k, v, True, [-5, 10_000, 77])
    o2, lse2 = _run(fa, q, k, v, True, [0, N, 77])
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    _compare(o, lse, q, k, v, True, [-5, 10_000, 77], label="kpad clamped lengths")


def test_kpad_and_gqa_raw_entry_points(fa):
    """The C ABI directly, with raw device pointers: FA_OK, and the same bits as the tensor-level calls."""
    B, H, Hkv, N, d = 2, 4, 2, 130, 64
    q, k, v = (t.to("cuda:0") for t in _qkv(B, H, Hkv, N, d, seed=370))
    lens = torch.tensor([130, 40], dtype=torch.int32, device="cuda:0")
    sc = ai.default_scale(d)
    stream = torch.cuda.current_stream().cuda_stream
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    lse1, lse2 = (torch.empty((B, H, N), dtype=torch.float32, device="cuda:0") for _ in range(2))
    assert fa.fa_fwd_kpad(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(), lse1.data_ptr(), lens.data_ptr(),
                          B, H, Hkv, N, d, 0, sc, stream) == fa.FA_OK
    assert fa.fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), lse2.data_ptr(), B, H, Hkv, N, d,
                         0, sc, stream) == fa.FA_OK
    assert fa.fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), lse2.data_ptr(), B, H, 3, N, d, 0,
                         sc, stream) == fa.FA_ERR_SHAPE
    o1t, lse1t = fa.forward(q, k, v, causal=False, scale=sc, kv_len=lens)
    o2t, lse2t = fa.forward(q, k, v, causal=False, scale=sc)
    torch.cuda.synchronize()
    assert torch.equal(o1, o1t) and torch.equal(lse1, lse1t)
    assert torch.equal(o2, o2t) and torch.equal(lse2, lse2t)
    assert torch.equal(o1[0], o2[0]) and not torch.equal(o1[1], o2[1])  # only batch 1 is padded
