"""Every workgroup shape of the bf16 forward kernel against the fp64 oracle, every row, with a ragged query tail.

The library picks one of three shapes from the grid size alone (fa_fwd_instance names the instance it launches):
  * wide:   8 waves x 32 rows, 128-key tiles, when ceil(N/256) * B*H >= 512;
  * narrow: 4 waves x 32 rows, 64-key tiles, when ceil(N/128) * B*H >= 512 but the wide grid is smaller;
  * split:  8 waves on 128 rows, the two waves of each 32-row group taking the two 64-key halves of every
            128-key tile and merging their partial (m, l, o) at the end, otherwise;
  * split64: causal d = 64 grids whose 64-row blocks fit at two workgroups per CU (ceil(N/64) * B*H <= 512): the
            split shape on 64 rows and 4 waves, complementary query blocks paired on each CU.
Each test asks the library which instance it launches for its sizes, so a change of the rule cannot silently move
a case to another shape. Every shape runs at d in {64, 128}, causal and not, with N = 1000 (not a multiple of any
tile), and with key padding, grouped heads and packed sequences. Bar: max |o - o_oracle| and max |lse -
lse_oracle| <= 2e-2 over every row (bf16 inputs).
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle

pytestmark = pytest.mark.gpu

TOL = 2e-2
N = 1000
# (B, H) that put B*H heads of N = 1000 rows on each shape: ceil(1000/256) = 4, ceil(1000/128) = 8,
# ceil(1000/64) = 16; causal d = 64 takes split64 while 16 * B*H <= 512, so its split cases use 48 heads
HEADS = {"wide": (2, 64), "narrow": (2, 32), "split": (2, 4), "split64": (2, 4)}
SIGNATURE = {"wide": "8, 2, 2, {p}, 1>", "narrow": "4, 2, 1, {p}, 1>", "split": "8, 2, 2, {p}, 2>",
             "split64": "4, 2, 2, {p}, 2>"}


def _heads(shape, d, causal):
    if shape == "split" and d == 64 and causal:
        return (2, 24)
    return HEADS[shape]


# (shape, d, causal) of every instance a non-packed call can launch
CASES = [(sh, d, c) for sh in ("wide", "narrow", "split") for d in (64, 128) for c in (False, True)] + \
    [("split64", 64, True)]


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_13_amd as fa_mod
    return fa_mod


def _expect_shape(fa, shape, B, H, n, d, causal, packed=False):
    name = fa.fa_fwd_instance(B, H, n, d, int(causal), int(packed))
    want = f"fa_fwd_bf16_kernel<{d}, {'true' if causal else 'false'}, " + SIGNATURE[shape].format(
        p="true" if packed else "false")
    assert name == want, f"{shape}: the library launches {name}, expected {want}"
    print(f"[case] {name} B={B} H={H} N={n}", flush=True)


def _compare(label, o, lse, q, k, v, causal, scale, kv_len=None):
    d = q.shape[-1]
    o_ref, lse_ref = oracle.attention_rows(q, k, v, causal, scale, kv_len=kv_len)
    og = o.float().cpu().numpy().astype(np.float64).reshape(-1, d)
    lg = lse.cpu().numpy().astype(np.float64).reshape(-1)
    fin = np.isfinite(lse_ref)
    assert np.all(np.isfinite(og)) and np.array_equal(np.isfinite(lg), fin), label
    eo = float(np.abs(og - o_ref).max())
    el = float(np.abs(lg[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    print(f"[parity] {label} rows={og.shape[0]} max|do|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL, f"{label}: o error {eo}"
    assert el <= TOL, f"{label}: lse error {el}"


@pytest.mark.parametrize("shape,d,causal", CASES)
def test_every_shape_every_row(fa, shape, d, causal):
    B, H = _heads(shape, d, causal)
    _expect_shape(fa, shape, B, H, N, d, causal)
    q, k, v = ai.make_qkv(B, H, N, d, seed=900 + 10 * d + causal, dtype="bf16")
    scale = ai.default_scale(d)
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    _compare(f"{shape} d={d} causal={causal}", o, lse, q, k, v, causal, scale)


@pytest.mark.parametrize("shape,d,causal", [(sh, 128, c) for sh in ("wide", "narrow", "split") for c in (False, True)]
                         + [("split64", 64, True)])
def test_every_shape_with_key_padding_and_grouped_heads(fa, shape, d, causal):
    """Per-batch key lengths (one that ends inside a 64-key part, one past the first tile) together with 4 query
    heads per key/value head."""
    B, H = _heads(shape, d, causal)
    Hkv = H // 4
    _expect_shape(fa, shape, B, H, N, d, causal)
    q, k, v = ai.make_qkv(B, H, N, d, seed=940 + causal, dtype="bf16", Hkv=Hkv)
    lens = [517, 40]
    scale = ai.default_scale(d)
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale,
                        kv_len=torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    _compare(f"{shape} kv_len={lens} H={H} Hkv={Hkv} causal={causal}", o, lse, q, k, v, causal, scale, kv_len=lens)


@pytest.mark.parametrize("shape,causal", [(sh, c) for sh in ("wide", "narrow", "split") for c in (False, True)]
                         + [("split64", True)])
def test_every_shape_multi_query(fa, shape, causal):
    """One key/value head for every query head of a batch (d = 64)."""
    d = 64
    B, H = _heads(shape, d, causal)
    _expect_shape(fa, shape, B, H, N, d, causal)
    q, k, v = ai.make_qkv(B, H, N, d, seed=950 + causal, dtype="bf16", Hkv=1)
    scale = ai.default_scale(d)
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    _compare(f"{shape} multi-query causal={causal}", o, lse, q, k, v, causal, scale)


# Packed batches of 4 sequences, the longest 1000 tokens: max_seqlen = 1000 and B*H = 128, 64 or 8 heads pick the
# shape (packed calls never take split64).
VARLEN_H = {"wide": 32, "narrow": 16, "split": 2}


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", ["wide", "narrow", "split"])
def test_every_shape_packed(fa, shape, causal):
    lens = (1000, 777, 130, 1)
    H, d = VARLEN_H[shape], 128
    Hkv = H // 2
    _expect_shape(fa, shape, len(lens), H, max(lens), d, causal, packed=True)
    q, k, v = ai.make_qkv_varlen(lens, H, d, seed=960 + causal, Hkv=Hkv)
    scale = ai.default_scale(d)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device="cuda:0")
    o, lse = fa.forward_varlen(q.cuda(), k.cuda(), v.cuda(), cu, max(lens), causal=causal, scale=scale)
    torch.cuda.synchronize()
    T = sum(lens)
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, [0] + list(np.cumsum(lens)), causal, scale)
    og = o.float().cpu().numpy().astype(np.float64).reshape(T * H, d)
    lg = lse.cpu().numpy().astype(np.float64).T.reshape(T * H)
    eo, el = float(np.abs(og - o_ref).max()), float(np.abs(lg - lse_ref).max())
    print(f"[parity] {shape} packed lens={lens} H={H} Hkv={Hkv} causal={causal} max|do|={eo:.3e} "
          f"max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL and el <= TOL

