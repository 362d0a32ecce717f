"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle, on the GPU.

Tolerances: max |o_gpu - o_oracle| <= 2e-2 for bf16 inputs and <= 1e-4 for fp32 inputs, absolute, over every
checked element; the same bounds for lse. Inputs are the seeded synthetic workloads of attn_inputs.
"""
import json
import math
from pathlib import Path

import numpy as np
import pytest
import torch

import attn_inputs as ai
import oracle

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
GOLDEN = Path(__file__).resolve().parent / "golden" / "closed_form_cases.json"


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_13_amd as fa_mod
    return fa_mod


def _run(fa, q, k, v, causal, scale, kv_len=None):
    qd, kd, vd = (t.to("cuda:0") for t in (q, k, v))
    lens = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device="cuda:0")
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale, kv_len=lens)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _compare(o_gpu, lse_gpu, q, k, v, causal, scale, dtype, rows=None, label="", kv_len=None):
    B, H, N, d = q.shape
    o_ref, lse_ref = oracle.attention_rows(q, k, v, causal, scale, rows=rows, kv_len=kv_len)
    og = o_gpu.reshape(-1, d)
    lg = lse_gpu.reshape(-1)
    if rows is not None:
        og, lg = og[rows], lg[rows]
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg)), label
    eo = float(np.abs(og - o_ref).max())
    el = float(np.abs(lg - lse_ref).max())
    print(f"[parity] {label} max|do|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL[dtype], f"{label}: o error {eo}"
    assert el <= TOL[dtype], f"{label}: lse error {el}"
    return eo, el


# --- the workloads, full size -------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(ai.WORKLOADS))
def test_workload_parity(fa, name):
    w = ai.WORKLOADS[name]
    print(f"[case] {name}", flush=True)
    q, k, v = ai.make_workload(w)
    lens = ai.kv_len_of(w)
    o, lse = _run(fa, q, k, v, w.causal, w.scale, lens)
    rows = ai.check_rows(w)  # None: every row (C1-C3); else 256 sampled rows and tile edges
    if rows is not None:  # and the tile edges of the last head
        rows = np.unique(np.concatenate([rows, (w.B * w.H - 1) * w.N + ai.edge_rows(w.N, 256, 128)]))
    _compare(o, lse, q, k, v, w.causal, w.scale, w.dtype, rows=rows, label=name, kv_len=lens)


# --- ragged sizes: several tiles and a tail, every row checked ----------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 7, 63, 64, 65, 77, 127, 128, 129, 130, 333, 1000])
def test_ragged_bf16(fa, N, d, causal):
    q, k, v = ai.make_qkv(2, 3, N, d, seed=101 + N, dtype="bf16")
    o, lse = _run(fa, q, k, v, causal, ai.default_scale(d))
    _compare(o, lse, q, k, v, causal, ai.default_scale(d), "bf16", label=f"bf16 N={N} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 5, 64, 77, 200, 257])
def test_ragged_f32(fa, N, d, causal):
    q, k, v = ai.make_qkv(1, 2, N, d, seed=102 + N, dtype="f32")
    o, lse = _run(fa, q, k, v, causal, ai.default_scale(d))
    _compare(o, lse, q, k, v, causal, ai.default_scale(d), "f32", label=f"f32 N={N} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_heads_not_multiple_of_8_and_other_scales(fa, causal):
    q, k, v = ai.make_qkv(3, 5, 300, 128, seed=103, dtype="bf16")
    for scale in (0.03, 0.5):
        o, lse = _run(fa, q, k, v, causal, scale)
        _compare(o, lse, q, k, v, causal, scale, "bf16", label=f"B3H5 scale={scale} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_extreme_scales(fa, d, causal):
    """Scales at both ends of what the entry point accepts: 1e-38 (8 / (scale * log2 e) overflows to +inf, so the
    exponent reference is set once and never moves) and 1e-30 (uniform weights: o is the mean of the visible
    values), and 20 (every row one dominant key; the reference moves on many tiles). Every row against the
    oracle; B*H = 6 puts the grid on the split shape, whose second wave sees no key of the first tile's rows."""
    q, k, v = ai.make_qkv(2, 3, 300, d, seed=106, dtype="bf16")
    for scale in (1e-38, 1e-30, 20.0):
        o, lse = _run(fa, q, k, v, causal, scale)
        _compare(o, lse, q, k, v, causal, scale, "bf16", label=f"d{d} scale={scale} causal={causal}")


# --- closed forms on the GPU ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_golden_closed_forms_zero_padded(fa, dtype, causal):
    """The hand-derived examples, zero-padded to d = 64 (padding adds 0 to every dot product)."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for c in json.loads(GOLDEN.read_text())["cases"]:
        qs = np.asarray(c["q"], dtype=np.float32)
        N, dd = qs.shape

        def pad(a):
            t = torch.zeros((1, 1, N, 64), dtype=torch.float32)
            t[0, 0, :, :dd] = torch.tensor(np.asarray(a, dtype=np.float32))
            return t.to(tdt)

        o, lse = _run(fa, pad(c["q"]), pad(c["k"]), pad(c["v"]), causal, c["scale"])
        exp = c["causal" if causal else "noncausal"]
        env = {"e": math.e, "ln": math.log}
        o_ref = np.array([[eval(x, {"__builtins__": {}}, env) for x in row] for row in exp["o"]])
        lse_ref = np.array([eval(x, {"__builtins__": {}}, env) for x in exp["lse"]])
        assert np.abs(o[0, 0, :, :dd] - o_ref).max() <= TOL[dtype], c["name"]
        assert np.all(o[0, 0, :, dd:] == 0), c["name"]
        assert np.abs(lse[0, 0] - lse_ref).max() <= TOL[dtype], c["name"]


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_visible_values(fa, causal):
    _, k, v = ai.make_qkv(2, 4, 700, 128, seed=104, dtype="bf16")
    q = torch.zeros_like(k)
    o, lse = _run(fa, q, k, v, causal, 0.088)
    vd = v.double().numpy()
    N = 700
    cnt = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = np.cumsum(vd, axis=2) / cnt[None, None, :, None] if causal else vd.mean(axis=2, keepdims=True)
    assert np.abs(o - mean).max() <= 2e-2
    assert np.abs(lse - np.log(cnt)).max() <= 1e-5


def test_single_key_is_exact(fa):
    q, k, v = ai.make_qkv(2, 3, 1, 128, seed=105, dtype="bf16")
    for causal in (False, True):
        o, lse = _run(fa, q, k, v, causal, 0.1)
        np.testing.assert_array_equal(o, v.double().numpy())  # p = 1, l = 1: exact in bf16


@pytest.mark.parametrize("causal", [False, True])
def test_identity_readout_exposes_probabilities(fa, causal):
    N, d = 64, 64
    q, k, _ = ai.make_qkv(1, 1, N, d, seed=106, dtype="bf16")
    v = torch.zeros((1, 1, N, d), dtype=torch.bfloat16)
    v[0, 0, :, :N] = torch.eye(N, dtype=torch.bfloat16)
    o, _ = _run(fa, q, k, v, causal, 0.125)
    p = o[0, 0]
    assert np.all(p >= 0)
    assert np.abs(p.sum(axis=1) - 1).max() <= 2e-2
    if causal:
        assert np.all(p[np.triu_indices(N, 1)] == 0.0)  # masked probabilities are exactly zero
    po, _ = oracle.attention(q, k, v, causal, 0.125)
    assert np.abs(p - po[0, 0]).max() <= 2e-2


# --- determinism, buffers, streams ------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_bitwise_deterministic(fa, causal):
    q, k, v = (t.cuda() for t in ai.make_qkv(2, 8, 1111, 128, seed=107, dtype="bf16"))
    o1, l1 = fa.forward(q, k, v, causal=causal)
    o2, l2 = fa.forward(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_writes_stay_inside_o_and_lse(fa):
    """q, k, v, o, lse as adjacent slices of one allocation, with canary regions around o and lse."""
    B, H, N, d = 1, 3, 200, 64
    n = B * H * N * d
    nl = B * H * N
    guard = 4096  # elements of bf16
    buf = torch.full((3 * n + guard + n + guard,), 7.0, dtype=torch.bfloat16, device="cuda")
    q, k, v = ai.make_qkv(B, H, N, d, seed=108, dtype="bf16")
    buf[:n].copy_(q.reshape(-1))
    buf[n:2 * n].copy_(k.reshape(-1))
    buf[2 * n:3 * n].copy_(v.reshape(-1))
    o = buf[3 * n + guard:3 * n + guard + n].view(B, H, N, d)
    lbuf = torch.full((nl + 2 * 1024,), -5.0, dtype=torch.float32, device="cuda")
    lse = lbuf[1024:1024 + nl].view(B, H, N)
    fa.forward(buf[:n].view(B, H, N, d), buf[n:2 * n].view(B, H, N, d), buf[2 * n:3 * n].view(B, H, N, d),
               causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(buf[3 * n:3 * n + guard] == 7.0) and torch.all(buf[3 * n + guard + n:] == 7.0)
    assert torch.all(lbuf[:1024] == -5.0) and torch.all(lbuf[1024 + nl:] == -5.0)
    assert torch.equal(buf[:n].cpu(), q.reshape(-1))
    _compare(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), q, k, v, True,
             ai.default_scale(d), "bf16", label="adjacent buffers")


def test_runs_on_a_side_stream(fa):
    q, k, v = (t.cuda() for t in ai.make_qkv(1, 8, 512, 64, seed=109, dtype="bf16"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, lse = fa.forward(q, k, v, causal=True)
    s.synchronize()
    o0, l0 = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, l0)


def test_empty_problem(fa):
    q = torch.empty((2, 4, 0, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = fa.forward(q, q.clone(), q.clone())
    assert o.shape == (2, 4, 0, 64) and lse.shape == (2, 4, 0)


@pytest.mark.parametrize("causal", [False, True])
def test_long_sequence(fa, causal):
    """One head of N = 2^18 + 77 keys (a ragged last tile), d = 64: 192 seeded random rows plus the tile edges of
    the first and last blocks against the oracle (each oracle row is a full 262221-key softmax)."""
    B, H, N, d = 1, 1, (1 << 18) + 77, 64
    print(f"[case] B={B} H={H} N={N} d={d} causal={causal}", flush=True)
    q, k, v = ai.make_qkv(B, H, N, d, seed=130, dtype="bf16")
    o, lse = _run(fa, q, k, v, causal, ai.default_scale(d))
    rows = np.unique(np.concatenate([ai.sample_rows(B, H, N, 192, 131), ai.edge_rows(N)]))
    _compare(o, lse, q, k, v, causal, ai.default_scale(d), "bf16", rows=rows, label=f"N={N} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_largest_head_count(fa, causal):
    """B*H = 65535, the largest grid the ABI accepts (B*H is the grid's y extent), with short sequences: every row
    of every head against the oracle, forward and gradients (the dq grid is also B*H high, the dk/dv grid B*H_kv)."""
    B, H, N, d = 65535, 1, 3, 64
    print(f"[case] B={B} H={H} N={N} d={d} causal={causal}", flush=True)
    q, k, v = ai.make_qkv(B, H, N, d, seed=120, dtype="bf16")
    o, lse = _run(fa, q, k, v, causal, ai.default_scale(d))
    _compare(o, lse, q, k, v, causal, ai.default_scale(d), "bf16", label=f"B*H=65535 causal={causal}")
    g = torch.Generator("cpu").manual_seed(121)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    qd, kd, vd, dd = (t.to("cuda:0") for t in (q, k, v, dout))
    od, ld = fa.forward(qd, kd, vd, causal=causal)
    grads = fa.backward(qd, kd, vd, od, ld, dd, causal=causal)
    torch.cuda.synchronize()
    refs = oracle.attention_bwd(q, k, v, dout, causal, ai.default_scale(d))
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        err = float(np.abs(got.double().cpu().numpy() - ref).max())
        bound = 2e-2 * float(np.abs(ref).max()) + 1e-5
        print(f"[parity] B*H=65535 {name} max|err|={err:.3e} bound {bound:.3e}", flush=True)
        assert err <= bound, name


def test_raw_entry_point_reports_errors(fa):
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, 64), dtype=torch.float32, device="cuda")
    rc = fa.fa_fwd(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), lse.data_ptr(), 1, 1, 64, 64, 0, 0.125, 0)
    assert rc == fa.FA_ERR_ALIAS
    rc = fa.fa_fwd(q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(), lse.data_ptr(), 1, 1, 64, 64, 0, 0.125, 0)
    assert rc == fa.FA_OK
    torch.cuda.synchronize()


@pytest.mark.parametrize("d,causal", [(64, False), (128, True)])
def test_both_workgroup_shapes(fa, d, causal):
    """4x32 heads at N=1024 launch the wide instance (8 waves, 256-row workgroups, 128-key tiles); the first 2x32
    heads the narrow one (4 waves, 128-row workgroups, 64-key tiles); the first 32 heads alone the split one (8
    waves on 128 rows, two waves per 32-row group splitting every 128-key tile and merging at the end). All must
    match the oracle on the first batch, and each is deterministic run to run."""
    q, k, v = (t.cuda() for t in ai.make_qkv(4, 32, 1024, d, seed=110, dtype="bf16"))
    rows = ai.sample_rows(1, 32, 1024, 300, seed=110)
    cases = [(q[:nb].contiguous(), k[:nb].contiguous(), v[:nb].contiguous(), label)
             for nb, label in ((4, "wide"), (2, "narrow"), (1, "split"))]
    for qq, kk, vv, label in cases:
        o1, l1 = fa.forward(qq, kk, vv, causal=causal)
        o2, l2 = fa.forward(qq, kk, vv, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), label
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), label
        _compare(o1[:1].float().cpu().numpy().astype(np.float64), l1[:1].cpu().numpy().astype(np.float64),
                 q[:1].cpu(), k[:1].cpu(), v[:1].cpu(), causal, ai.default_scale(d), "bf16", rows=rows,
                 label=f"{label} grid d={d} causal={causal}")


def test_split_shape_edges(fa):
    """The split instance (grids too small for two waves per SIMD) where the second key half of every tile sees no
    key (kv_len 40 < 64, so that wave's partial has l = 0 and must drop out of the merge), with grouped heads and a
    ragged tail; and one long causal head (N = 16389) at sampled rows and the tile edges."""
    B, H, Hkv, N, d = 2, 4, 2, 777, 128
    g = torch.Generator("cpu").manual_seed(121)
    q = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16)
    k = torch.randn((B, Hkv, N, d), generator=g).to(torch.bfloat16)
    v = torch.randn((B, Hkv, N, d), generator=g).to(torch.bfloat16)
    lens = [40, 700]
    print(f"[case] split grid B={B} H={H} Hkv={Hkv} N={N} d={d} kv_len={lens}", flush=True)
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), scale=ai.default_scale(d),
                        kv_len=torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    _compare(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), q, k, v, False,
             ai.default_scale(d), "bf16", label="split grid, key padding", kv_len=lens)

    N = 16389
    print(f"[case] split grid one causal head N={N} d={d}", flush=True)
    g = torch.Generator("cpu").manual_seed(122)
    q, k, v = (torch.randn((1, 1, N, d), generator=g).to(torch.bfloat16) for _ in range(3))
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([ai.sample_rows(1, 1, N, 256, seed=122), ai.edge_rows(N, 256, 128)]))
    _compare(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), q, k, v, True,
             ai.default_scale(d), "bf16", rows=rows, label="split grid, one causal head")
