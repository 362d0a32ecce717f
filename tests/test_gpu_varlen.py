"""Parity of the packed variable-length forward (fa_fwd_varlen, through the C ABI) with the fp64 oracle.

Same bar as the plain forward: max |o_gpu - o_oracle| and max |lse_gpu - lse_oracle| <= 2e-2 over every checked
element (bf16 inputs). Structural checks are bitwise: one packed sequence equals the [1, H, N, d] forward of the
same data, and nothing outside o and lse is written.
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


def _run(fa, q, k, v, lens, causal, scale):
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device="cuda:0")
    o, lse = fa.forward_varlen(q.to("cuda:0"), k.to("cuda:0"), v.to("cuda:0"), cu, max(max(lens), 1), causal=causal,
                               scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _compare(label, o, lse, q, k, v, lens, causal, scale, rows=None):
    T, H, d = q.shape
    cu = [0] + list(np.cumsum(lens))
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, cu, causal, scale, rows=rows)
    og = o.float().cpu().numpy().astype(np.float64).reshape(T * H, d)
    lg = lse.cpu().numpy().astype(np.float64).T.reshape(T * H)  # [H, T] -> rows t*H + h
    if rows is not None:
        og, lg = og[rows], lg[rows]
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg)), label
    eo = float(np.abs(og - o_ref).max()) if og.size else 0.0
    el = float(np.abs(lg - lse_ref).max()) if lg.size else 0.0
    print(f"[parity] {label} max|do|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL, f"{label}: o error {eo}"
    assert el <= TOL, f"{label}: lse error {el}"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv", [(4, 4), (4, 2), (4, 1)])
@pytest.mark.parametrize("lens", [(1, 7, 63, 64, 65, 300, 0, 129), (1000,), (0, 257, 0, 5)])
def test_varlen_ragged(fa, lens, H, Hkv, d, causal):
    label = f"varlen lens={lens} H{H} Hkv{Hkv} d{d} causal={causal}"
    print(f"[case] {label}", flush=True)
    q, k, v = ai.make_qkv_varlen(lens, H, d, seed=800 + sum(lens), Hkv=Hkv)
    scale = ai.default_scale(d)
    o, lse = _run(fa, q, k, v, lens, causal, scale)
    _compare(label, o, lse, q, k, v, lens, causal, scale)


@pytest.mark.parametrize("name", sorted(ai.VARLEN_WORKLOADS))
def test_varlen_workload_sampled_rows(fa, name):
    w = ai.VARLEN_WORKLOADS[name]
    print(f"[case] {name}", flush=True)
    q, k, v = ai.make_qkv_varlen(w.lens, w.H, w.d, w.seed, Hkv=w.Hkv or None)
    o, lse = _run(fa, q, k, v, w.lens, w.causal, w.scale)
    cu = np.array(w.cu_seqlens)
    g = torch.Generator("cpu").manual_seed(w.seed + 1000)
    rnd = torch.randperm(w.T * w.H, generator=g)[: w.sampled_rows].numpy()
    # every sequence's first and last token and the tokens around 128-row blocks, for the first and last head
    toks = np.unique(np.concatenate([cu[:-1], cu[1:] - 1, np.minimum(cu[:-1] + 127, cu[1:] - 1),
                                     np.minimum(cu[:-1] + 128, cu[1:] - 1)]))
    toks = toks[(toks >= 0) & (toks < w.T)]
    edges = np.concatenate([toks * w.H, toks * w.H + w.H - 1])
    rows = np.unique(np.concatenate([rnd, edges]))
    _compare(name, o, lse, q, k, v, w.lens, w.causal, w.scale, rows=rows)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T,H,Hkv", [(333, 4, 4), (4096, 4, 2), (4096, 32, 8)])
def test_one_packed_sequence_equals_the_padded_forward(fa, T, H, Hkv, causal):
    """The same data as one [1, H, T, d] problem through fa_fwd_gqa gives the same bits (same tiles, same order).
    The packed and padded launches choose the workgroup shape by the same rule (fa_fwd_instance): the 32-head case
    takes the wide instance (16 x 32 = 512 workgroups of 256 rows), the others the split-key one."""
    split = 2 if H == 4 else 1
    for packed in (0, 1):
        assert fa.fa_fwd_instance(1, H, T, 128, int(causal), packed).endswith("8, 2, 2, %s, %d>" % (
            "true" if packed else "false", split))
    d = 128
    q, k, v = ai.make_qkv_varlen((T,), H, d, seed=850, Hkv=Hkv)
    o, lse = _run(fa, q, k, v, (T,), causal, ai.default_scale(d))
    qp, kp, vp = (x.transpose(0, 1)[None].contiguous().to("cuda:0") for x in (q, k, v))
    o2, l2 = fa.forward(qp, kp, vp, causal=causal, scale=ai.default_scale(d))
    torch.cuda.synchronize()
    assert torch.equal(o, o2[0].transpose(0, 1)) and torch.equal(lse, l2[0])


def test_varlen_writes_nothing_outside_o_and_lse(fa):
    lens = (5, 0, 130, 64)
    H, Hkv, d = 4, 2, 64
    T = sum(lens)
    q, k, v = (x.to("cuda:0") for x in ai.make_qkv_varlen(lens, H, d, seed=860, Hkv=Hkv))
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device="cuda:0")
    pad = 4096
    n_o, n_l = T * H * d, T * H
    ob = torch.full((n_o + 2 * pad,), 1234.0, dtype=torch.bfloat16, device="cuda:0")
    lb = torch.full((n_l + 2 * pad,), 777.0, dtype=torch.float32, device="cuda:0")
    o, lse = ob[pad: pad + n_o], lb[pad: pad + n_l]
    rc = fa.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), cu.data_ptr(),
                          len(lens), H, Hkv, T, max(lens), d, 1, ai.default_scale(d),
                          torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_OK
    torch.cuda.synchronize()
    assert torch.all(ob[:pad] == 1234.0) and torch.all(ob[pad + n_o:] == 1234.0)
    assert torch.all(lb[:pad] == 777.0) and torch.all(lb[pad + n_l:] == 777.0)
    ref = fa.forward_varlen(q, k, v, cu, max(lens), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o.view(T, H, d), ref[0]) and torch.equal(lse.view(H, T), ref[1])


# Gradients (fa_bwd_varlen): per gradient tensor max |g - g_oracle| <= 2e-2 max |g_oracle| + 1e-5, the bar of the
# padded gradient call, with o and lse from the library's packed forward.
RTOL_G, ATOL_G = 2e-2, 1e-5


def _bwd(fa, q, k, v, dout, lens, causal, scale):
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device="cuda:0")
    qd, kd, vd, dd = (x.to("cuda:0") for x in (q, k, v, dout))
    ms = max(max(lens), 1)
    o, lse = fa.forward_varlen(qd, kd, vd, cu, ms, causal=causal, scale=scale)
    g = fa.backward_varlen(qd, kd, vd, o, lse, dd, cu, ms, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return g


def _check_grad(label, got, ref):
    g = got.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), label
    err = float(np.abs(g - ref).max()) if g.size else 0.0
    mag = float(np.abs(ref).max()) if ref.size else 0.0
    print(f"[parity] {label} max|err|={err:.3e} max|ref|={mag:.3e} rel={err / max(mag, 1e-300):.3e}", flush=True)
    assert err <= RTOL_G * mag + ATOL_G, f"{label}: error {err} above {RTOL_G} x {mag} + {ATOL_G}"


def _dout_varlen(T, H, d, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn((T, H, d), generator=g, dtype=torch.float32).to(torch.bfloat16)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv", [(4, 4), (4, 1)])
@pytest.mark.parametrize("lens", [(1, 7, 63, 64, 65, 300, 0, 129), (0, 257, 0, 5)])
def test_varlen_backward_ragged(fa, lens, H, Hkv, d, causal):
    label = f"bwd varlen lens={lens} H{H} Hkv{Hkv} d{d} causal={causal}"
    print(f"[case] {label}", flush=True)
    q, k, v = ai.make_qkv_varlen(lens, H, d, seed=900 + sum(lens), Hkv=Hkv)
    dout = _dout_varlen(sum(lens), H, d, 901 + sum(lens))
    scale = ai.default_scale(d)
    dq, dk, dv = _bwd(fa, q, k, v, dout, lens, causal, scale)
    rq, rk, rv = oracle.attention_bwd_varlen(q, k, v, dout, [0] + list(np.cumsum(lens)), causal, scale)
    _check_grad(f"{label} dq", dq, rq)
    _check_grad(f"{label} dk", dk, rk)
    _check_grad(f"{label} dv", dv, rv)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_many_sequences(fa, causal):
    """100 sequences (more than the 64 the kernels order longest-first; past that they take the plain
    workgroup order), lengths 0 .. 200 drawn at random: every row of the forward and every gradient row."""
    rng = np.random.default_rng(940)
    lens = [int(x) for x in rng.integers(0, 201, size=100)]
    H, Hkv, d = 4, 2, 64
    label = f"varlen 100 sequences (total {sum(lens)}) H{H} Hkv{Hkv} d{d} causal={causal}"
    print(f"[case] {label}", flush=True)
    q, k, v = ai.make_qkv_varlen(lens, H, d, seed=941, Hkv=Hkv)
    scale = ai.default_scale(d)
    o, lse = _run(fa, q, k, v, lens, causal, scale)
    _compare(label, o, lse, q, k, v, lens, causal, scale)
    dout = _dout_varlen(sum(lens), H, d, 942)
    dq, dk, dv = _bwd(fa, q, k, v, dout, lens, causal, scale)
    rq, rk, rv = oracle.attention_bwd_varlen(q, k, v, dout, [0] + list(np.cumsum(lens)), causal, scale)
    _check_grad(f"{label} dq", dq, rq)
    _check_grad(f"{label} dk", dk, rk)
    _check_grad(f"{label} dv", dv, rv)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_backward_medium(fa, causal):
    lens, H, Hkv, d = (700, 1, 1500, 333), 8, 2, 128
    label = f"bwd varlen lens={lens} H{H} Hkv{Hkv} d{d} causal={causal}"
    print(f"[case] {label}", flush=True)
    q, k, v = ai.make_qkv_varlen(lens, H, d, seed=910, Hkv=Hkv)
    dout = _dout_varlen(sum(lens), H, d, 911)
    scale = ai.default_scale(d)
    dq, dk, dv = _bwd(fa, q, k, v, dout, lens, causal, scale)
    rq, rk, rv = oracle.attention_bwd_varlen(q, k, v, dout, [0] + list(np.cumsum(lens)), causal, scale)
    _check_grad(f"{label} dq", dq, rq)
    _check_grad(f"{label} dk", dk, rk)
    _check_grad(f"{label} dv", dv, rv)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_backward_one_sequence_equals_fa_bwd(fa, causal):
    T, H, Hkv, d = 1000, 4, 2, 64
    q, k, v = ai.make_qkv_varlen((T,), H, d, seed=920, Hkv=Hkv)
    dout = _dout_varlen(T, H, d, 921)
    scale = ai.default_scale(d)
    a = _bwd(fa, q, k, v, dout, (T,), causal, scale)
    qp, kp, vp, dp = (x.transpose(0, 1)[None].contiguous().to("cuda:0") for x in (q, k, v, dout))
    o, lse = fa.forward(qp, kp, vp, causal=causal, scale=scale)
    b = fa.backward(qp, kp, vp, o, lse, dp, causal=causal, scale=scale)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y[0].transpose(0, 1))


def test_varlen_backward_writes_nothing_outside_its_outputs(fa):
    lens, H, Hkv, d = (5, 0, 130, 64), 4, 2, 64
    T = sum(lens)
    q, k, v = (x.to("cuda:0") for x in ai.make_qkv_varlen(lens, H, d, seed=930, Hkv=Hkv))
    dout = _dout_varlen(T, H, d, 931).to("cuda:0")
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device="cuda:0")
    o, lse = fa.forward_varlen(q, k, v, cu, max(lens), causal=True)
    pad = 4096
    sizes = (T * H * d, T * Hkv * d, T * Hkv * d)
    buf = torch.full((sum(sizes) + 4 * pad,), 1234.0, dtype=torch.bfloat16, device="cuda:0")
    offs = [pad, 2 * pad + sizes[0], 3 * pad + sizes[0] + sizes[1]]
    views = [buf[offs[i]: offs[i] + sizes[i]] for i in range(3)]
    ws = torch.empty((fa.fa_bwd_workspace_bytes(len(lens), H, Hkv, max(lens), d),), dtype=torch.uint8,
                     device="cuda:0")
    rc = fa.fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                          views[0].data_ptr(), views[1].data_ptr(), views[2].data_ptr(), ws.data_ptr(), cu.data_ptr(),
                          len(lens), H, Hkv, T, max(lens), d, 1, ai.default_scale(d),
                          torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_OK
    torch.cuda.synchronize()
    mask = torch.ones_like(buf, dtype=torch.bool)
    for i in range(3):
        mask[offs[i]: offs[i] + sizes[i]] = False
    assert torch.all(buf[mask] == 1234.0)
    ref = fa.backward_varlen(q, k, v, o, lse, dout, cu, max(lens), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(views[0].view(T, H, d), ref[0])
    assert torch.equal(views[1].view(T, Hkv, d), ref[1]) and torch.equal(views[2].view(T, Hkv, d), ref[2])
