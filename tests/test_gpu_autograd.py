"""The differentiable wrappers (attention, attention_varlen): their outputs and the gradients autograd delivers
are the library's forward and gradient calls, bit for bit, and agree with fp64 autograd through the plain
definition on the CPU."""
import math

import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_13_amd
    return exact_attention_13_amd


def _inputs(B, H, Hkv, N, d, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16)
    k = torch.randn((B, Hkv, N, d), generator=g).to(torch.bfloat16)
    v = torch.randn((B, Hkv, N, d), generator=g).to(torch.bfloat16)
    dout = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16)
    return q, k, v, dout


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hkv", [4, 2])
def test_autograd_gradients_are_the_library_gradients(fa, causal, Hkv):
    B, H, N, d = 2, 4, 200, 64
    q, k, v, dout = (t.cuda() for t in _inputs(B, H, Hkv, N, d, seed=61 + Hkv))
    print(f"[autograd] B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal}", flush=True)
    qg, kg, vg = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = fa.attention(qg, kg, vg, causal=causal)
    o.backward(dout)
    o_ref, lse = fa.forward(q, k, v, causal=causal)
    dq, dk, dv = fa.backward(q, k, v, o_ref, lse, dout, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    assert torch.equal(qg.grad, dq) and torch.equal(kg.grad, dk) and torch.equal(vg.grad, dv)
    assert kg.grad.shape == (B, Hkv, N, d)


def test_autograd_with_key_padding(fa):
    B, H, N, d = 3, 2, 130, 128
    q, k, v, dout = (t.cuda() for t in _inputs(B, H, H, N, d, seed=71))
    kv_len = torch.tensor([130, 0, 57], dtype=torch.int32, device="cuda")
    print(f"[autograd] kpad B={B} H={H} N={N} d={d}", flush=True)
    qg, kg, vg = (t.clone().requires_grad_(True) for t in (q, k, v))
    fa.attention(qg, kg, vg, kv_len=kv_len).backward(dout)
    o, lse = fa.forward(q, k, v, kv_len=kv_len)
    dq, dk, dv = fa.backward(q, k, v, o, lse, dout, kv_len=kv_len)
    torch.cuda.synchronize()
    assert torch.equal(qg.grad, dq) and torch.equal(kg.grad, dk) and torch.equal(vg.grad, dv)
    assert torch.count_nonzero(qg.grad[1]) == 0


def test_autograd_varlen(fa):
    lens, H, Hkv, d = [37, 0, 129, 64], 4, 2, 64
    T = sum(lens)
    g = torch.Generator("cpu").manual_seed(81)
    q = torch.randn((T, H, d), generator=g).to(torch.bfloat16).cuda()
    k = torch.randn((T, Hkv, d), generator=g).to(torch.bfloat16).cuda()
    v = torch.randn((T, Hkv, d), generator=g).to(torch.bfloat16).cuda()
    dout = torch.randn((T, H, d), generator=g).to(torch.bfloat16).cuda()
    cu = torch.tensor([0, 37, 37, 166, 230], dtype=torch.int32, device="cuda")
    print(f"[autograd] varlen lens={lens} H={H} Hkv={Hkv} d={d}", flush=True)
    qg, kg, vg = (t.clone().requires_grad_(True) for t in (q, k, v))
    fa.attention_varlen(qg, kg, vg, cu, max(lens), causal=True).backward(dout)
    o, lse = fa.forward_varlen(q, k, v, cu, max(lens), causal=True)
    dq, dk, dv = fa.backward_varlen(q, k, v, o, lse, dout, cu, max(lens), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(qg.grad, dq) and torch.equal(kg.grad, dk) and torch.equal(vg.grad, dv)


def test_autograd_against_fp64_definition(fa):
    """A small problem, gradients through the plain definition in fp64 on the CPU (softmax of the scaled scores
    with the causal mask, times v), within the gradient tolerance: 2e-2 of the tensor's largest entry + 1e-5."""
    B, H, N, d = 1, 2, 96, 64
    q, k, v, dout = _inputs(B, H, H, N, d, seed=91)
    scale = 1.0 / math.sqrt(d)
    print(f"[autograd] fp64 reference B={B} H={H} N={N} d={d} causal", flush=True)
    qg, kg, vg = (t.cuda().requires_grad_(True) for t in (q, k, v))
    fa.attention(qg, kg, vg, causal=True).backward(dout.cuda())
    q64, k64, v64 = (t.double().requires_grad_(True) for t in (q, k, v))
    s = torch.matmul(q64, k64.transpose(-1, -2).contiguous()) * scale
    mask = torch.ones((N, N), dtype=torch.bool).triu(1)
    o64 = torch.matmul(torch.softmax(s.masked_fill(mask, float("-inf")), dim=-1), v64)
    o64.backward(dout.double())
    for name, got, ref in (("dq", qg.grad, q64.grad), ("dk", kg.grad, k64.grad), ("dv", vg.grad, v64.grad)):
        err = (got.double().cpu() - ref).abs().max().item()
        assert err <= 2e-2 * ref.abs().max().item() + 1e-5, (name, err)


def test_calls_on_an_explicit_stream(fa):
    """forward/backward (and the packed variants) given another stream run there and give the current stream's
    results bit for bit; the workspace and outputs they allocate stay reserved for that stream, so memory taken
    on the current stream meanwhile does not disturb the running kernels."""
    B, H, N, d = 2, 4, 300, 128
    q, k, v, dout = (t.cuda() for t in _inputs(B, H, 2, N, d, seed=83))
    print(f"[stream] B={B} H={H} Hkv=2 N={N} d={d} causal=True", flush=True)
    o_ref, lse_ref = fa.forward(q, k, v, causal=True)
    g_ref = fa.backward(q, k, v, o_ref, lse_ref, dout, causal=True)
    lens = [300, 1, 170]
    cu = torch.tensor([0, 300, 301, 471], dtype=torch.int32, device="cuda")
    qv, kv, vv, dv_ = (torch.cat([t[0].transpose(0, 1), t[1].transpose(0, 1)[:sum(lens) - N]]).contiguous()
                       for t in (q, k, v, dout))
    ov_ref, lsev_ref = fa.forward_varlen(qv, kv, vv, cu, max(lens), causal=True)
    gv_ref = fa.backward_varlen(qv, kv, vv, ov_ref, lsev_ref, dv_, cu, max(lens), causal=True)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    st = side.cuda_stream
    o, lse = fa.forward(q, k, v, causal=True, stream=st)
    g = fa.backward(q, k, v, o_ref, lse_ref, dout, causal=True, stream=st)
    ov, lsev = fa.forward_varlen(qv, kv, vv, cu, max(lens), causal=True, stream=st)
    gv = fa.backward_varlen(qv, kv, vv, ov_ref, lsev_ref, dv_, cu, max(lens), causal=True, stream=st)
    junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(8)]  # allocations on the current stream
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    assert all(torch.equal(a, b) for a, b in zip(g, g_ref))
    assert torch.equal(ov, ov_ref) and torch.equal(lsev, lsev_ref)
    assert all(torch.equal(a, b) for a, b in zip(gv, gv_ref))
