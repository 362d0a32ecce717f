"""The forward and the no-allocation gradient call recorded into a HIP graph (torch.cuda.CUDAGraph) and replayed.

Both entry points only enqueue kernels on the caller's stream (no allocation, no synchronisation, no memset), so a
captured graph must reproduce the eager results bit for bit on every replay. Between replays the test does eager work
of its own on the same buffers (it overwrites the outputs) and synchronises, then checks every replay.
"""
import pytest
import torch

import attn_inputs as ai

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_13_amd as fa_mod
    return fa_mod


@pytest.mark.parametrize("causal", [False, True])
def test_forward_and_noalloc_gradients_replay_in_a_graph(fa, causal):
    B, H, Hkv, N, d = 2, 8, 2, 1000, 128
    print(f"[case] graph replay B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal}", flush=True)
    g = torch.Generator("cpu").manual_seed(70 + causal)
    q = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16).cuda()
    k = torch.randn((B, Hkv, N, d), generator=g).to(torch.bfloat16).cuda()
    v = torch.randn((B, Hkv, N, d), generator=g).to(torch.bfloat16).cuda()
    dout = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16).cuda()
    sc = ai.default_scale(d)
    o, lse = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def enqueue(stream):
        rc = fa.fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Hkv, N, d,
                           int(causal), sc, stream)
        assert rc == fa.FA_OK, fa.fa_strerror(rc)
        rc = fa.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                               dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d,
                               int(causal), sc, stream)
        assert rc == fa.FA_OK, fa.fa_strerror(rc)

    # eager results (the first no-allocation call also looks up the scratch buffer, outside the capture)
    enqueue(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        enqueue(side.cuda_stream)  # warm-up on the capturing stream
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            enqueue(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (o, lse, dq, dk, dv):  # eager work between replays: clobber every output
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), ref):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want.view(torch.int32)), \
                f"replay {rep}: {name} differs from the eager result"
    print(f"[graph] causal={causal}: 3 replays bitwise equal to the eager calls", flush=True)
