"""A seeded sweep over random small configurations of the forward entry points (plain, grouped heads, key padding,
packed variable-length batches; both head dims; causal or not; several scales and input magnitudes) against the
fp64 oracle, with the forward's bar: max |o - o_oracle| and max |lse - lse_oracle| <= 2e-2, and lse = -inf exactly
where a row sees no key. Each case prints its parameters before it runs."""
import math
import random

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

TOL = 2e-2
N_CASES = 120


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_13_amd as fa_mod
    return fa_mod


def _compare(label, o, lse, o_ref, lse_ref):
    fin = np.isfinite(lse_ref)
    assert np.all(lse[~fin] == -np.inf), f"{label}: rows without keys must give lse = -inf"
    e_o = float(np.abs(o - o_ref).max()) if o.size else 0.0
    e_l = float(np.abs(lse[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    assert e_o <= TOL and e_l <= TOL, f"{label}: o error {e_o}, lse error {e_l}"
    return e_o, e_l


def test_random_configurations(fa):
    rng = random.Random(20261203)
    worst_o = worst_l = 0.0
    for case in range(N_CASES):
        d = rng.choice([64, 128])
        causal = rng.random() < 0.5
        H = rng.choice([1, 2, 4, 8])
        Hkv = rng.choice([h for h in (1, 2, 4, 8) if H % h == 0])
        mode = rng.choice(["plain", "plain", "kpad", "varlen"])
        scale = rng.choice([1.0 / math.sqrt(d), 0.3, 0.05])
        amp = rng.choice([0.5, 1.0, 2.0, 3.0])
        seed = rng.randrange(1 << 30)
        g = torch.Generator("cpu").manual_seed(seed)
        if mode == "varlen":
            lens = [rng.choice([0, 1, rng.randrange(1, 300)]) for _ in range(rng.randrange(1, 5))]
            if sum(lens) == 0:
                lens.append(5)
            T = sum(lens)
            label = f"case {case}: varlen lens={lens} H={H} Hkv={Hkv} d={d} causal={causal} scale={scale:.3f} amp={amp}"
            print(f"[sweep] {label}", flush=True)
            q = (torch.randn((T, H, d), generator=g) * amp).to(torch.bfloat16)
            k = (torch.randn((T, Hkv, d), generator=g) * amp).to(torch.bfloat16)
            v = torch.randn((T, Hkv, d), generator=g).to(torch.bfloat16)
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            o, lse = fa.forward_varlen(q.cuda(), k.cuda(), v.cuda(), torch.tensor(cu, device="cuda"), max(lens),
                                       causal=causal, scale=scale)
            torch.cuda.synchronize()
            o_ref, lse_ref = oracle.attention_varlen(q, k, v, cu, causal, scale)
            e = _compare(label, o.double().cpu().numpy().reshape(-1, d), lse.cpu().numpy().T.reshape(-1),
                         o_ref, lse_ref)
        else:
            B = rng.randrange(1, 4)
            N = rng.choice([1, 2, 63, 64, 65, rng.randrange(1, 700)])
            kv_len = [rng.randrange(0, N + 1) for _ in range(B)] if mode == "kpad" else None
            label = (f"case {case}: {mode} B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} kv_len={kv_len} "
                     f"scale={scale:.3f} amp={amp}")
            print(f"[sweep] {label}", flush=True)
            q = (torch.randn((B, H, N, d), generator=g) * amp).to(torch.bfloat16)
            k = (torch.randn((B, Hkv, N, d), generator=g) * amp).to(torch.bfloat16)
            v = torch.randn((B, Hkv, N, d), generator=g).to(torch.bfloat16)
            kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device="cuda")
            o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, kv_len=kl)
            torch.cuda.synchronize()
            o_ref, lse_ref = oracle.attention(q, k, v, causal, scale, kv_len=kv_len)
            e = _compare(label, o.double().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)
        worst_o, worst_l = max(worst_o, e[0]), max(worst_l, e[1])
    print(f"[sweep] {N_CASES} cases, worst o error {worst_o:.3e}, worst lse error {worst_l:.3e}", flush=True)
