"""Every row of the long causal workloads, checked against properties of exact attention that need no N x N work.

The oracle compares 256 sampled rows (plus tile edges) of these workloads with its fp64 definition
(tests/test_gpu_parity.py). Here every row of the GPU output is held to facts that hold for the exact result of
any size (the definition on the unite.ai page "Flash Attention: revolutionizing transformer efficiency", opening code
block; causal visibility j <= i):
  * o_i is a convex combination of the visible v_j: min_j v_jc <= o_ic <= max_j v_jc per column (prefix minima and
    maxima of V), up to the bf16 rounding of o (2^-8 relative) and of the weights;
  * lse_i = ln sum_j exp(s_ij) lies between ln(n_i) + mean_j s_ij (Jensen; the mean of the visible scores is
    scale q_i . mean_j k_j, from prefix sums of K) and ln(n_i) + max_j s_ij <= ln(n_i) + scale |q_i| max_j |k_j|
    (Cauchy-Schwarz), and it is at least the row's own diagonal score s_ii;
  * row 0 sees only key 0: o_0 = v_0 exactly and lse_0 = s_00.
A wrong row, tile, head or causal side in the kernel breaks the hull or the lse bounds on some row. The lse bounds
allow 5e-3 for the kernel's own error (the bf16 rounding of the weights moves lse by at most 2^-8, the fp32 score
and sum arithmetic by less than 1e-3).
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai

pytestmark = pytest.mark.gpu

LSE_SLACK = 5e-3


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_13_amd as fa_mod
    return fa_mod


@pytest.mark.parametrize("name", ["c4_bf16_b1h32n16384d128_causal", "c5_bf16_b1h8n32768d64_causal_k3",
                                  "mqa_bf16_b1h32kv1n16384d128_causal"])
def test_every_row_satisfies_the_invariants(fa, name):
    w = ai.WORKLOADS[name]
    print(f"[case] {name} every row", flush=True)
    q, k, v = ai.make_workload(w)
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=w.scale)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    sc = float(np.float32(w.scale))
    n = np.arange(1, w.N + 1, dtype=np.float64)
    group = w.H // w.Hk
    worst = {"hull": 0.0, "jensen": 0.0, "cs": 0.0, "diag": 0.0}
    for b in range(w.B):
        for h in range(w.H):
            qh = q[b, h].double().numpy()
            kh = k[b, h // group].double().numpy()
            vh = v[b, h // group].float().numpy()
            oh, lh = o[b, h], lse[b, h]
            # hull of the visible values, with the rounding of o and of the weights
            lo = np.minimum.accumulate(vh, axis=0)
            hi = np.maximum.accumulate(vh, axis=0)
            slack = 2.0 ** -8 * np.abs(oh) + 2.0 ** -8 * (hi - lo) + 1e-6
            excess = np.maximum(lo - slack - oh, oh - hi - slack)
            worst["hull"] = max(worst["hull"], float(excess.max()))
            assert np.all(excess <= 0), f"{name} b{b} h{h}: o outside the hull of the visible v"
            # lse bounds
            mean_s = sc * np.einsum("id,id->i", qh, np.cumsum(kh, axis=0) / n[:, None])
            lower = np.log(n) + mean_s
            worst["jensen"] = max(worst["jensen"], float((lower - lh).max()))
            assert np.all(lh >= lower - LSE_SLACK), f"{name} b{b} h{h}: lse below ln n + mean score"
            kmax = np.maximum.accumulate(np.linalg.norm(kh, axis=1))
            upper = np.log(n) + sc * np.linalg.norm(qh, axis=1) * kmax
            worst["cs"] = max(worst["cs"], float((lh - upper).max()))
            assert np.all(lh <= upper + LSE_SLACK), f"{name} b{b} h{h}: lse above the Cauchy-Schwarz bound"
            diag = sc * np.einsum("id,id->i", qh, kh)
            worst["diag"] = max(worst["diag"], float((diag - lh).max()))
            assert np.all(lh >= diag - LSE_SLACK), f"{name} b{b} h{h}: lse below the diagonal score"
            # row 0
            assert np.array_equal(oh[0], vh[0]), f"{name} b{b} h{h}: o_0 != v_0"
            assert abs(lh[0] - diag[0]) <= 1e-3 + 1e-4 * abs(diag[0])
    print(f"[invariants] {name}: worst excess over hull {worst['hull']:.3e}, over Jensen {worst['jensen']:.3e}, "
          f"over Cauchy-Schwarz {worst['cs']:.3e}, over diagonal {worst['diag']:.3e} (the lse ones must stay below 5e-3)",
          flush=True)
