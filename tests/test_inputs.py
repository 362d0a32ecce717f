"""The seeded input generator: determinism, dtype rounding, the sampled-row recipe."""
import numpy as np
import torch

import attn_inputs as ai


def test_same_seed_same_bytes_different_seed_different_bytes():
    a = ai.make_qkv(1, 2, 64, 64, seed=3)
    b = ai.make_qkv(1, 2, 64, 64, seed=3)
    c = ai.make_qkv(1, 2, 64, 64, seed=4)
    assert ai.sha256(*a) == ai.sha256(*b)
    assert ai.sha256(*a) != ai.sha256(*c)


def test_bf16_is_round_to_nearest_even_of_the_fp32_draw():
    q, k, v = ai.make_qkv(1, 1, 32, 64, seed=5, dtype="bf16")
    g = torch.Generator("cpu").manual_seed(5)
    q32 = torch.randn((1, 1, 32, 64), generator=g, dtype=torch.float32)
    bits = q32.view(torch.int32).numpy().astype(np.int64)
    # round-to-nearest-even on the top 16 bits, done by hand on the integer bits
    lsb = (bits >> 16) & 1
    rne = ((bits + 0x7FFF + lsb) >> 16) & 0xFFFF
    got = q.view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    np.testing.assert_array_equal(got, rne)
    assert q.dtype == torch.bfloat16 and q.is_contiguous() and q.shape == (1, 1, 32, 64)


def test_k_scale_applied_before_rounding():
    _, k1, _ = ai.make_qkv(1, 1, 16, 64, seed=5, dtype="f32")
    _, k3, _ = ai.make_qkv(1, 1, 16, 64, seed=5, dtype="f32", k_scale=3.0)
    torch.testing.assert_close(k3, k1 * 3.0, rtol=0, atol=0)


def test_sampled_rows_are_distinct_in_range_and_seeded():
    r = ai.sample_rows(1, 32, 16384, 256, seed=4)
    assert len(np.unique(r)) == 256 and r.min() >= 0 and r.max() < 32 * 16384
    np.testing.assert_array_equal(r, ai.sample_rows(1, 32, 16384, 256, seed=4))
    w = ai.WORKLOADS["c4_bf16_b1h32n16384d128_causal"]
    rows = ai.check_rows(w)
    assert set(ai.edge_rows(w.N)).issubset(set(rows.tolist()))


def test_workload_flops_and_bytes():
    w = ai.WORKLOADS["c3_bf16_b2h16n4096d128"]
    assert w.flops == 4 * 2 * 16 * 4096 ** 2 * 128
    assert w.algorithmic_bytes == 134_742_016
    wc = ai.WORKLOADS["c4_bf16_b1h32n16384d128_causal"]
    assert wc.flops == 2 * 32 * 16384 ** 2 * 128
    assert ai.default_scale(128) == float(np.float32(1 / np.sqrt(128)))
