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


def test_grouped_heads_draw_fewer_key_value_heads_in_the_same_order():
    q, k, v = ai.make_qkv(2, 8, 16, 64, seed=9, dtype="f32", Hkv=2)
    assert q.shape == (2, 8, 16, 64) and k.shape == v.shape == (2, 2, 16, 64)
    g = torch.Generator("cpu").manual_seed(9)
    q_ref = torch.randn((2, 8, 16, 64), generator=g)
    k_ref = torch.randn((2, 2, 16, 64), generator=g)
    assert torch.equal(q, q_ref) and torch.equal(k, k_ref)
    # Hkv = H draws exactly what the plain recipe draws
    assert ai.sha256(*ai.make_qkv(1, 4, 8, 64, seed=9, Hkv=4)) == ai.sha256(*ai.make_qkv(1, 4, 8, 64, seed=9))


def test_grouped_and_padded_workload_accounting():
    w = ai.WORKLOADS["gqa_bf16_b2h32kv8n4096d128"]
    assert w.Hk == 8 and w.flops == 4 * 2 * 32 * 4096 ** 2 * 128
    assert w.algorithmic_bytes == (2 * 2 * 32 + 2 * 2 * 8) * 4096 * 128 * 2 + 4 * 2 * 32 * 4096
    m = ai.WORKLOADS["mqa_bf16_b1h32kv1n16384d128_causal"]
    assert m.Hk == 1 and m.flops == 2 * 32 * 16384 ** 2 * 128
    p = ai.WORKLOADS["kpad_bf16_b8h16n4096d128"]
    assert len(p.kv_len) == p.B and all(0 < L <= p.N for L in p.kv_len)
    assert p.flops == 4 * 16 * 128 * 4096 * sum(p.kv_len)   # non-causal: every query sees L keys
    assert p.algorithmic_bytes == (2 * 8 * 16 * 4096 + 2 * 16 * sum(p.kv_len)) * 128 * 2 + 4 * 8 * 16 * 4096
    assert ai.kv_len_of(p) == list(p.kv_len) and ai.kv_len_of(w) is None
    # causal with padding: the triangle of the valid keys plus the rows past it
    wc = ai.Workload("x", 1, 1, 10, 64, True, "bf16", 1, kv_len=(4,))
    assert wc.flops == 4 * 64 * (4 * 4 / 2 + 6 * 4)
