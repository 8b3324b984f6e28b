"""Checks of the seeded input generators (not of the method)."""
import numpy as np

from moe_expert_offload_amd.synth import (WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits,
                                          generator, zipf_reuse_trace)


def test_bf16_round_to_nearest_even():
    v = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 1 + 2 ** -9], np.float32)
    assert f32_to_bf16_bits(v).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F80]
    r = np.random.default_rng(0).normal(size=1000).astype(np.float32)
    back = bf16_bits_to_f32(f32_to_bf16_bits(r))
    assert np.all(np.abs(back - r) <= np.abs(r) * 2.0 ** -8)


def test_trace_shape_distinct_and_reuse():
    rng = generator(2, 3)
    L, E, k, B, S = 6, 128, 8, 3, 300
    tr = zipf_reuse_trace(L, E, k, B, S, 1.1, 0.6, rng)
    assert tr.shape == (S, L, B, k)
    assert all(len(set(row.tolist())) == k for row in tr.reshape(-1, k))
    kept = np.mean([len(set(tr[s, l, b].tolist()) & set(tr[s - 1, l, b].tolist())) / k
                    for s in range(1, S) for l in range(L) for b in range(B)])
    assert 0.6 <= kept <= 0.8  # 0.6 kept plus chance redraws of popular experts


def test_seeded_and_workload_sizes():
    a = generator(1, 2, 5).normal(size=4)
    b = generator(1, 2, 5).normal(size=4)
    assert np.array_equal(a, b)
    assert WORKLOADS["decode-L40-d2048-E128-top8"].n_slots == 1894
    assert WORKLOADS["decode-L43-d4096-E256-top6"].n_slots == 1210
    assert WORKLOADS["decode-L40-d2048-E128-top8"].shape.record_bytes == 9437184
    assert WORKLOADS["decode-L43-d4096-E256-top6"].shape.record_bytes == 50331648
