"""The seeded input generator: distribution, determinism, sub-range consistency, bf16 rounding."""
import numpy as np
import scipy.stats as st
import torch

import synth


def test_normal_distribution():
    z = synth.normal_f32(77, (1 << 20,)).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    assert abs(st.kurtosis(z, fisher=False) - 3) < 0.05
    assert st.kstest(z, "norm").pvalue > 1e-3
    s = synth.normal_f32(78, (1 << 16,), sigma=0.02).std()
    assert abs(s / 0.02 - 1) < 0.02


def test_deterministic_and_subrange_consistent():
    a = synth.normal_f32(5, (1000,))
    b = synth.normal_f32(5, (1000,))
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(synth.normal_f32(5, (300,), first=400), a[400:700])
    assert not np.array_equal(a, synth.normal_f32(6, (1000,)))


def test_bf16_is_rne_of_fp32_draw():
    f = synth.normal_f32(9, (50000,), 0.3)
    b = synth.normal_bf16(9, (50000,), 0.3)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, ref)


def test_expert_weight_subset_matches_full():
    spec = synth.SKEWED_128E.with_(E=6, d=64, f=128)
    full = synth.gen_expert_weight(spec, "down")
    part = synth.gen_expert_weight(spec, "down", experts=[4, 1])
    np.testing.assert_array_equal(part, full[[4, 1]])
    assert full.shape == (6, 64, 128)


def test_skewed_logits_bias():
    lg = synth.skewed_logits(4001, 20000, 8, 2.0).astype(np.float64)
    b = lg.mean(0)
    ref = 2.0 * np.log(1.0 / np.arange(1, 9))
    np.testing.assert_allclose(b, ref, atol=0.03)
