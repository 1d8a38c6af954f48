"""The seeded generator is deterministic, shaped like the workloads, and its bf16
rounding agrees with torch's float32 -> bfloat16 conversion (CPU only)."""
import numpy as np
import torch

import kvsynth as ks


def test_deterministic_and_shaped():
    w = ks.get_workload("tiny")
    a = ks.generate_table(w, 0, 0)
    b = ks.generate_table(w, 0, 0)
    assert a.dtype == np.uint16 and a.shape == (4, 64, 64)
    assert np.array_equal(a, b)
    s = ks.rotation_signs(w, 0, 0)
    assert set(np.unique(s).tolist()) <= {-1, 1} and s.shape == (64,)
    om = ks.sketch_omega(w, 0, 0, 8)
    assert om.shape == (4 * 8, 40)


def test_workload_table_counts_and_budgets():
    assert ks.get_workload("mistral_t512").n_tables == 16
    assert ks.get_workload("llama13b_t2048").n_tables == 20
    assert ks.get_workload("tiny").budgets() == [16384]
    assert ks.get_workload("mistral_t512").budgets() == [33554432]
    assert ks.get_workload("mistral_t1024_flash").budgets() == [44739242]
    assert ks.get_workload("llama13b_t2048").budgets() == [838860800, 559240533]


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(2 * rng.standard_normal(100000))).astype(np.float32)
    ours = ks.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_keys_have_outlier_channels_and_values_are_flat():
    w = ks.get_workload("mistral_t512")
    k = ks.bf16_bits_to_f64(ks.generate_table(w, 0, 0)[:4])
    v = ks.bf16_bits_to_f64(ks.generate_table(w, 0, 1)[:4])
    ck = np.sqrt(np.mean(k ** 2, axis=(0, 1)))
    cv = np.sqrt(np.mean(v ** 2, axis=(0, 1)))
    assert ck.max() / np.median(ck) > 4.0
    assert cv.max() / np.median(cv) < 2.5
