"""Pins of the modelled candidate table (the pages' separable error model D ~ eps^2(b) tau,
tables from spectra only): the calibration against the high-rate uniform-quantizer law,
and tau against an explicit partial Tucker reconstruction (the ST-HOSVD energy identity)."""
import numpy as np
import pytest

import kvsynth as ks
from oracle import jolt_oracle as O


def test_gaussian_eps2_follows_the_high_rate_law():
    """At 4 and 8 bits the block quantizer's error per value is close to step^2 / 12 with
    step = max|g| / (2^(b-1) - 1) per row (uniform error within a step); eps^2 falls with b."""
    rng = np.random.default_rng(0)
    G = rng.standard_normal((4096, 128))
    e = O.gaussian_eps2(G, (0, 2, 4, 8))
    assert e[0] == 1.0 and e[0] > e[2] > e[4] > e[8] > 0
    m2 = np.max(np.abs(G), axis=1) ** 2
    for b, tol in ((4, 0.08), (8, 0.03)):
        q = (1 << (b - 1)) - 1
        law = float(np.sum(m2 / (q * q) / 12.0) * G.shape[1] / np.sum(G * G))
        assert abs(e[b] / law - 1) < tol, (b, e[b], law)


@pytest.mark.parametrize("seed", [0, 1])
def test_tau_equals_the_partial_tucker_error(seed):
    """b = 0 entries with eps^2(0) = 1 are tau; tau equals ||X - X~||^2 / ||X||^2 of the partial
    Tucker reconstruction with unrounded factors (built by the oracle's reconstruction path)."""
    rng = np.random.default_rng(seed)
    N, T, D = 3, 24, 16
    X = rng.standard_normal((N, T, D)) @ np.diag(np.linspace(2.0, 0.1, D))
    rT, rd = (4, 8, T), (4, 8, D)
    tab = O.model_table(X, rT, rd, (0,), {0: 1.0})
    xn2 = float(np.sum(X * X))
    lam_d, Ud = O.feature_factor(X)
    for j, r_d in enumerate(rd):
        Yr = X if r_d == D else X @ Ud[:, :r_d]
        _, UT = O.token_factor_exact(O.token_unfolding(Yr), 8)
        for i, r_T in enumerate(rT):
            Ut, Udr, G = O._factors_for(X, Ud, UT, r_T, r_d, round_fp16=False)
            err = float(np.sum((X - O.reconstruct(Ut, Udr, G)) ** 2)) / xn2
            assert abs(tab[i * len(rd) + j] - err) <= 1e-12 * max(err, 1e-3), (r_T, r_d, tab[i * len(rd) + j], err)


def test_randomized_tau_equals_exact_when_the_sketch_spans_the_unfolding():
    rng = np.random.default_rng(3)
    N, T, D = 2, 20, 8
    X = rng.standard_normal((N, T, D))
    rT, rd = (4, 8, T), (4, D)
    om = {r: ks.f32_to_bf16_bits(rng.standard_normal((N * r, N * r + 4)).astype(np.float32)) for r in rd}
    ex = O.model_table(X, rT, rd, (0,), {0: 1.0})
    rn = O.model_table(X, rT, rd, (0,), {0: 1.0}, "randomized", om)
    assert np.allclose(ex, rn, rtol=1e-9, atol=1e-12)


def test_model_scales_with_eps2():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((2, 16, 8))
    eps = {0: 1.0, 2: 0.5, 4: 0.01, 8: 4e-5}
    t = O.model_table(X, (4, 16), (4, 8), (0, 2, 4, 8), eps).reshape(2, 2, 4)
    for b_i, b in enumerate((2, 4, 8)):
        assert np.allclose(t[:, :, b_i + 1], eps[b] * t[:, :, 0], rtol=1e-15, atol=0)
    assert np.all(t[1, 1] == 0.0)  # (T, D)
