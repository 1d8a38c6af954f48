"""Pins of the oracle's attention over a decoded cache (the fused decode-into-attention
check): facts that hold whatever the implementation, each able to catch a wrong axis,
scale or normalisation."""
import math

import numpy as np
import pytest

from oracle import jolt_oracle as O


def test_single_token_returns_its_value():
    rng = np.random.default_rng(0)
    K, V, Q = rng.standard_normal((3, 1, 8)), rng.standard_normal((3, 1, 8)), rng.standard_normal((3, 5, 8))
    out = O.attention(K, V, Q, 0.7)
    assert np.allclose(out, np.repeat(V, 5, axis=1), atol=1e-15)


def test_equal_keys_give_the_mean_value():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((2, 1, 16))
    K = np.repeat(k, 9, axis=1)
    V = rng.standard_normal((2, 9, 16))
    out = O.attention(K, V, rng.standard_normal((2, 3, 16)), 0.25)
    assert np.allclose(out, np.repeat(V.mean(axis=1, keepdims=True), 3, axis=1), atol=1e-14)


def test_two_tokens_closed_form():
    """o = w v1 + (1 - w) v2 with w = 1 / (1 + exp(-scale q.(k1 - k2)))."""
    q = np.array([0.5, -1.0, 2.0, 0.25])
    k1, k2 = np.array([1.0, 0.0, 0.5, -2.0]), np.array([-0.5, 1.5, 0.0, 1.0])
    v1, v2 = np.array([1.0, 2.0, 3.0, 4.0]), np.array([-1.0, 0.0, 1.0, 0.5])
    scale = 0.5
    d = scale * sum(a * (b - c) for a, b, c in zip(q, k1, k2))
    w = 1.0 / (1.0 + math.exp(-d))
    want = w * v1 + (1.0 - w) * v2
    out = O.attention(np.stack([k1, k2])[None], np.stack([v1, v2])[None], q[None, None], scale)
    assert np.allclose(out[0, 0], want, atol=1e-15)


@pytest.mark.parametrize("shift", [1.0, 1e3])
def test_shifting_every_key_by_one_vector_changes_nothing(shift):
    """Every score moves by the same q.k0, which the softmax removes (also when the scores are
    far outside the exponential's range)."""
    rng = np.random.default_rng(2)
    K, V, Q = rng.standard_normal((2, 12, 8)), rng.standard_normal((2, 12, 8)), rng.standard_normal((2, 4, 8))
    k0 = shift * rng.standard_normal((2, 1, 8))
    a = O.attention(K, V, Q, 0.3)
    b = O.attention(K + k0, V, Q, 0.3)
    assert np.all(np.isfinite(b))
    assert np.allclose(a, b, atol=1e-12 * max(1.0, shift))


def test_slices_and_queries_are_independent():
    rng = np.random.default_rng(3)
    K, V, Q = rng.standard_normal((3, 7, 8)), rng.standard_normal((3, 7, 8)), rng.standard_normal((3, 2, 8))
    full = O.attention(K, V, Q, 0.4)
    for n in range(3):
        for i in range(2):
            one = O.attention(K[n:n + 1], V[n:n + 1], Q[n:n + 1, i:i + 1], 0.4)
            assert np.allclose(one[0, 0], full[n, i], atol=1e-15)
