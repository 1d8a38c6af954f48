"""Pins of the oracle's rotation and block quantizer against library routines,
closed forms, brute force and the pages' printed numbers (CPU only)."""
import math
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import jolt_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if line:
            k, *v = line.split()
            rows[k] = [float(x) for x in v]
    return rows


@pytest.mark.parametrize("D", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hadamard_matches_scipy(D):
    # scipy.linalg.hadamard builds the Sylvester matrix by Kronecker doubling
    assert np.array_equal(O.hadamard(D), scipy.linalg.hadamard(D).astype(np.float64))


def test_hadamard_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        O.hadamard(96)


@pytest.mark.parametrize("D", [64, 128])
def test_rotation_orthogonal_and_energy_preserving(D):
    rng = np.random.default_rng(D)
    sigma = np.where(rng.integers(0, 2, D) == 1, -1, 1).astype(np.int8)
    Q = O.rotation_matrix(sigma)
    assert np.max(np.abs(Q.T @ Q - np.eye(D))) < 1e-12
    R = rng.standard_normal((37, D)) * np.exp(rng.standard_normal(D))[None, :]
    Y = O.rotate_rows(R, sigma)
    assert abs(np.sum(Y * Y) / np.sum(R * R) - 1.0) < 1e-12
    assert np.max(np.abs(O.unrotate_rows(Y, sigma) - R)) < 1e-12 * np.max(np.abs(R))
    # random signs: rotating a signed unit vector e_j gives sigma_j * H[:, j] / sqrt(D)
    j = 5
    e = np.zeros((1, D)); e[0, j] = 1.0
    expect = sigma[j] * scipy.linalg.hadamard(D)[:, j] / math.sqrt(D)
    assert np.allclose(O.rotate_rows(e, sigma)[0], expect, rtol=0, atol=1e-15)


def test_rotation_spreads_an_outlier():
    # a single-coordinate spike becomes flat after rotation (max |Y| = |x| / sqrt(D))
    D = 128
    sigma = np.ones(D, np.int8)
    x = np.zeros((1, D)); x[0, 17] = 8.0
    Y = O.rotate_rows(x, sigma)
    assert np.allclose(np.abs(Y), 8.0 / math.sqrt(D), atol=1e-14)


def test_quantizer_ties_round_half_to_even():
    # b = 4: qmax = 7; a block max of 7 * 2^-3 gives the scale s = 2^-3 exactly
    s = 2.0 ** -3
    y = s * np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 7.0])
    q, sc, yh = O.quantize_blocks(y[None, :], 4, 8)
    assert sc[0, 0] == s
    assert q[0].tolist() == [0, 2, 2, 4, 0, -2, -2, 7]
    assert np.array_equal(yh[0], s * np.array([0, 2, 2, 4, 0, -2, -2, 7.0]))


@pytest.mark.parametrize("b", [2, 4, 8])
def test_quantizer_codes_are_nearest_levels_bruteforce(b):
    rng = np.random.default_rng(b)
    blk = 16
    Y = rng.standard_normal((200, 4 * blk)) * np.exp(rng.standard_normal((200, 1)))
    q, s, yh = O.quantize_blocks(Y, b, blk)
    levels = np.arange(-(1 << (b - 1)), 1 << (b - 1))
    Yb = Y.reshape(200, 4, blk)
    qb = q.reshape(200, 4, blk)
    for r in range(0, 200, 7):
        for k in range(4):
            sc = s[r, k]
            assert sc == np.float32(np.max(np.abs(Yb[r, k])) / ((1 << (b - 1)) - 1))
            for i in range(blk):
                dist = np.abs(Yb[r, k, i] - sc * levels)
                best = levels[dist == dist.min()]
                expect = best[0] if len(best) == 1 else best[best % 2 == 0][0]
                assert qb[r, k, i] == expect
    # by construction the most negative level is never produced
    assert q.min() >= -((1 << (b - 1)) - 1)


def test_quantizer_zero_block_and_b0():
    Y = np.zeros((2, 8))
    q, s, yh = O.quantize_blocks(Y, 8, 8)
    assert np.all(q == 0) and np.all(s == 0) and np.all(yh == 0)
    q0, s0, yh0 = O.quantize_blocks(np.ones((2, 8)), 0, 8)
    assert q0 is None and s0 is None and np.all(yh0 == 0)


def test_two_bit_error_never_exceeds_zero_bit_error():
    rng = np.random.default_rng(3)
    Y = rng.standard_normal((500, 128))
    _, _, y2 = O.quantize_blocks(Y, 2, 128)
    assert np.all(np.abs(Y - y2) <= np.abs(Y) + 1e-15)


def test_mse_ratio_per_two_bits_matches_pages_band():
    """Gaussian rotated residuals, blocks of 128: adjacent-bit MSE ratios land near the
    values printed for the toy and NN-scale runs (loose band: the inputs differ)."""
    g = _read_golden("quant_mse_ratios.txt")
    rng = np.random.default_rng(11)
    Y = rng.standard_normal((4000, 128))
    mse = {}
    for b in (2, 4, 6, 8):
        _, _, yh = O.quantize_blocks(Y, b, 128)
        mse[b] = np.mean((Y - yh) ** 2)
    ratios = [mse[2] / mse[4], mse[4] / mse[6], mse[6] / mse[8]]
    # 4->6 and 6->8 bits are near the high-rate regime, where the printed ratios do not
    # depend on the unknown test data; 2 bits is far from it (the printed 2->4 ratio
    # depends on block size and data), so only its direction is checked
    for r, toy, nn in list(zip(ratios, g["toy"], g["nn_scale"]))[1:]:
        assert 0.8 * min(toy, nn) < r < 1.2 * max(toy, nn), (ratios, toy, nn)
    assert ratios[0] > g["predicted"][0]
    # at high rate the ratio approaches the printed 16x prediction
    assert abs(ratios[2] / g["predicted"][0] - 1.0) < 0.15


def test_bf16_rounding_bruteforce():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(20000) * np.exp(3 * rng.standard_normal(20000))
    # exact ties: midpoints of adjacent bf16 values
    base = O.f64_to_bf16_bits(rng.standard_normal(2000))
    lo = O.bf16_bits_to_f64(base)
    hi = O.bf16_bits_to_f64(base + np.uint16(1))
    mids = 0.5 * (lo + hi)
    zeros = O.f64_to_bf16_bits(np.array([0.0, -0.0]))
    assert zeros.tolist() == [0x0000, 0x8000]
    x = np.concatenate([x, mids])
    got = O.f64_to_bf16_bits(x)
    gv = O.bf16_bits_to_f64(got)
    for delta in (-1, 1):
        nb = O.bf16_bits_to_f64((got.astype(np.int64) + delta).astype(np.uint16))
        d_got = np.abs(x - gv)
        d_nb = np.abs(x - nb)
        assert np.all((d_got < d_nb) | ((d_got == d_nb) & (got % 2 == 0)))
