"""Pins of the oracle's partial Tucker / score stage against textbook identities,
library SVDs and the direct distortion definition (CPU only)."""
import numpy as np
import pytest

import kvsynth as ks
from oracle import jolt_oracle as O

RT = (4, 8, 16, 32, 64)
RD = (4, 8, 16, 32, 64)
BITS = (0, 2, 4, 8)


def _tiny(seed=0, N=4, T=64, D=64):
    w = ks.get_workload("tiny")
    X = O.bf16_bits_to_f64(ks.generate_table(w, 0, 0))
    sigma = ks.rotation_signs(w, 0, 0)
    return X[:N, :T, :D], sigma


def _svd_spectra(X, rd):
    """Feature spectrum of X and token spectrum of X projected on its top-rd right
    singular vectors, both from numpy's SVD (independent of the oracle's eigh)."""
    N, T, D = X.shape
    _, s, Vt = np.linalg.svd(X.reshape(N * T, D), full_matrices=False)
    lam_d = s ** 2
    Y = X @ Vt[:rd].T if rd < D else X
    A = Y.transpose(1, 0, 2).reshape(T, -1)
    lam_t = np.linalg.svd(A, compute_uv=False) ** 2
    return lam_d, lam_t


def test_sthosvd_error_identity_without_rounding():
    X, sigma = _tiny()
    N, T, D = X.shape
    r = O.build_table(X, sigma, RT, RD, BITS, 64, round_fp16=False)
    Dt = r.D.reshape(5, 5, 4)
    for j, rd in enumerate(RD):
        lam_d, lam_t = _svd_spectra(X, rd)
        for i, rT in enumerate(RT):
            expect = lam_d[rd:].sum() + lam_t[rT:].sum()
            assert abs(Dt[i, j, 0] * r.xnorm2 - expect) <= 1e-9 * r.xnorm2, (rT, rd)


def test_full_token_rank_column_closed_form():
    X, sigma = _tiny()
    r = O.build_table(X, sigma, RT, RD, BITS, 64, round_fp16=False)
    Dt = r.D.reshape(5, 5, 4)
    lam_d, _ = _svd_spectra(X, 64)
    for j, rd in enumerate(RD):
        assert abs(Dt[4, j, 0] - lam_d[rd:].sum() / lam_d.sum()) < 1e-12


def test_eckart_young_single_slice():
    rng = np.random.default_rng(2)
    T, D = 64, 64
    X = rng.standard_normal((1, T, D)) @ np.diag(np.arange(1, D + 1) ** -0.7) @ np.linalg.qr(rng.standard_normal((D, D)))[0]
    sigma = np.ones(D, np.int8)
    r = O.build_table(X, sigma, RT, RD, (0,), 64, round_fp16=False)
    s = np.linalg.svd(X[0], compute_uv=False) ** 2
    Dt = r.D.reshape(5, 5)
    for i, rT in enumerate(RT):
        for j, rd in enumerate(RD):
            k = min(rT, rd)
            assert abs(Dt[i, j] - s[k:].sum() / s.sum()) < 1e-12, (rT, rd)


def test_full_rank_candidate_is_lossless_and_costs_the_raw_tensor():
    X, sigma = _tiny()
    r = O.build_table(X, sigma, RT, RD, BITS, 64)
    Dt = r.D.reshape(5, 5, 4)
    assert np.all(Dt[4, 4, :] == 0.0)
    N, T, D = X.shape
    assert r.C.reshape(5, 5, 4)[4, 4, 0] == 256 + 2 * N * T * D


def test_monotone_in_both_ranks_without_rounding():
    X, sigma = _tiny()
    r = O.build_table(X, sigma, RT, RD, BITS, 64, round_fp16=False)
    D0 = r.D.reshape(5, 5, 4)[:, :, 0]
    assert np.all(np.diff(D0, axis=0) <= 1e-15)
    assert np.all(np.diff(D0, axis=1) <= 1e-15)


def test_two_bits_never_worse_than_no_residual():
    X, sigma = _tiny()
    r = O.build_table(X, sigma, RT, RD, BITS, 64)
    Dt = r.D.reshape(5, 5, 4)
    assert np.all(Dt[..., 1] <= Dt[..., 0])
    # and more bits help on average on this data (high-rate behaviour)
    assert np.all(Dt[..., 3][Dt[..., 0] > 0] < Dt[..., 2][Dt[..., 0] > 0])


def test_rotated_domain_score_equals_direct_distortion():
    """The table entry (rotated-domain sum) equals ||X - X^||^2/||X||^2 computed on the
    explicitly decoded cache X^ = X~ + Q^T Q_b(Q R) with a dense rotation matrix."""
    X, sigma = _tiny()
    N, T, D = X.shape
    r = O.build_table(X, sigma, RT, RD, BITS, 64, keep_factors=True)
    Dt = r.D.reshape(5, 5, 4)
    Qd = O.rotation_matrix(sigma)
    for (i, rT), (j, rd) in [((1, 8), (2, 16)), ((3, 32), (4, 64)), ((4, 64), (0, 4)), ((0, 4), (3, 32))]:
        Ut, Ud, G = O._factors_for(X, r.Ud, r.UT[rd], rT, rd)
        Xt = O.reconstruct(Ut, Ud, G)
        for k, b in enumerate(BITS):
            Y = (X - Xt) @ Qd.T
            _, _, Yh = O.quantize_blocks(Y, b, 64)
            Xhat = Xt + Yh @ Qd
            direct = np.sum((X - Xhat) ** 2) / np.sum(X ** 2)
            assert abs(direct - Dt[i, j, k]) <= 1e-12 * max(direct, 1e-300), (rT, rd, b)
            e = O.Encoded(rT, rd, b, 64, sigma, Ut, Ud, G, None, *O.encode_with_factors(X, sigma, Ut, Ud, G, b, 64)[:2])
            dec = O.decode_f64(e)
            assert abs(np.sum((X - dec) ** 2) / np.sum(X ** 2) - Dt[i, j, k]) <= 1e-12 * max(direct, 1e-300)
            if b == 0:
                assert np.array_equal(dec, Xt)


def test_energy_gap_is_rounding_level():
    X, sigma = _tiny()
    r = O.build_table(X, sigma, RT, RD, BITS, 64)
    assert np.max(np.abs(r.energy_gap)) < 1e-12 * r.xnorm2


def test_feature_factor_matches_svd_subspace():
    X, _ = _tiny()
    N, T, D = X.shape
    lam, U = O.feature_factor(X)
    _, s, Vt = np.linalg.svd(X.reshape(N * T, D), full_matrices=False)
    assert np.allclose(lam, s ** 2, rtol=1e-10)
    for k in (4, 8, 16, 32):
        P1 = U[:, :k] @ U[:, :k].T
        P2 = Vt[:k].T @ Vt[:k]
        assert np.max(np.abs(P1 - P2)) < 1e-8
    # sign convention: largest-magnitude entry of each vector is positive
    idx = np.argmax(np.abs(U), axis=0)
    assert np.all(U[idx, np.arange(D)] > 0)


@pytest.mark.parametrize("rd", [4, 8])
def test_randomized_equals_exact_when_sketch_spans_unfolding(rd):
    """N * r_d <= 40 sketch columns: the range finder captures the whole token unfolding,
    so the randomized token factor gives the exact candidate distortions."""
    X, sigma = _tiny()
    w = ks.get_workload("tiny")
    omegas = {r: ks.sketch_omega(w, 0, 0, r) for r in RD}
    ex = O.build_table(X, sigma, RT, RD, BITS, 64, "exact", round_fp16=False)
    rn = O.build_table(X, sigma, RT, RD, BITS, 64, "randomized", omegas=omegas, round_fp16=False)
    j = RD.index(rd)
    a = ex.D.reshape(5, 5, 4)[:, j, 0]
    b = rn.D.reshape(5, 5, 4)[:, j, 0]
    assert np.allclose(a, b, rtol=1e-10, atol=1e-14)


def test_randomized_close_to_exact_on_larger_unfolding():
    X, sigma = _tiny()
    w = ks.get_workload("tiny")
    omegas = {r: ks.sketch_omega(w, 0, 0, r) for r in RD}
    ex = O.build_table(X, sigma, RT, RD, BITS, 64, "exact")
    rn = O.build_table(X, sigma, RT, RD, BITS, 64, "randomized", omegas=omegas)
    # randomized can only lose energy relative to the exact top subspace (b = 0)
    a = ex.D.reshape(5, 5, 4)[..., 0]
    b = rn.D.reshape(5, 5, 4)[..., 0]
    assert np.all(b >= a * (1 - 1e-3))
    assert np.all(b <= a * 1.5 + 1e-12)


def test_row_sampled_decode_and_encode_equal_full_versions():
    X, sigma = _tiny()
    for z in [(8, 16, 4), (64, 8, 8), (16, 64, 2), (4, 4, 0)]:
        e = O.encode(X, sigma, *z, 64)
        full = O.decode_f64(e)
        rng = np.random.default_rng(1)
        n_idx = rng.integers(0, X.shape[0], 20)
        t_idx = rng.integers(0, X.shape[1], 20)
        assert np.allclose(O.decode_rows_f64(e, n_idx, t_idx), full[n_idx, t_idx], rtol=0, atol=1e-12)
        if z[2]:
            q, s = O.encode_rows(X[n_idx, t_idx], e, n_idx, t_idx)
            assert np.array_equal(q, e.codes[n_idx, t_idx]) and np.array_equal(s[:, 0], e.scales[n_idx, t_idx, 0])


# ------------------------------------------------------------ randomized range finder
def _power_sketch_factor(A, Om, q, k):
    """Top-k left singular vectors of A restricted to span((A A^T)^q A Omega), with the
    power formed explicitly by matrix powers (no re-orthonormalisation in between): the
    subspace that q rounds of subspace iteration on the sketch A Omega reach in exact
    arithmetic (Halko, Martinsson and Tropp, randomized subspace iteration)."""
    K = np.linalg.matrix_power(A @ A.T, q) @ (A @ Om)
    Qk, _ = np.linalg.qr(K)
    UB, _, _ = np.linalg.svd(Qk.T @ A, full_matrices=False)
    return Qk @ UB[:, :k]


def _proj_gap(U, V):
    return float(np.max(np.abs(U @ U.T - V @ V.T)))


def test_range_finder_reaches_the_twice_power_iterated_sketch():
    """A 48 x 40 matrix of known, slowly decaying singular values 0.85^i and a 10-column
    sketch: the oracle's factor with two power iterations spans exactly the top-4 singular
    directions of A within span((A A^T)^2 A Omega).  The same construction with one or three
    powers is measurably different, so a wrong loop count cannot pass."""
    rng = np.random.default_rng(5)
    T, M, l, k = 48, 40, 10, 4
    U, _ = np.linalg.qr(rng.standard_normal((T, T)))
    V, _ = np.linalg.qr(rng.standard_normal((M, M)))
    A = (U[:, :M] * 0.85 ** np.arange(M)) @ V.T
    Om = rng.standard_normal((M, l))
    got = O.token_factor_randomized(A, Om, 2, k)
    assert _proj_gap(got, _power_sketch_factor(A, Om, 2, k)) < 1e-10
    for q in (0, 1, 3):
        assert _proj_gap(got, _power_sketch_factor(A, Om, q, k)) > 1e-4, q
    # orthonormal columns
    assert np.max(np.abs(got.T @ got - np.eye(k))) < 1e-12


def test_table_build_uses_two_power_iterations():
    """The token factor that build_table computes for the unprojected chain (r_d = D) of the
    tiny table in randomized mode, against the explicit power sketch of its token unfolding
    A[t, n D + j] = X[n, t, j] with the same Omega: q = 2 (the count the FlashJoLT setting
    fixes) matches at every nested rank, q = 1 and q = 3 do not."""
    X, sigma = _tiny()
    N, T, D = X.shape
    w = ks.get_workload("tiny")
    omegas = {r: ks.sketch_omega(w, 0, 0, r) for r in RD}
    res = O.build_table(X, sigma, RT, RD, BITS, 64, "randomized", omegas=omegas, keep_factors=True)
    A = np.concatenate([X[n] for n in range(N)], axis=1)  # column n*D + j is X[n, :, j]
    Om = O.bf16_bits_to_f64(omegas[D])
    UT = res.UT[D]
    assert UT.shape == (T, 32)
    for kk in (4, 8, 16, 32):
        assert _proj_gap(UT[:, :kk], _power_sketch_factor(A, Om, 2, kk)) < 1e-6, kk
    for q in (1, 3):
        assert _proj_gap(UT, _power_sketch_factor(A, Om, q, 32)) > 1e-2, q
