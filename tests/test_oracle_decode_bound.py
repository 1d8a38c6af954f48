"""Pins of the oracle's acceptance of a decode evaluated in fp32: bf16_consistent (brute
force over neighbouring bf16 values) and decode_eval_bound (an fp32 evaluation of the
decoded rows, in two different summation orders, stays within the bound, also on rows built
to cancel to zero)."""
import numpy as np
import pytest

from oracle import jolt_oracle as O


def _bits_add(b, k):
    """bf16 bits k steps along the ordered line from b (positive values only here)."""
    return (b.astype(np.int64) + k).astype(np.uint16)


def test_bf16_consistent_without_bound_is_one_ulp():
    rng = np.random.default_rng(0)
    x = np.abs(rng.standard_normal(2000)) + 0.1
    w = O.f64_to_bf16_bits(x)
    zero = np.zeros_like(x)
    for k, ok in ((0, True), (1, True), (-1, True), (2, False), (-2, False)):
        assert np.all(O.bf16_consistent(_bits_add(w, k), x, zero) == ok), k


def test_bf16_consistent_accepts_exactly_the_roundings_inside_the_bound():
    x = np.array([1e-6, -3e-7, 0.0, 2.5])
    bound = np.array([1e-5, 1e-6, 1e-9, 1e-9])
    inside = O.f64_to_bf16_bits(np.array([-5e-6, 6e-7, -8e-10, 2.5]))
    outside = O.f64_to_bf16_bits(np.array([2e-5, 1e-5, 5e-9, 2.53]))
    assert O.bf16_consistent(inside, x, bound).all()
    assert not O.bf16_consistent(outside, x, bound).any()


def _record(rng, kind, b, N=3, T=64, D=64):
    sigma = np.where(rng.random(D) < 0.5, -1, 1).astype(np.int8)
    if kind == "rd":        # r_T < T, r_d < D
        Ut, Ud, G = O.fp16_round(0.3 * rng.standard_normal((T, 16))), O.fp16_round(0.3 * rng.standard_normal((D, 8))), \
            O.fp16_round(5 * rng.standard_normal((N, 16, 8)))
    elif kind == "full_d":  # r_T < T, r_d = D
        Ut, Ud, G = O.fp16_round(0.3 * rng.standard_normal((T, 32))), None, O.fp16_round(rng.standard_normal((N, 32, D)))
    else:                   # r_T = T
        Ut, Ud, G = None, O.fp16_round(0.3 * rng.standard_normal((D, 32))), O.fp16_round(rng.standard_normal((N, T, 32)))
    codes = scales = None
    if b:
        codes = rng.integers(-(1 << (b - 1)), 1 << (b - 1), size=(N, T, D))
        scales = O.f32_round(0.01 * rng.random((N, T, 1)))
    return O.Encoded(0, 0, b, D, sigma, Ut, Ud, G, None, codes, scales)


def _fp32_decode(e, order):
    """X^ of every row in fp32: Rm, then L Rm, then the unrotated residual, each product
    summed in fp32 (np.float32 arithmetic), in forward or reversed k order."""
    f = np.float32
    G = e.G.astype(f)
    N = G.shape[0]
    if e.Ut is None:  # X~_n = G_n U_d^T: L = the per-token core rows, Rm = U_d^T
        Ls = [G[:, :, k] for k in range(G.shape[2])]
        Rs = [np.broadcast_to(e.Ud[:, k].astype(f), (N, e.Ud.shape[0])) for k in range(G.shape[2])]
    else:             # X~_n = U_T (G_n U_d^T): L = U_T, Rm = G_n U_d^T (or G_n)
        Rm = G if e.Ud is None else np.einsum("nkj,fj->nkf", G, e.Ud.astype(f)).astype(f)
        Ls = [np.broadcast_to(e.Ut[:, k].astype(f), (N, e.Ut.shape[0])) for k in range(e.Ut.shape[1])]
        Rs = [Rm[:, k, :] for k in range(Rm.shape[1])]
    ks = range(len(Ls)) if order > 0 else range(len(Ls) - 1, -1, -1)
    acc = None
    for k in ks:
        term = (Ls[k][..., None] * Rs[k][:, None, :]).astype(f)
        acc = term if acc is None else (acc + term).astype(f)
    if e.b:
        D = acc.shape[2]
        Q = O.rotation_matrix(e.sigma).astype(f)
        Yh = (e.codes * e.scales).astype(f)
        acc = (acc + (Yh.reshape(-1, D) @ Q).reshape(acc.shape).astype(f)).astype(f)
    return acc.astype(np.float64)


@pytest.mark.parametrize("kind", ["rd", "full_d", "full_t"])
@pytest.mark.parametrize("b", [0, 4, 8])
def test_fp32_evaluation_stays_inside_the_bound(kind, b):
    rng = np.random.default_rng(hash((kind, b)) % 2 ** 32)
    e = _record(rng, kind, b)
    N, T = e.G.shape[0], (e.Ut.shape[0] if e.Ut is not None else e.G.shape[1])
    n_idx, t_idx = np.meshgrid(np.arange(N), np.arange(T), indexing="ij")
    n_idx, t_idx = n_idx.reshape(-1), t_idx.reshape(-1)
    exact = O.decode_rows_f64(e, n_idx, t_idx)
    bound = O.decode_eval_bound(e, n_idx, t_idx)
    assert np.all(bound > 0) and np.all(bound < 1e-4 * np.abs(exact).max())
    for order in (1, -1):
        got = _fp32_decode(e, order).reshape(-1, exact.shape[1])
        assert np.all(np.abs(got - exact) <= bound), order


def test_bound_holds_on_rows_that_cancel_to_zero():
    """Token rows of U_T chosen so that X~ of every row is a difference of two large equal
    terms: the exact value is tiny, the fp32 evaluation is off by the rounding of the large
    terms, and the bound covers it."""
    rng = np.random.default_rng(3)
    N, T, D = 2, 64, 64
    e = _record(rng, "full_d", 0, N=N, T=T, D=D)
    Ut = e.Ut.copy()
    Ut[:, 1] = Ut[:, 0]
    G = e.G.copy()
    G[:, 1, :] = -G[:, 0, :] + O.fp16_round(1e-3 * rng.standard_normal((N, D)))
    Ut[:, 2:] = 0.0
    e = O.Encoded(0, 0, 0, D, e.sigma, Ut, None, G, None, None, None)
    n_idx, t_idx = np.meshgrid(np.arange(N), np.arange(T), indexing="ij")
    n_idx, t_idx = n_idx.reshape(-1), t_idx.reshape(-1)
    exact = O.decode_rows_f64(e, n_idx, t_idx)
    bound = O.decode_eval_bound(e, n_idx, t_idx)
    got = _fp32_decode(e, 1).reshape(-1, D)
    assert np.all(np.abs(got - exact) <= bound)
    assert O.bf16_consistent(O.f64_to_bf16_bits(got), exact, bound).all()
