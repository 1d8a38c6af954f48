"""GPU parity of the modelled candidate tables (jolt_model_tables) against the oracle's
separable error model D(z) = eps^2(b) tau(r_T, r_d) on the same seeded inputs.

The quantizer factor eps^2(b) is decided in fp64 on both sides from the same fp32
Gaussian rows and must agree to summation order (1e-12 relative).  tau comes from the
feature and token eigenvalues: fp64 factors meet 1e-3 relative; fp32 factors add an
absolute allowance of eps^2(b) 2^-19, a few times the fp32 resolution of the energy
ratios (the captured energy is a sum of eigenvalues of a Gram whose largest eigenvalue
is at most ||X||^2).
"""
import numpy as np
import pytest

import kvsynth as ks
from oracle import jolt_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BITS = (0, 2, 4, 8)


def _run(w, ids, N, T, precision, rows=4096):
    import partial_tucker_rotated_amd as J
    print(f"model tables {w.name} tables={ids} N={N} T={T} precision={precision}", flush=True)
    D = w.D
    xb = [np.ascontiguousarray(ks.generate_table(w, g, c)[:N, :T]) for g, c in ids]
    sg = np.stack([ks.rotation_signs(w, g, c) for g, c in ids])
    mode = J.TOKEN_EXACT if w.token_mode == "exact" else J.TOKEN_RANDOMIZED
    rds = (4, 8, 16, 32, D)
    oms, omh = None, []
    if mode == J.TOKEN_RANDOMIZED:
        oms = []
        for g, c in ids:
            blocks = {r: ks.sketch_omega(w, g, c, r)[: N * r] for r in rds}
            omh.append(blocks)
            oms.append(torch.from_numpy(np.concatenate([blocks[r].reshape(-1) for r in rds]).view(np.int16)).cuda())
    cfg = J.default_config(N, T, D, len(ids), mode, factor_precision=precision)
    ws = torch.empty(J.workspace_size(cfg), dtype=torch.uint8, device="cuda")
    G = ks.gaussian_rows(D, rows)
    xs = [torch.from_numpy(b.view(np.int16)).cuda() for b in xb]
    Dm, C, xn, e2 = J.model_tables(cfg, xs, torch.from_numpy(sg).cuda(), oms, torch.from_numpy(G).cuda(), ws)
    torch.cuda.synchronize()
    eps_o = O.gaussian_eps2(G, BITS)
    np.testing.assert_allclose(e2, [eps_o[b] for b in BITS], rtol=1e-12, atol=0)
    C_o = O.cost_table(N, T, D, (4, 8, 16, 32, T), rds, BITS, D)
    tol_abs = 0.0 if precision == 1 else 2.0 ** -19
    for k in range(len(ids)):
        X = O.bf16_bits_to_f64(xb[k])
        ref = O.model_table(X, (4, 8, 16, 32, T), rds, BITS, eps_o, w.token_mode,
                            omh[k] if omh else None, w.power_iters)
        assert np.array_equal(C[k], np.asarray(C_o, np.uint64))
        # ||X||^2 from fp32 partial sums of exact bf16 products, added in fp64
        assert xn[k] == pytest.approx(float(np.sum(X * X)), rel=1e-6)
        zero = ref == 0
        assert np.all(Dm[k][zero] == 0.0)
        ebits = np.array([eps_o[b] for b in BITS] * (len(ref) // len(BITS)))
        err = np.abs(Dm[k] - ref)
        bound = 1e-3 * ref + tol_abs * ebits
        worst = int(np.argmax(err - bound))
        assert np.all(err <= bound), (k, worst, Dm[k][worst], ref[worst])


def test_model_tables_exact_short_window():
    # T = 128: token factors by the direct eigensolver
    _run(ks.get_workload("mistral_t512"), [(0, 0), (0, 1)], N=8, T=128, precision=0)


@pytest.mark.parametrize("precision", [0, 1])
def test_model_tables_exact_subspace(precision):
    # T = 512: token factors by subspace iteration (the r_d = D chain on the side stream)
    _run(ks.get_workload("mistral_t512"), [(1, 0), (1, 1)], N=8, T=512, precision=precision)


def test_model_tables_randomized():
    # the range finder needs 4 N >= 40 sketch columns
    _run(ks.get_workload("mistral_t1024_flash"), [(0, 0), (2, 1)], N=16, T=1024, precision=0)


def test_model_tables_tiny_fp64():
    _run(ks.get_workload("tiny"), [(0, 0)], N=4, T=64, precision=1, rows=512)


def test_model_tables_rejects_bad_arguments():
    import partial_tucker_rotated_amd as J
    w = ks.get_workload("tiny")
    cfg = J.default_config(4, 64, 64, 1, J.TOKEN_EXACT)
    ws = torch.empty(J.workspace_size(cfg), dtype=torch.uint8, device="cuda")
    xs = [torch.zeros((4, 64, 64), dtype=torch.int16, device="cuda")]
    sg = torch.ones((1, 64), dtype=torch.int8, device="cuda")
    with pytest.raises(ValueError):
        J.model_tables(cfg, xs, sg, None, torch.zeros((8, 32), dtype=torch.float32, device="cuda"), ws)
    with pytest.raises(J.JoltError):
        J.model_tables(cfg, xs, sg, None, torch.zeros((0, 64), dtype=torch.float32, device="cuda"), ws)
