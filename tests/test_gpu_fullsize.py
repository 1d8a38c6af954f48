"""GPU parity at the full sizes of the five seeded workloads, against the oracle's tables
stored in tests/golden/oracle_tables_*.json (written by tests/golden/make_oracle_tables.py,
which calls only the oracle and the seeded generator).

Each test regenerates the inputs (their SHA-256 must equal the stored one), builds every
table on the GPU in the benchmark's launch configuration (all tables of the workload in one
call) and checks, from the acceptance statement of the engine:
  * every D(z) within 1e-3 relative of the oracle's (D = 0 entries exact);
  * every C(z) bit-exact, ||X||^2 within 1e-7 (the trace of the feature Gram, whose row
    chunks are summed in fp32);
  * at every budget of the workload, the allocation from the GPU's tables equal to the
    oracle's on every table whose Lagrangian margin exceeds 1e-6, within the budget.
"""
import hashlib

import numpy as np
import pytest

import _tables
import kvsynth as ks

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

D_TOL = 1e-3
MARGIN = 1e-6


def _lib():
    import partial_tucker_rotated_amd as J
    return J


def _build(name, mode, part=None):
    J = _lib()
    gold = _tables.golden(name, mode, part)
    assert gold is not None, f"no stored oracle tables for {name} ({mode})"
    w = ks.get_workload(name)
    idx = [e["table"] for e in gold["tables"]]
    ids = [w.table_ids()[t] for t in idx]
    print(f"case {name} {mode} tables={idx}", flush=True)
    xs = []
    for t, e in zip(idx, gold["tables"]):
        b = _tables.table(name, t)
        assert hashlib.sha256(np.ascontiguousarray(b).tobytes()).hexdigest() == e["sha256"], (name, t)
        xs.append(torch.from_numpy(b.view(np.int16)).cuda())
        del b
    signs = torch.from_numpy(np.stack([ks.rotation_signs(w, g, c) for g, c in ids])).cuda()
    tm = J.TOKEN_EXACT if mode == "exact" else J.TOKEN_RANDOMIZED
    oms = None
    if tm == J.TOKEN_RANDOMIZED:
        oms = [torch.from_numpy(np.concatenate([ks.sketch_omega(w, g, c, r).reshape(-1) for r in w.rd])
                                .view(np.int16)).cuda() for g, c in ids]
    cfg = J.default_config(w.N, w.T, w.D, len(ids), tm)
    ws = torch.empty(J.workspace_size(cfg), dtype=torch.uint8, device="cuda")
    D, C, xn = J.build_tables(cfg, xs, signs, oms, ws)
    info = J.last_build_info(ws)
    print(f"  token factors: {info}", flush=True)
    worst = 0.0
    for k, e in enumerate(gold["tables"]):
        Dr = np.array([float(v) for v in e["D"]])
        nz = Dr > 0
        assert np.all(D[k][~nz] == 0.0), (name, k)
        rel = np.abs(D[k][nz] - Dr[nz]) / Dr[nz]
        worst = max(worst, float(rel.max()))
        assert rel.max() < D_TOL, (name, k, int(np.where(nz)[0][np.argmax(rel)]), float(rel.max()))
        assert np.array_equal(C[k], np.array(e["C"], np.uint64)), (name, k)
        # ||X||^2 is the trace of the feature Gram, summed in fp32 within row chunks
        assert abs(xn[k] / float(e["xnorm2"]) - 1.0) < 1e-7, (name, k)
    print(f"  {len(idx)} tables: max rel D error {worst:.3e}", flush=True)
    del xs, ws
    torch.cuda.empty_cache()
    return D, C, gold, info


def _check_allocations(D, C, gold):
    J = _lib()
    for a in gold["allocations"]:
        B = a["budget"]
        ch, lam, tot = J.allocate(D, C, B)
        assert tot <= B
        want = np.array(a["choice"])
        margin = np.array([float(m) for m in a["margin"]])
        firm = margin > MARGIN
        bad = np.where(firm & (ch != want))[0]
        print(f"  budget {B}: {int(np.sum(ch == want))}/{len(ch)} choices equal, {int(firm.sum())} with margin "
              f"> {MARGIN:g}; GPU {tot} B, oracle {a['total']} B", flush=True)
        assert len(bad) == 0, [(int(k), int(ch[k]), int(want[k]), float(margin[k])) for k in bad]


def test_fullsize_mistral_t512_exact_all_tables():
    D, C, gold, info = _build("mistral_t512", "exact")
    _check_allocations(D, C, gold)
    assert info["converged"], info


def test_fullsize_mistral_t1024_randomized_all_tables():
    D, C, gold, _ = _build("mistral_t1024_flash", "randomized")
    _check_allocations(D, C, gold)


def test_fullsize_mistral_t1024_exact_all_tables():
    D, C, gold, info = _build("mistral_t1024_flash", "exact")
    _check_allocations(D, C, gold)
    assert info["converged"], info


def test_fullsize_llama13b_t2048_randomized_all_tables_both_budgets():
    D, C, gold, _ = _build("llama13b_t2048", "randomized")
    assert len(gold["allocations"]) == 2
    _check_allocations(D, C, gold)


def test_fullsize_llama13b_t2048_exact_two_tables():
    D, C, gold, info = _build("llama13b_t2048", "exact", part=0)
    assert info["converged"], info


def test_fullsize_mistral_t32k_randomized_all_tables():
    D, C, gold, _ = _build("mistral_t32k", "randomized")
    _check_allocations(D, C, gold)
