"""Host-side checks of libjolt.so (no GPU needed): every symbol the headers declare
is exported, the byte costs and the lambda allocation equal the oracle's, and the
argument checks return the documented status codes."""
import ctypes
import os
import re

import numpy as np
import pytest

import kvsynth as ks
import partial_tucker_rotated_amd as J
from oracle import jolt_oracle as O

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")


def _declared():
    names = set()
    for h in ("jolt.h", "jolt_debug.h"):
        txt = open(os.path.join(INCLUDE, h)).read()
        names.update(re.findall(r"^\s*(?:jolt_status|void|const char\*)\s+(jolt_\w+)\s*\(", txt, re.M))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = J.load()
    declared = _declared()
    assert len(declared) >= 11
    missing = [n for n in declared if not hasattr(lib, n)]
    assert not missing, missing
    assert set(J.EXPORTED_SYMBOLS) <= set(declared)


@pytest.mark.parametrize("name", list(ks.WORKLOADS))
def test_cost_table_equals_oracle(name):
    w = ks.get_workload(name)
    cfg = J.default_config(w.N, w.T, w.D, w.n_tables,
                           J.TOKEN_EXACT if w.token_mode == "exact" else J.TOKEN_RANDOMIZED)
    C = J.cost_table(cfg)
    assert np.array_equal(C, O.cost_table(w.N, w.T, w.D, w.rT, w.rd, w.bits, w.quant_block))
    for i in (0, 37, 99):
        assert J.record_bytes(cfg, i) == int(C[i])


def test_allocation_equals_oracle_on_oracle_tables():
    w = ks.get_workload("tiny")
    X = O.bf16_bits_to_f64(ks.generate_table(w, 0, 0))
    r = O.build_table(X, ks.rotation_signs(w, 0, 0), w.rT, w.rd, w.bits, w.quant_block)
    for frac in (0.15, 0.3, 0.5, 0.8):
        B = int(frac * ks.fp16_bytes(w))
        a = O.allocate(r.D[None, :], r.C[None, :], B)
        ch, lam, tot = J.allocate(r.D[None, :], r.C[None, :], B)
        assert ch[0] == a.choice[0] and tot == a.total
        assert (a.lam == 0 and lam == 0) or abs(lam / a.lam - 1) < 1e-9


@pytest.mark.parametrize("seed", range(6))
def test_allocation_equals_oracle_many_tables(seed):
    rng = np.random.default_rng(seed)
    w = ks.get_workload("mistral_t512")
    C = O.cost_table(w.N, w.T, w.D, w.rT, w.rd, w.bits, w.quant_block)
    nt = 16
    Ct = np.tile(C, (nt, 1))
    # distortion falling with cost, table-dependent slope, noise
    D = np.exp(-Ct.astype(float) / (1e6 * np.exp(rng.standard_normal((nt, 1))))) * np.exp(0.2 * rng.standard_normal((nt, 100)))
    for ratio in (2.0, 3.0, 5.0):
        B = int(ks.fp16_bytes(w) / ratio)
        a = O.allocate(D, Ct, B)
        ch, lam, tot = J.allocate(D, Ct, B)
        assert np.array_equal(ch, a.choice) and tot == a.total <= B


@pytest.mark.parametrize("seed", range(4))
def test_allocation_equals_oracle_with_ties_and_distinct_cost_rows(seed):
    """Tables whose cost rows differ (and repeat), with many equal costs and equal
    distortions inside a table: the library's ordering of candidates by (cost, distortion,
    index) and its price search give the oracle's choice."""
    rng = np.random.default_rng(100 + seed)
    nt, nc = 12, 100
    rows = [rng.integers(1, 40, nc).astype(np.uint64) for _ in range(3)]
    Ct = np.stack([rows[t % 3] if t % 4 else rng.integers(1, 40, nc).astype(np.uint64) for t in range(nt)])
    D = rng.integers(0, 6, (nt, nc)).astype(np.float64) / 5.0
    for frac in (0.2, 0.5, 0.8):
        B = int(Ct.min(axis=1).sum() + frac * (Ct.max(axis=1).sum() - Ct.min(axis=1).sum()))
        a = O.allocate(D, Ct, B)
        ch, lam, tot = J.allocate(D, Ct, B)
        assert np.array_equal(ch, a.choice) and tot == a.total <= B


def test_allocation_errors():
    D = np.array([[0.5, 0.1]])
    C = np.array([[100, 400]], np.uint64)
    with pytest.raises(J.JoltError) as e:
        J.allocate(D, C, 99)
    assert e.value.name == "JOLT_EINFEASIBLE"
    with pytest.raises(J.JoltError) as e:
        J.allocate(np.array([[np.nan, 0.1]]), C, 1000)
    assert e.value.name == "JOLT_EINVAL"


@pytest.mark.parametrize("field,value", [("D", 96), ("T", 100), ("T", 32), ("quant_block", 64), ("s_bytes", 4),
                                         ("align_bytes", 128), ("q_cap", 16), ("n_tables", 0), ("n_tables", 65),
                                         ("factor_precision", 3), ("token_mode", 7), ("exact_iters", 0)])
def test_invalid_configs_rejected(field, value):
    cfg = J.default_config(32, 512, 128, 4)
    setattr(cfg, field, value)
    with pytest.raises(J.JoltError) as e:
        J.workspace_size(cfg)
    assert e.value.name == "JOLT_EINVAL"


def test_randomized_needs_enough_sketch_rows():
    cfg = J.default_config(4, 64, 64, 1, J.TOKEN_RANDOMIZED)
    with pytest.raises(J.JoltError):
        J.workspace_size(cfg)


def test_small_workspace_and_null_pointers_rejected_before_device_work():
    lib = J.load()
    cfg = J.default_config(4, 64, 64, 1)
    D = np.zeros((1, 100))
    C = np.zeros((1, 100), np.uint64)
    fake = (ctypes.c_void_p * 1)(0x1000)
    code = lib.jolt_build_tables(ctypes.byref(cfg), fake, ctypes.c_void_p(0x2000), None, D.ctypes.data,
                                 C.ctypes.data, None, ctypes.c_void_p(0x3000), 16, None)
    assert code == -2  # JOLT_ENOMEM
    code = lib.jolt_build_tables(ctypes.byref(cfg), fake, None, None, D.ctypes.data, C.ctypes.data, None,
                                 ctypes.c_void_p(0x3000), 1 << 30, None)
    assert code == -1  # JOLT_EINVAL
    assert lib.jolt_status_string(-4) == b"budget below the cheapest allocation"


def test_encode_built_needs_a_build_on_that_workspace():
    """Without a prior successful build on the workspace the reuse entry point refuses
    (host-side check, no device work)."""
    lib = J.load()
    cfg = J.default_config(4, 64, 64, 1)
    fake = (ctypes.c_void_p * 1)(0x1000)
    recs = (ctypes.c_void_p * 1)(0x4000)
    ch = np.zeros(1, np.int32)
    code = lib.jolt_encode_built(ctypes.byref(cfg), fake, ctypes.c_void_p(0x2000), ch.ctypes.data, recs,
                                 ctypes.c_void_p(0x3000), 1 << 30, None)
    assert code == -1  # JOLT_EINVAL
    ch[0] = 100
    code = lib.jolt_encode_built(ctypes.byref(cfg), fake, ctypes.c_void_p(0x2000), ch.ctypes.data, recs,
                                 ctypes.c_void_p(0x3000), 1 << 30, None)
    assert code == -1


def test_workspace_grows_with_workload():
    small = J.workspace_size(J.default_config(32, 512, 128, 16))
    big = J.workspace_size(J.default_config(32, 1024, 128, 16, J.TOKEN_RANDOMIZED))
    assert 0 < small < 1 << 30 and big > 0


def _tables(seed, nt=16):
    rng = np.random.default_rng(seed)
    w = ks.get_workload("mistral_t512")
    C = O.cost_table(w.N, w.T, w.D, w.rT, w.rd, w.bits, w.quant_block)
    Ct = np.tile(C, (nt, 1))
    D = np.exp(-Ct.astype(float) / (1e6 * np.exp(rng.standard_normal((nt, 1))))) * \
        np.exp(0.2 * rng.standard_normal((nt, Ct.shape[1])))
    return w, D, Ct


@pytest.mark.parametrize("seed", range(6))
def test_refine_swap_equals_oracle(seed):
    """Greedy swap after the bisection: the same moves as the oracle (both rank moves by the
    same fp64 expression), from the library's own bisection allocation."""
    w, D, Ct = _tables(seed)
    for ratio in (2.0, 3.0, 5.0):
        B = int(ks.fp16_bytes(w) / ratio)
        ch0, _, tot0 = J.allocate(D, Ct, B)
        ref, ref_tot = O.refine_swap(D, Ct, B, ch0)
        ch, tot, moves = J.refine_swap(D, Ct, B, ch0)
        assert np.array_equal(ch, ref) and tot == ref_tot <= B
        assert D[np.arange(len(ch)), ch].sum() <= D[np.arange(len(ch0)), ch0].sum()
        assert (moves == 0) == np.array_equal(ch, ch0)


def test_refine_swap_hand_worked_through_the_library():
    D = np.array([[10.0, 4.0, 3.9], [5.0, 2.0, 1.0]])
    C = np.array([[1, 3, 4], [1, 2, 5]], np.uint64)
    ch, tot, moves = J.refine_swap(D, C, 5, [0, 0])
    assert list(ch) == [1, 1] and tot == 5 and moves == 2
    ch, tot, moves = J.refine_swap(np.array([[5.0, 4.0, 1.0]]), np.array([[2, 2, 3]], np.uint64), 3, [0])
    assert list(ch) == [2] and tot == 3 and moves == 2


def test_refine_swap_errors():
    D = np.array([[0.5, 0.1]])
    C = np.array([[100, 400]], np.uint64)
    for start, budget in (([1], 300), ([2], 1000), ([-1], 1000)):
        with pytest.raises(J.JoltError) as e:
            J.refine_swap(D, C, budget, start)
        assert e.value.name == "JOLT_EINVAL"


@pytest.mark.parametrize("seed", range(4))
def test_allocate_common_equals_oracle(seed):
    """The shared-candidate baselines (all candidates, fixed b, fixed ranks) equal the oracle's
    wherever its best and second-best totals differ by more than 1e-12 relative (the library
    sums in table order, the oracle exactly)."""
    w, D, Ct = _tables(100 + seed)
    cands = O.candidate_list(w.T, w.D, w.rT, w.rd, w.bits)
    masks = [None] + [np.array([c[2] == b for c in cands]) for b in w.bits] + \
            [np.array([c[0] == 32 and c[1] == 32 for c in cands])]
    for ratio in (2.0, 3.0, 5.0):
        B = int(ks.fp16_bytes(w) / ratio)
        for mask in masks:
            try:
                ref = O.allocate_common(D, Ct, B, mask)
            except ValueError:
                with pytest.raises(J.JoltError) as e:
                    J.allocate_common(D, Ct, B, mask)
                assert e.value.name == "JOLT_EINFEASIBLE"
                continue
            i, tot, dist = J.allocate_common(D, Ct, B, mask)
            tots = sorted(float(D[:, j].sum()) for j in range(D.shape[1])
                          if (mask is None or mask[j]) and int(Ct[:, j].sum()) <= B)
            if len(tots) > 1 and tots[1] - tots[0] <= 1e-12 * tots[1]:
                continue
            assert i == ref and tot == int(Ct[:, i].sum()) <= B
            assert abs(dist - D[:, i].sum()) <= 1e-12 * dist


@pytest.mark.parametrize("name,tn", [("tiny", 64), ("mistral_t512", 256), ("mistral_t512", 320)])
def test_stream_block_bytes_equal_oracle(name, tn):
    """Block record sizes of every candidate equal the oracle's byte count of the layout."""
    w = ks.get_workload(name)
    cfg = J.default_config(w.N, w.T, w.D, 1, J.TOKEN_EXACT)
    cands = O.candidate_list(w.T, w.D, w.rT, w.rd, w.bits)
    for i, (rT, rd, b) in enumerate(cands):
        assert J.stream_block_bytes(cfg, i, tn) == O.block_bytes(w.N, tn, w.D, w.T, rT, rd, b, w.D), i
    # error sums per (slice, 256-token chunk), then the left-factor partial sums of at most
    # eight slice groups per 64-token tile (32 x 64 fp64 each)
    ng = min(w.N, 8)
    assert J.stream_workspace_size(cfg, tn) == 8 * (2 * w.N * -(-tn // 256) + ng * (tn // 64) * 2048)
    assert J.stream_state_bytes() == 8 * (32 * 32 + 32)


def test_stream_argument_errors_before_device_work():
    cfg = J.default_config(4, 64, 64, 1, J.TOKEN_EXACT)
    for tn in (0, 32, 100, 65600):
        with pytest.raises(J.JoltError) as e:
            J.stream_block_bytes(cfg, 5, tn)
        assert e.value.name == "JOLT_EINVAL"
    with pytest.raises(J.JoltError):
        J.stream_block_bytes(cfg, 100, 64)
    lib = J.load()
    assert lib.jolt_stream_prepare(ctypes.byref(cfg), None, None, None, None) == -1
    assert lib.jolt_stream_encode(ctypes.byref(cfg), None, None, None, None, 64, None, None, None, 0, None) == -1
    assert lib.jolt_stream_decode(ctypes.byref(cfg), None, None, None, 64, None, None) == -1


def _stored_oracle_tables():
    import glob
    import json
    out = []
    for path in sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "oracle_tables_*.json"))):
        g = json.load(open(path))
        if g.get("allocations"):
            out.append((os.path.basename(path), g))
    return out


@pytest.mark.parametrize("name,gold", _stored_oracle_tables(), ids=lambda v: v if isinstance(v, str) else "")
def test_price_search_on_the_oracle_tables_equals_the_oracle(name, gold):
    """jolt_allocate on the oracle's own full-size tables (every budget of the workload)
    returns exactly the oracle's allocation: the same candidate on every table, the same
    total bytes."""
    D = np.array([[float(v) for v in t["D"]] for t in gold["tables"]])
    C = np.array([t["C"] for t in gold["tables"]], np.uint64)
    assert len(gold["allocations"]) >= 1
    for a in gold["allocations"]:
        ch, lam, tot = J.allocate(D, C, a["budget"])
        assert np.array_equal(ch, np.array(a["choice"])), (name, a["budget"])
        assert tot == a["total"] <= a["budget"]
