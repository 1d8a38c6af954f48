"""Pins of the oracle's byte cost and Lagrangian allocation: closed forms, the pages'
printed footprint, brute force over all allocations and Everett's theorem (CPU only)."""
import itertools
import os
import struct

import numpy as np
import pytest

from oracle import jolt_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split()
            out[k] = float(v)
    return out


def test_footprint_matches_printed_megabytes():
    g = _golden("footprint_mistral7b_ctx2048.txt")
    L, H, T, D = int(g["layers"]), int(g["kv_heads"]), int(g["tokens"]), int(g["head_dim"])
    fp16 = 2 * L * H * T * D * 2
    assert round(fp16 / 1e6, 1) == g["printed_fp16_megabytes"]
    # storing every (group, K/V) verbatim costs the fp16 bytes plus one header per table
    n_tables = (L // 4) * 2
    N = 4 * H
    verb = n_tables * O.candidate_cost(N, T, D, T, D, 0, 128)
    assert verb == fp16 + n_tables * O.HDR_BYTES
    assert round(verb / 1e6, 1) == g["printed_fp16_megabytes"]
    # a 2x budget is half of that, below the printed compressed footprint
    assert fp16 // 2 / 1e6 <= g["printed_2x_megabytes"]


def test_cost_closed_forms():
    N, T, D = 32, 512, 128
    # shared factors + core, no residual
    assert O.candidate_cost(N, T, D, 32, 32, 0, 128) == 256 + 2 * 512 * 32 + 2 * 128 * 32 + 2 * 32 * 32 * 32
    # the printed formula with per-slice factors would count s*N*(rT*T + rd*rT + rd*D)
    assert 2 * N * (32 * T + 32 * 32 + 32 * D) == 1376256
    # residual: b bits per value plus one fp32 scale per block of D values
    c4 = O.candidate_cost(N, T, D, 4, 4, 4, 128)
    c0 = O.candidate_cost(N, T, D, 4, 4, 0, 128)
    assert c4 - c0 == N * T * D // 2 + 4 * N * T
    # identity token factor: core is N x T x r_d and no token factor is stored
    assert O.candidate_cost(N, T, D, T, 8, 0, 128) == 256 + O.pad(2 * D * 8) + 2 * N * T * 8
    # alignment padding
    assert O.candidate_cost(4, 64, 64, 4, 4, 2, 64) == 256 + O.pad(2 * 64 * 4) + O.pad(2 * 64 * 4) + O.pad(2 * 4 * 16) + O.pad(2 * 4 * 64 * 64 // 8) + O.pad(4 * 4 * 64)
    assert O.pad(1) == 256 and O.pad(256) == 256 and O.pad(257) == 512


def test_candidate_order():
    c = O.candidate_list(64, 64, (4, 8, 16, 32, 64), (4, 8, 16, 32, 64), (0, 2, 4, 8))
    assert len(c) == 100
    assert c[0] == (4, 4, 0) and c[1] == (4, 4, 2) and c[4] == (4, 8, 0) and c[20] == (8, 4, 0) and c[99] == (64, 64, 8)


def _toy_tables(seed, nt=2, nc=100):
    rng = np.random.default_rng(seed)
    C = rng.integers(1000, 200000, size=(nt, nc)).astype(np.uint64)
    # distortion decreasing in cost with noise: a realistic rate-distortion cloud
    D = np.exp(-np.asarray(C, np.float64) / 40000.0) * np.exp(0.3 * rng.standard_normal((nt, nc)))
    return D, C


def _exhaustive(D, C, B):
    best = None
    for i, j in itertools.product(range(D.shape[1]), repeat=2):
        c = int(C[0, i]) + int(C[1, j])
        if c <= B:
            d = D[0, i] + D[1, j]
            if best is None or d < best[0]:
                best = (d, c, (i, j))
    return best


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_everett_lagrangian_is_optimal_at_its_own_budget(seed):
    D, C = _toy_tables(seed)
    B = int(0.5 * (int(C[0].min()) + int(C[1].min()) + int(C[0].max()) + int(C[1].max())) * 0.4)
    a = O.allocate(D, C, B)
    assert a.total <= B
    lag = D[0, a.choice[0]] + D[1, a.choice[1]]
    ex = _exhaustive(D, C, a.total)
    assert ex[0] == lag  # Everett: optimal for the budget it spends
    ex_b = _exhaustive(D, C, B)
    assert ex_b[0] <= lag  # duality gap at the requested budget is non-negative


@pytest.mark.parametrize("seed", [3, 4])
def test_price_is_minimal_and_total_monotone(seed):
    D, C = _toy_tables(seed, nt=5)
    B = int(np.sum(C.min(axis=1)) * 3)
    a = O.allocate(D, C, B)
    # any cheaper price overspends
    ch = O.lagrangian_choice(D, C, a.lam * (1 - 1e-9)) if a.lam > 0 else None
    if ch is not None:
        assert sum(int(C[t, ch[t]]) for t in range(5)) > B
    lams = np.geomspace(1e-9, 1e-3, 60)
    tots = [sum(int(C[t, c]) for t, c in enumerate(O.lagrangian_choice(D, C, l))) for l in lams]
    assert all(x >= y for x, y in zip(tots[:-1], tots[1:]))
    # margins are non-negative, and at a positive price one table sits at a tie
    assert np.all(a.margin >= 0)
    if a.lam > 0:
        assert np.min(a.margin) < 1e-12


def test_allocation_ties_and_zero_price():
    # candidate 0 and 1 identical; candidate 2 same distortion, higher cost
    D = np.array([[0.5, 0.5, 0.5, 0.1]])
    C = np.array([[100, 100, 150, 400]], np.uint64)
    a = O.allocate(D, C, 1000)
    assert a.lam == 0.0 and a.choice[0] == 3
    a = O.allocate(D, C, 399)
    assert a.choice[0] == 0 and a.total == 100
    assert abs(a.lam - 0.4 / 300) < 1e-18
    with pytest.raises(ValueError):
        O.allocate(D, C, 99)


def _write_record(N, T, D, rT, rd, b, blk, sigma, Ut, Ud, G, codes, scales):
    """Minimal writer of the documented record layout, used to pin the parser."""
    pad = O.pad
    off = 256
    secs = {}
    for name, arr in (("ut", Ut), ("ud", Ud), ("core", G)):
        if arr is not None:
            secs[name] = (off, arr.astype(np.float16).tobytes())
            off += pad(len(secs[name][1]))
    if b:
        u = (codes.reshape(-1) & ((1 << b) - 1)).astype(np.uint64)
        bitsarr = ((u[:, None] >> np.arange(b, dtype=np.uint64)[None, :]) & np.uint64(1)).astype(np.uint8)
        raw = np.packbits(bitsarr.reshape(-1), bitorder="little").tobytes()
        secs["codes"] = (off, raw); off += pad(len(raw))
        sb = scales.astype(np.float32).tobytes()
        secs["scales"] = (off, sb); off += pad(len(sb))
    buf = bytearray(off)
    struct.pack_into("<IIiiiiiiii", buf, 0, O.MAGIC, 1, N, T, D, rT, rd, b, blk, 0)
    struct.pack_into("<QQQQQQ", buf, 40, off, *(secs.get(k, (0, b""))[0] for k in ("ut", "ud", "core", "codes", "scales")))
    sb = np.packbits((np.asarray(sigma) < 0).astype(np.uint8), bitorder="little").tobytes()
    buf[128:128 + len(sb)] = sb
    for o, raw in secs.values():
        buf[o:o + len(raw)] = raw
    return bytes(buf)


@pytest.mark.parametrize("b", [0, 2, 4, 8])
def test_record_parser_roundtrip_and_size(b):
    rng = np.random.default_rng(b)
    N, T, D, rT, rd, blk = 3, 64, 64, 8, 16, 64
    sigma = np.where(rng.integers(0, 2, D) == 1, -1, 1)
    Ut = O.fp16_round(rng.standard_normal((T, rT)))
    Ud = O.fp16_round(rng.standard_normal((D, rd)))
    G = O.fp16_round(rng.standard_normal((N, rT, rd)))
    codes = rng.integers(-(1 << (b - 1)) + 1, 1 << (b - 1), size=(N, T, D)) if b else None
    scales = O.f32_round(rng.random((N, T, D // blk))) if b else None
    buf = _write_record(N, T, D, rT, rd, b, blk, sigma, Ut, Ud, G, codes, scales)
    assert len(buf) == O.candidate_cost(N, T, D, rT, rd, b, blk)
    e = O.parse_record(buf, N, T, D)
    assert np.array_equal(e.sigma, sigma) and np.array_equal(e.Ut, Ut) and np.array_equal(e.Ud, Ud) and np.array_equal(e.G, G)
    if b:
        assert np.array_equal(e.codes, codes) and np.array_equal(e.scales, scales)


# ------------------------------------------------------------------ greedy swap, baselines
def _read_swap_cases():
    path = os.path.join(os.path.dirname(__file__), "golden", "greedy_swap_toy.txt")
    cases, cur = [], None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, rest = line.partition(" ")
        if key == "case":
            cur = {"name": rest}
            cases.append(cur)
        elif key in ("costs", "dist"):
            cur[key] = [[float(v) for v in row.split()] for row in rest.split("/")]
        elif key == "moves":
            cur[key] = [tuple(int(v) for v in m.split(":")) for m in rest.split()]
        else:
            cur[key] = [int(v) for v in rest.split()]
    return cases


@pytest.mark.parametrize("case", _read_swap_cases(), ids=lambda c: c["name"])
def test_refine_swap_hand_worked(case):
    C = np.array(case["costs"], np.uint64)
    D = np.array(case["dist"])
    trace = []
    ch, tot = O.refine_swap(D, C, case["budget"][0], case["start"], trace)
    assert trace == case["moves"]
    assert list(ch) == case["final"] and tot == case["total"][0]


def _random_tables(rng, nt, nc):
    C = rng.integers(1, 40, size=(nt, nc)).astype(np.uint64)
    D = rng.random((nt, nc)) * np.exp(-C.astype(np.float64) / 15.0)
    return D, C


@pytest.mark.parametrize("seed", range(8))
def test_refine_swap_properties(seed):
    """Feasible, never worse than its start, and stopped only where no single-table move of
    lower distortion still fits the budget (checked by enumerating every move)."""
    rng = np.random.default_rng(seed)
    D, C = _random_tables(rng, 4, 7)
    for frac in (0.2, 0.5, 0.8):
        B = int(frac * int(C.sum(axis=0).max()))
        if int(C.min(axis=1).sum()) > B:
            continue
        start = O.allocate(D, C, B).choice
        ch, tot = O.refine_swap(D, C, B, start)
        assert tot == sum(int(C[t][ch[t]]) for t in range(4)) <= B
        assert sum(D[t][ch[t]] for t in range(4)) <= sum(D[t][start[t]] for t in range(4)) + 1e-15
        for t in range(4):
            for i in range(7):
                assert not (D[t][i] < D[t][ch[t]] and tot - int(C[t][ch[t]]) + int(C[t][i]) <= B)


@pytest.mark.parametrize("seed", range(6))
def test_allocate_common_brute_force(seed):
    """Every allocation vector is enumerated; among those giving all tables one candidate the
    least total distortion within budget (ties: lower cost, lower index) is the answer, and the
    unrestricted optimum of the same enumeration is never worse than it."""
    rng = np.random.default_rng(100 + seed)
    nt, nc = 3, 5
    D, C = _random_tables(rng, nt, nc)
    for frac in (0.3, 0.6, 1.0):
        B = int(frac * int(C.sum(axis=0).max()))
        best_common, best_any = None, None
        for v in itertools.product(range(nc), repeat=nt):
            cost = sum(int(C[t][v[t]]) for t in range(nt))
            if cost > B:
                continue
            dist = sum(D[t][v[t]] for t in range(nt))
            best_any = dist if best_any is None else min(best_any, dist)
            if len(set(v)) == 1:
                key = (dist, cost, v[0])
                best_common = key if best_common is None or key < best_common else best_common
        if best_common is None:
            with pytest.raises(ValueError):
                O.allocate_common(D, C, B)
            continue
        i = O.allocate_common(D, C, B)
        assert i == best_common[2]
        assert best_any <= best_common[0] + 1e-15
        mask = np.zeros(nc, bool)
        mask[i] = True
        assert O.allocate_common(D, C, B, mask) == i
