"""GPU parity of streaming admission (jolt_stream_prepare / _encode / _decode) against the
oracle's stream_left_factor / stream_encode / block_distortion.

Frozen records come from jolt_encode on the first T tokens of a seeded table; the incoming
block is the next t' tokens of the same table (the same AR(1) process continued), so the
block is distributed like the cache it joins.

Bars:
  * left-factor rows (fp16): equal to the oracle's own fit, except for storage roundings
    flipped by fp64 summation order: at most 1e-3 of the values, each by one fp16 ulp;
  * conditional code parity (the oracle quantizes with the GPU's stored rows): at most 1e-4
    of the codes differ, each by at most 1; scales within 1e-6 relative;
  * decoded block within one bf16 ulp of the oracle's decode of the GPU's block record,
    except values within the decoder's fp32 evaluation bound (oracle.decode_eval_bound, plus
    1e-14 of the block's largest magnitude for the rounding residue the oracle's fp64
    unrotation leaves on exact zeros), which may round from anywhere inside it;
  * block distortion within 1e-6 relative of the oracle's on the GPU's block (the same rows
    and codes), and within 1e-3 relative (plus 1e-12 absolute) of the oracle's own encode.
"""
import dataclasses

import numpy as np
import pytest

import kvsynth as ks
from oracle import jolt_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _cand(T, D, rT, rd, b):
    rts, rds, bs = (4, 8, 16, 32, T), (4, 8, 16, 32, D), (0, 2, 4, 8)
    return (rts.index(rT) * 5 + rds.index(rd)) * 4 + bs.index(b)


def _f16_ulp_dist(a, b):
    ia = a.astype(np.float16).view(np.int16).astype(np.int64)
    ib = b.astype(np.float16).view(np.int16).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFF), ib)
    return np.abs(ia - ib)


def _run(w, tabs, T, tn, N=None, xmod=None):
    """tabs: list of ((g, c), (r_T, r_d, b)).  Frozen on tokens [0, T), block [T, T + tn)
    of the tables of workload w (which must hold at least T + tn tokens)."""
    import partial_tucker_rotated_amd as J
    N = N or w.N
    D = w.D
    assert w.T >= T + tn
    print(f"stream {w.name} N={N} T={T} t'={tn} tables={tabs}", flush=True)
    full = [ks.generate_table(w, g, c)[:N, : T + tn] for (g, c), _ in tabs]
    if xmod is not None:
        full = [xmod(k, b) for k, b in enumerate(full)]
    xb = [np.ascontiguousarray(b[:, :T]) for b in full]
    nb = [np.ascontiguousarray(b[:, T: T + tn]) for b in full]
    sg = np.stack([ks.rotation_signs(w, g, c) for (g, c), _ in tabs])
    ch = np.array([_cand(T, D, *z) for _, z in tabs], np.int32)
    cfg = J.default_config(N, T, D, len(tabs), J.TOKEN_EXACT)
    ws = torch.empty(J.workspace_size(cfg), dtype=torch.uint8, device="cuda")
    xs = [torch.from_numpy(b.view(np.int16)).cuda() for b in xb]
    recs = [torch.zeros(J.record_bytes(cfg, int(c)), dtype=torch.uint8, device="cuda") for c in ch]
    J.encode(cfg, xs, torch.from_numpy(sg).cuda(), None, ch, recs, ws)
    states = [torch.empty(J.stream_state_bytes(), dtype=torch.uint8, device="cuda") for _ in tabs]
    J.stream_prepare(cfg, recs, ch, states)
    xn = [torch.from_numpy(b.view(np.int16)).cuda() for b in nb]
    blocks = [torch.full((J.stream_block_bytes(cfg, int(c), tn),), 0xAB, dtype=torch.uint8, device="cuda") for c in ch]
    sws = torch.empty(J.stream_workspace_size(cfg, tn), dtype=torch.uint8, device="cuda")
    dist = torch.full((len(tabs),), -1.0, dtype=torch.float64, device="cuda")
    J.stream_encode(cfg, recs, ch, states, xn, tn, blocks, sws, dist=dist)
    outs = [torch.empty_like(x) for x in xn]
    J.stream_decode(cfg, recs, ch, blocks, tn, outs)
    torch.cuda.synchronize()
    dist = dist.cpu().numpy()
    results = []
    for k, (_, (rT, rd, b)) in enumerate(tabs):
        frozen = O.parse_record(recs[k].cpu().numpy().tobytes(), N, T, D)
        Xn = O.bf16_bits_to_f64(nb[k])
        raw = blocks[k].cpu().numpy().tobytes()
        assert len(raw) == O.block_bytes(N, tn, D, T, rT, rd, b, D)
        gb = O.parse_block(raw, frozen, N, tn, D)
        assert np.frombuffer(raw, np.uint32)[18] == 0, "fp16 overflow flag"
        own = O.stream_encode(frozen, Xn)
        where = f"table {k} z=({rT},{rd},{b})"
        if frozen.Xv is None:
            Lg = gb.Ut if gb.Ut is not None else gb.G
            Lo = own.Ut if own.Ut is not None else own.G
            du = _f16_ulp_dist(Lg, Lo)
            frac = float(np.mean(du > 0))
            print(f"  {where}: left factor {Lg.shape}, differing fp16 values {frac:.2e}", flush=True)
            assert du.max() <= 1 and frac <= 1e-3, (where, du.max(), frac)
            if b > 0:
                cond = O.stream_encode(frozen, Xn, L=Lg)
                dq = np.abs(cond.codes.astype(np.int64) - gb.codes)
                cf = float(np.mean(dq > 0))
                assert dq.max() <= 1 and cf <= 1e-4, (where, dq.max(), cf)
                srel = np.abs(cond.scales - gb.scales) / np.maximum(np.abs(cond.scales), 1e-30)
                assert srel.max() < 1e-6, (where, srel.max())
        got = outs[k].cpu().numpy().view(np.uint16).reshape(-1, D)
        n_idx, t_idx = np.meshgrid(np.arange(N), np.arange(tn), indexing="ij")
        n_idx, t_idx = n_idx.reshape(-1), t_idx.reshape(-1)
        xhat = O.decode_rows_f64(gb, n_idx, t_idx)
        # within one bf16 ulp of the exact value's rounding, or within the decoder's fp32
        # evaluation bound (values near zero, and the oracle's rounding residue of exact zeros)
        ok = O.bf16_consistent(got, xhat, O.decode_eval_bound(gb, n_idx, t_idx) + 1e-14 * float(np.abs(Xn).max()))
        assert ok.all(), (where, int(np.sum(~ok)))
        d_same = O.block_distortion(Xn, gb)
        d_own = O.block_distortion(Xn, own)
        print(f"  {where}: block distortion gpu {dist[k]:.6e} oracle {d_own:.6e}", flush=True)
        assert abs(dist[k] - d_same) <= 1e-6 * d_same + 1e-300, (where, dist[k], d_same)
        assert abs(dist[k] - d_own) <= 1e-3 * d_own + 1e-12, (where, dist[k], d_own)
        results.append(dist[k])
    return results


def test_stream_every_record_kind():
    """Every chain kind and bit width: r_d chains (r_T < r_d, r_T > r_d), the unprojected
    chain r_d = D, the full-token chain r_T = T, and a verbatim record; a ragged last
    chunk of 64 tokens (t' = 320)."""
    w = ks.get_workload("mistral_t512")
    tabs = [((0, 0), (16, 8, 4)), ((0, 1), (32, 32, 2)), ((1, 0), (8, 128, 8)), ((1, 1), (256, 16, 4)),
            ((2, 0), (256, 128, 0)), ((2, 1), (4, 4, 0)), ((3, 0), (32, 4, 8)), ((3, 1), (256, 4, 2))]
    d = _run(w, tabs, T=256, tn=256, N=8)
    assert d[4] == 0.0
    tabs2 = [(gc, (128 if z[0] == 256 else z[0], z[1], z[2])) for gc, z in tabs[:4]]
    _run(w, tabs2, T=128, tn=320, N=8)


def test_stream_rank_deficient_operator_and_small_block():
    """N r_d < r_T (4 slices, r_d = 4, r_T = 32): the minimum-norm rows; t' = 64."""
    w = dataclasses.replace(ks.get_workload("tiny"), T=128)  # D = 64
    _run(w, [((0, 0), (32, 4, 4))], T=64, tn=64, N=4)
    _run(w, [((0, 0), (16, 8, 2)), ((0, 0), (64, 4, 8))], T=64, tn=64, N=4)


def test_stream_zero_cases():
    """An all-zero block (distortion 0, zero rows) and an all-zero frozen table (A = 0: zero
    rows, the whole block goes to the residual)."""
    def zero_block(k, b):
        b = b.copy()
        b[:, 128:] = 0
        return b

    w = ks.get_workload("mistral_t512")
    d = _run(w, [((0, 0), (16, 8, 4)), ((0, 1), (128, 8, 2))], T=128, tn=64, N=8, xmod=zero_block)
    assert d == [0.0, 0.0]

    def zero_frozen(k, b):
        b = b.copy()
        b[:, :128] = 0
        return b

    _run(w, [((1, 0), (16, 8, 8)), ((1, 1), (32, 128, 4)), ((2, 0), (128, 16, 4))], T=128, tn=64, N=8,
         xmod=zero_frozen)


def test_stream_full_size_block():
    """All 16 tables of the Mistral-shaped cache (32 slices, D = 128), frozen on 256 tokens
    at typical candidates, a 256-token block each."""
    w = ks.get_workload("mistral_t512")
    zs = [(16, 32, 4), (32, 32, 4), (32, 16, 2), (8, 128, 4)]
    tabs = [(gc, zs[k % 4]) for k, gc in enumerate(w.table_ids())]
    _run(w, tabs, T=256, tn=256)


def test_stream_rejects_bad_arguments():
    import partial_tucker_rotated_amd as J
    cfg = J.default_config(4, 64, 64, 1, J.TOKEN_EXACT)
    with pytest.raises(J.JoltError):
        J.stream_block_bytes(cfg, 5, 100)
    with pytest.raises(J.JoltError):
        J.stream_workspace_size(cfg, 0)
    rec = torch.zeros(J.record_bytes(cfg, 5), dtype=torch.uint8, device="cuda")
    st = torch.zeros(J.stream_state_bytes(), dtype=torch.uint8, device="cuda")
    x = torch.zeros((4, 64, 64), dtype=torch.int16, device="cuda")
    blk = torch.zeros(J.stream_block_bytes(cfg, 5, 64), dtype=torch.uint8, device="cuda")
    short = torch.zeros(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(J.JoltError) as e:
        J.stream_encode(cfg, [rec], [5], [st], [x], 64, [blk], short)
    assert e.value.name == "JOLT_ENOMEM"
    with pytest.raises(J.JoltError):
        J.stream_encode(cfg, [rec], [100], [st], [x], 64, [blk], short)
