"""Fused decode-into-attention (jolt_attend) against the oracle: the oracle parses the two
records, decodes them with its own code and runs fp64 attention; the kernel rebuilds the
same bf16 caches tile by tile and attends in fp32.

Tolerance: the decoded caches agree to at most 1 bf16 ulp (the decode parity bar; on these
cases they are bit-identical), so the difference is the fp32 arithmetic of the kernel: the
scores are sums of D exact products of bf16 values, so their error is below
D * 2^-24 * sum|q||k| (under 1e-4 absolute here); a score error e moves the output by at most
2 e max|V| (softmax is 1-Lipschitz in each score, outputs are convex combinations), and the
weighted sums add 2^-24 * T relative.  |O_gpu - O_ref| <= 1e-3 max|V| covers that with room;
the measured errors are printed."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
import kvsynth as ks
from oracle import jolt_oracle as O

pytestmark = pytest.mark.gpu
O_TOL = 1e-3


def _lib():
    import partial_tucker_rotated_amd as J
    return J


def _group(wname, N=None, T=None):
    J = _lib()
    w = ks.get_workload(wname)
    N, T = N or w.N, T or w.T
    xb = [np.ascontiguousarray(ks.generate_table(w, 0, c)[:N, :T]) for c in (0, 1)]
    sg = np.stack([ks.rotation_signs(w, 0, c) for c in (0, 1)])
    xs = [torch.from_numpy(b.view(np.int16)).cuda() for b in xb]
    signs = torch.from_numpy(sg).cuda()
    cfg = J.default_config(N, T, w.D, 2, J.TOKEN_EXACT)
    ws = torch.empty(J.workspace_size(cfg), dtype=torch.uint8, device="cuda")
    J.build_tables(cfg, xs, signs, None, ws)
    return w, cfg, xs, signs, ws, N, T


@pytest.mark.parametrize("wname,N,T,pairs", [
    ("tiny", None, None, [(0, 1), (3, 42), (63, 81), (96, 99), (86, 17)]),
    ("mistral_t512", 32, 512, [(27, 63), (2, 79), (98, 94), (51, 3)]),
])
def test_attend_equals_oracle(wname, N, T, pairs):
    J = _lib()
    w, cfg, xs, signs, ws, N, T = _group(wname, N, T)
    D = w.D
    nq = 4
    qb = ks.generate_queries(w, 0, nq)[:N]
    q = torch.from_numpy(qb.view(np.int16)).cuda()
    Q = O.bf16_bits_to_f64(qb)
    scale = 1.0 / np.sqrt(D)
    aws = torch.empty(J.attend_workspace_size(cfg, 1, nq), dtype=torch.uint8, device="cuda")
    for ck, cv in pairs:
        print(f"case {wname} N={N} T={T} cand_k={ck} cand_v={cv} nq={nq}", flush=True)
        choice = np.array([ck, cv], np.int32)
        recs = [torch.zeros(J.record_bytes(cfg, int(c)), dtype=torch.uint8, device="cuda") for c in choice]
        J.encode_built(cfg, xs, signs, choice, recs, ws)
        out = torch.empty((N, nq, D), dtype=torch.float32, device="cuda")
        J.attend(cfg, [recs[0]], [ck], [recs[1]], [cv], [q], [out], aws, scale)
        xh = [torch.empty_like(x) for x in xs]
        J.decode(cfg, recs, choice, xh)
        torch.cuda.synchronize()
        dec = []
        for k in range(2):
            e = O.parse_record(recs[k].cpu().numpy().tobytes(), N, T, D)
            ref_bits = O.decode_bf16(e)
            n_idx, t_idx = np.meshgrid(np.arange(N), np.arange(T), indexing="ij")
            n_idx, t_idx = n_idx.reshape(-1), t_idx.reshape(-1)
            got = xh[k].cpu().numpy().view(np.uint16).reshape(-1, D)
            ok = O.bf16_consistent(got, O.decode_rows_f64(e, n_idx, t_idx), O.decode_eval_bound(e, n_idx, t_idx))
            assert ok.all(), int(np.sum(~ok))
            dec.append(O.bf16_bits_to_f64(ref_bits))
        ref = O.attention(dec[0], dec[1], Q, scale)
        got = out.cpu().numpy().astype(np.float64)
        vmax = float(np.abs(dec[1]).max())
        err = float(np.abs(got - ref).max())
        print(f"  max |O - O_ref| = {err:.3e} ({err / vmax:.3e} of max|V|)", flush=True)
        assert np.all(np.isfinite(got))
        assert err <= O_TOL * vmax


def test_attend_many_groups_in_one_call():
    """Nine groups (two launches of up to eight): each output equals the oracle's for its own
    queries; the records are shared, the queries differ."""
    J = _lib()
    w, cfg, xs, signs, ws, N, T = _group("tiny")
    D, nq, ng = w.D, 3, 9
    choice = np.array([42, 81], np.int32)
    recs = [torch.zeros(J.record_bytes(cfg, int(c)), dtype=torch.uint8, device="cuda") for c in choice]
    J.encode_built(cfg, xs, signs, choice, recs, ws)
    torch.cuda.synchronize()
    dec = [O.bf16_bits_to_f64(O.decode_bf16(O.parse_record(r.cpu().numpy().tobytes(), N, T, D))) for r in recs]
    rng = np.random.default_rng(5)
    qb = [ks.f32_to_bf16_bits(rng.standard_normal((N, nq, D)).astype(np.float32)) for _ in range(ng)]
    qs = [torch.from_numpy(b.view(np.int16)).cuda() for b in qb]
    outs = [torch.empty((N, nq, D), dtype=torch.float32, device="cuda") for _ in range(ng)]
    aws = torch.empty(J.attend_workspace_size(cfg, ng, nq), dtype=torch.uint8, device="cuda")
    print(f"case tiny groups={ng} nq={nq}", flush=True)
    J.attend(cfg, [recs[0]] * ng, [42] * ng, [recs[1]] * ng, [81] * ng, qs, outs, aws)
    torch.cuda.synchronize()
    vmax = float(np.abs(dec[1]).max())
    for g in range(ng):
        ref = O.attention(dec[0], dec[1], O.bf16_bits_to_f64(qb[g]), 1.0 / np.sqrt(D))
        err = float(np.abs(outs[g].cpu().numpy() - ref).max())
        assert err <= O_TOL * vmax, (g, err)


def test_attend_rejects_bad_arguments():
    J = _lib()
    w, cfg, xs, signs, ws, N, T = _group("tiny")
    aws = torch.empty(J.attend_workspace_size(cfg, 1, 4), dtype=torch.uint8, device="cuda")
    rec = torch.zeros(J.record_bytes(cfg, 0), dtype=torch.uint8, device="cuda")
    q = torch.zeros((N, 4, w.D), dtype=torch.int16, device="cuda")
    out = torch.empty((N, 4, w.D), dtype=torch.float32, device="cuda")
    for ck, cv in ((100, 0), (0, -1)):
        with pytest.raises(J.JoltError):
            J.attend(cfg, [rec], [ck], [rec], [cv], [q], [out], aws)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(J.JoltError):
        J.attend(cfg, [rec], [0], [rec], [0], [q], [out], small)
    q17 = torch.zeros((N, 17, w.D), dtype=torch.int16, device="cuda")
    with pytest.raises(J.JoltError):
        J.attend(cfg, [rec], [0], [rec], [0], [q17], [torch.empty((N, 17, w.D), dtype=torch.float32, device="cuda")],
                 aws)
