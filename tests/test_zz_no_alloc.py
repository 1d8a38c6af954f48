"""jolt_stream_encode_noalloc (the streaming encode for callers that cannot allocate device
memory) against jolt_stream_encode with a caller workspace, through the C ABI: the block
records and distortions of two calls in a row, the second with a smaller input (fewer
tokens and fewer tables), are identical to the byte; a request beyond the scratch limit is
refused before any device work."""
import numpy as np
import pytest

import kvsynth as ks

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _cand(T, D, rT, rd, b):
    rts, rds, bs = (4, 8, 16, 32, T), (4, 8, 16, 32, D), (0, 2, 4, 8)
    return (rts.index(rT) * 5 + rds.index(rd)) * 4 + bs.index(b)


def _setup(ntab, T, tn):
    import partial_tucker_rotated_amd as J
    w = ks.get_workload("mistral_t512")
    zs = [(16, 32, 4), (32, 128, 8), (512, 16, 2), (8, 32, 0), (512, 128, 4), (32, 8, 8)]
    ids = w.table_ids()[:ntab]
    full = [ks.generate_table(w, g, c)[:, : T + tn] for g, c in ids]
    sg = torch.from_numpy(np.stack([ks.rotation_signs(w, g, c) for g, c in ids])).cuda()
    ch = np.array([_cand(T, w.D, *zs[k % len(zs)]) if zs[k % len(zs)][0] != 512 else
                   _cand(T, w.D, T, *zs[k % len(zs)][1:]) for k in range(ntab)], np.int32)
    cfg = J.default_config(w.N, T, w.D, ntab, J.TOKEN_EXACT)
    ws = torch.empty(J.workspace_size(cfg), dtype=torch.uint8, device="cuda")
    xs = [torch.from_numpy(np.ascontiguousarray(b[:, :T]).view(np.int16)).cuda() for b in full]
    recs = [torch.zeros(J.record_bytes(cfg, int(c)), dtype=torch.uint8, device="cuda") for c in ch]
    J.encode(cfg, xs, sg, None, ch, recs, ws)
    states = [torch.empty(J.stream_state_bytes(), dtype=torch.uint8, device="cuda") for _ in ids]
    J.stream_prepare(cfg, recs, ch, states)
    xn = [torch.from_numpy(np.ascontiguousarray(b[:, T: T + tn]).view(np.int16)).cuda() for b in full]
    return J, cfg, ch, recs, states, xn


def _both(J, cfg, ch, recs, states, xn, tn):
    blocks_a = [torch.full((J.stream_block_bytes(cfg, int(c), tn),), 0x5A, dtype=torch.uint8, device="cuda")
                for c in ch]
    blocks_b = [torch.full_like(b, 0xC3) for b in blocks_a]
    dist_a = torch.full((len(ch),), -1.0, dtype=torch.float64, device="cuda")
    dist_b = torch.full_like(dist_a, -2.0)
    sws = torch.empty(J.stream_workspace_size(cfg, tn), dtype=torch.uint8, device="cuda")
    J.stream_encode(cfg, recs, ch, states, xn, tn, blocks_a, sws, dist=dist_a)
    J.stream_encode_noalloc(cfg, recs, ch, states, xn, tn, blocks_b, dist=dist_b)
    torch.cuda.synchronize()
    for k in range(len(ch)):
        assert torch.equal(blocks_a[k], blocks_b[k]), k
    assert torch.equal(dist_a, dist_b)
    assert bool((dist_a >= 0).all())
    return dist_a.cpu().numpy()


def test_noalloc_stream_encode_equals_workspace_version():
    print("case noalloc: 6 tables t'=256, then 3 tables t'=128", flush=True)
    J, cfg, ch, recs, states, xn = _setup(6, 256, 256)
    d1 = _both(J, cfg, ch, recs, states, xn, 256)
    print(f"  first call: dist {d1}", flush=True)
    J, cfg, ch, recs, states, xn = _setup(3, 256, 128)
    d2 = _both(J, cfg, ch, recs, states, xn, 128)
    print(f"  second call: dist {d2}", flush=True)


def test_noalloc_stream_encode_refuses_beyond_its_scratch():
    import partial_tucker_rotated_amd as J
    cfg = J.default_config(32, 512, 128, 16, J.TOKEN_EXACT)
    tn = 4096
    assert J.stream_workspace_size(cfg, tn) > J.NOALLOC_SCRATCH_BYTES
    ch = np.zeros(16, np.int32)
    rec = torch.zeros(J.record_bytes(cfg, 0), dtype=torch.uint8, device="cuda")
    st = torch.zeros(J.stream_state_bytes(), dtype=torch.uint8, device="cuda")
    x = torch.zeros((32, tn, 128), dtype=torch.int16, device="cuda")
    blk = torch.zeros(J.stream_block_bytes(cfg, 0, tn), dtype=torch.uint8, device="cuda")
    with pytest.raises(J.JoltError) as e:
        J.stream_encode_noalloc(cfg, [rec] * 16, ch, [st] * 16, [x] * 16, tn, [blk] * 16)
    assert e.value.name == "JOLT_ENOMEM"
