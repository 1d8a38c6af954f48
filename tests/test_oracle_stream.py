"""Pins of the oracle's streaming admission (an incoming token block encoded against a
frozen record): exact recovery of blocks that lie in the frozen Tucker model, the ST-HOSVD
identity that folds the original tokens back onto U_T, the least-squares optimality and
minimum-norm conditions, row independence, and the block record byte count."""
import numpy as np
import pytest

from oracle import jolt_oracle as O


def _f16(rng, shape, scale=1.0):
    return O.fp16_round(scale * rng.standard_normal(shape))


def _frozen(rng, N, T, D, rT, rd, b, sigma=None):
    """A frozen record with fp16-valued random factors (r_T < T or r_T = T, r_d < D or = D)."""
    sigma = sigma if sigma is not None else np.where(rng.random(D) < 0.5, -1, 1).astype(np.int8)
    Ut = _f16(rng, (T, rT), 0.2) if rT < T else None
    Ud = _f16(rng, (D, rd), 0.2) if rd < D else None
    G = _f16(rng, (N, rT, rd)) if rT < T else None
    return O.Encoded(rT, rd, b, D, sigma, Ut, Ud, G, None, None, None)


@pytest.mark.parametrize("rT,rd", [(16, 8), (8, 64), (64, 8)])
def test_block_inside_the_model_is_recovered_exactly(rT, rd):
    """X'_n = V G_n U_d^T (r_T < T) or V_n U_d^T (r_T = T) with fp16-valued V: the fold-in
    returns V bit for bit and the block's distortion vanishes."""
    rng = np.random.default_rng(rT + rd)
    N, T, D, tn = 4, 64, 64, 16
    e = _frozen(rng, N, T, D, rT, rd, 4)
    if rT < T:
        V = _f16(rng, (tn, rT), 0.3)
        Xn = O.reconstruct(V, e.Ud, e.G)
    else:
        V = _f16(rng, (N, tn, rd))
        Xn = O.reconstruct(None, e.Ud, V)
    L = O.stream_left_factor(e, Xn)
    assert np.array_equal(L, V)
    blk = O.stream_encode(e, Xn)
    assert O.block_distortion(Xn, blk) < 1e-24


def test_original_tokens_fold_back_onto_the_token_factor():
    """With the unrounded ST-HOSVD factors, G_n = U_T^T Y_n gives sum_n Y_n G_n^T = M U_T =
    U_T Lambda and sum_n G_n G_n^T = Lambda, so the fold-in of the table's own tokens is
    U_T itself (feature chain r_d < D and the unprojected chain r_d = D)."""
    rng = np.random.default_rng(3)
    N, T, D = 6, 48, 32
    X = rng.standard_normal((N, T, D)) @ np.diag(np.linspace(3.0, 0.2, D))
    _, Ud = O.feature_factor(X)
    for rT, rd in ((8, 16), (16, D)):
        Yr = X if rd == D else X @ Ud[:, :rd]
        _, UT = O.token_factor_exact(O.token_unfolding(Yr), 16)
        Ut, Udr, G = O._factors_for(X, Ud, UT, rT, rd, round_fp16=False)
        e = O.Encoded(rT, rd, 0, D, np.ones(D, np.int8), Ut, Udr, G, None, None, None)
        L = O.stream_left_factor(e, X, round_fp16=False)
        np.testing.assert_allclose(L, Ut, atol=1e-10)


@pytest.mark.parametrize("rT,rd", [(16, 8), (16, 64)])
def test_fold_in_meets_the_normal_equations(rT, rd):
    """The unrounded left factor of a generic block leaves a residual orthogonal to every
    direction of the frozen operator: sum_n (X'_n - L R_n) R_n^T = 0."""
    rng = np.random.default_rng(11)
    N, T, D, tn = 5, 64, 64, 24
    e = _frozen(rng, N, T, D, rT, rd, 2)
    Xn = rng.standard_normal((N, tn, D))
    L = O.stream_left_factor(e, Xn, round_fp16=False)
    R = e.G @ e.Ud.T if e.Ud is not None else e.G
    grad = sum((Xn[n] - L @ R[n]) @ R[n].T for n in range(N))
    scale = sum(np.abs(Xn[n]) @ np.abs(R[n]).T for n in range(N)).max()
    assert np.abs(grad).max() < 1e-12 * scale


def test_full_token_chain_is_a_per_slice_fit():
    """r_T = T: every slice's rows are its own least-squares fit against U_d alone, and with
    an orthonormal U_d the fit is the projection X'_n U_d."""
    rng = np.random.default_rng(5)
    N, T, D, tn, rd = 3, 64, 32, 8, 8
    Q, _ = np.linalg.qr(rng.standard_normal((D, rd)))
    e = O.Encoded(T, rd, 0, D, np.ones(D, np.int8), None, Q, None, None, None, None)
    Xn = rng.standard_normal((N, tn, D))
    L = O.stream_left_factor(e, Xn, round_fp16=False)
    np.testing.assert_allclose(L, Xn @ Q, atol=1e-12)


def test_rank_deficient_operator_gives_the_minimum_norm_rows():
    """N r_d < r_T: many rows fit equally well.  The returned rows satisfy the normal
    equations and lie in the row space of the stacked operator (no component along its
    null space), which characterises the minimum-norm solution."""
    rng = np.random.default_rng(8)
    N, T, D, tn, rT, rd = 1, 64, 32, 6, 16, 4
    e = _frozen(rng, N, T, D, rT, rd, 0)
    Xn = rng.standard_normal((N, tn, D))
    L = O.stream_left_factor(e, Xn, round_fp16=False)
    R = e.G[0] @ e.Ud.T                    # [rT, D], rank 4
    _, sv, Vt = np.linalg.svd(R.T, full_matrices=True)
    null = Vt[np.sum(sv > 1e-9 * sv[0]):]  # null space of R^T in R^rT
    assert null.shape[0] == rT - rd
    assert np.abs(L @ null.T).max() < 1e-10
    assert np.abs((Xn[0] - L @ R) @ R.T).max() < 1e-10 * np.abs(R).sum()


def test_zero_cores_leave_the_whole_block_to_the_residual():
    rng = np.random.default_rng(2)
    N, T, D, tn = 2, 64, 32, 8
    e = _frozen(rng, N, T, D, 8, 8, 8)
    e.G[:] = 0.0
    Xn = rng.standard_normal((N, tn, D))
    blk = O.stream_encode(e, Xn)
    assert np.all(blk.Ut == 0.0)
    Y = O.rotate_rows(Xn, e.sigma)
    q, s, Yh = O.quantize_blocks(Y, 8, D)
    assert np.array_equal(blk.codes, q) and np.array_equal(blk.scales, s)
    np.testing.assert_allclose(O.decode_f64(blk), O.unrotate_rows(Yh, e.sigma), atol=1e-15)


def test_rows_are_encoded_independently():
    """No step couples tokens: the block encoded whole equals its two halves encoded apart."""
    rng = np.random.default_rng(9)
    N, T, D, tn = 3, 64, 32, 16
    for rT in (8, T):
        e = _frozen(rng, N, T, D, rT, 8, 4)
        Xn = rng.standard_normal((N, tn, D))
        whole = O.stream_encode(e, Xn)
        a, b = O.stream_encode(e, Xn[:, :7]), O.stream_encode(e, Xn[:, 7:])
        if rT < T:
            assert np.array_equal(whole.Ut, np.concatenate([a.Ut, b.Ut]))
        else:
            assert np.array_equal(whole.G, np.concatenate([a.G, b.G], axis=1))
        assert np.array_equal(whole.codes, np.concatenate([a.codes, b.codes], axis=1))


def test_verbatim_block_and_block_bytes():
    rng = np.random.default_rng(4)
    N, T, D, tn = 2, 64, 32, 8
    e = O.Encoded(T, D, 0, D, np.ones(D, np.int8), None, None, None, np.zeros((N, T, D)), None, None)
    Xn = rng.standard_normal((N, tn, D))
    blk = O.stream_encode(e, Xn)
    assert np.array_equal(O.decode_f64(blk), Xn) and O.block_distortion(Xn, blk) == 0.0
    # hand-counted: N = 32, t' = 64, D = 128, r_T = 16, r_d = 8, b = 4, blocks of 128:
    # header 256 + left factor 2*64*16 = 2048 + codes 4*32*64*128/8 = 131072 + scales 4*32*64 = 8192
    assert O.block_bytes(32, 64, 128, 512, 16, 8, 4, 128) == 256 + 2048 + 131072 + 8192
    # r_T = T: per-slice rows 2*32*64*8 = 32768; b = 0 stores no codes
    assert O.block_bytes(32, 64, 128, 512, 512, 8, 0, 128) == 256 + 32768
    # (T, D): verbatim 2*32*64*128 = 524288; a 100-byte section pads to 256
    assert O.block_bytes(32, 64, 128, 512, 512, 128, 2, 128) == 256 + 524288
    assert O.block_bytes(1, 10, 64, 64, 4, 4, 0, 64) == 256 + 256


def _write_block(frozen, N, tn, D, T, L, codes, scales, xv=None):
    """Minimal writer of the documented block record layout (header words 0-9, then the
    64-bit total and the offsets of L, codes and scales at byte 40; 256-aligned sections),
    used to pin the parser."""
    import struct
    pad = O.pad
    b, blk = frozen.b, frozen.blk
    off = 256
    secs = {}
    if xv is not None:
        raw = xv
    else:
        raw = np.asarray(L).astype(np.float16).tobytes()
    secs["l"] = (off, raw)
    off += pad(len(raw))
    if xv is None and b:
        u = (codes.reshape(-1) & ((1 << b) - 1)).astype(np.uint64)
        bitsarr = ((u[:, None] >> np.arange(b, dtype=np.uint64)[None, :]) & np.uint64(1)).astype(np.uint8)
        craw = np.packbits(bitsarr.reshape(-1), bitorder="little").tobytes()
        secs["codes"] = (off, craw)
        off += pad(len(craw))
        sraw = scales.astype(np.float32).tobytes()
        secs["scales"] = (off, sraw)
        off += pad(len(sraw))
    buf = bytearray(off)
    struct.pack_into("<IIiiiiiiii", buf, 0, O.BLOCK_MAGIC, 1, N, tn, D, frozen.rT, frozen.rd, b, blk, T)
    struct.pack_into("<QQQQ", buf, 40, off, *(secs.get(k, (0, b""))[0] for k in ("l", "codes", "scales")))
    for o, r in secs.values():
        buf[o:o + len(r)] = r
    return bytes(buf)


@pytest.mark.parametrize("rT,rd,b", [(16, 8, 2), (16, 64, 4), (64, 8, 8), (8, 16, 0)])
def test_block_parser_roundtrip_and_size(rT, rd, b):
    """Every field written in the documented layout comes back from parse_block: the left
    factor (shared rows for r_T < T, per-slice rows for r_T = T), the packed two's-complement
    codes including the most negative ones, the scales; the byte count equals block_bytes."""
    rng = np.random.default_rng(rT * 100 + rd + b)
    N, T, D, tn = 3, 64, 64, 128
    e = _frozen(rng, N, T, D, rT, rd, b)
    L = _f16(rng, (tn, rT)) if rT < T else _f16(rng, (N, tn, rd))
    codes = scales = None
    if b:
        codes = rng.integers(-(1 << (b - 1)), 1 << (b - 1), size=(N, tn, D))
        codes[0, 0, :4] = [-(1 << (b - 1)), (1 << (b - 1)) - 1, 0, -1]
        scales = O.f32_round(rng.random((N, tn, 1)))
    buf = _write_block(e, N, tn, D, T, L, codes, scales)
    assert len(buf) == O.block_bytes(N, tn, D, T, rT, rd, b, D)
    got = O.parse_block(buf, e, N, tn, D)
    if rT < T:
        assert np.array_equal(got.Ut, L) and np.array_equal(got.G, e.G)
    else:
        assert got.Ut is None and np.array_equal(got.G, L)
    assert (got.Ud is None) == (rd == D) and (got.Ud is None or np.array_equal(got.Ud, e.Ud))
    assert np.array_equal(got.sigma, e.sigma) and (got.rT, got.rd, got.b) == (rT, rd, b)
    if b:
        assert np.array_equal(got.codes, codes) and np.array_equal(got.scales, scales)
    else:
        assert got.codes is None and got.scales is None
    # a header for another shape is refused
    with pytest.raises(ValueError):
        O.parse_block(buf, e, N, tn + 64, D)


def test_block_parser_verbatim_and_hand_packed_codes():
    """A verbatim (T, D) block returns its bf16 values; and a 2-bit block whose code bytes
    are written by hand (0b11100100 = codes 0, 1, -2, -1 from the low bits up) decodes to
    exactly those codes."""
    rng = np.random.default_rng(7)
    N, T, D, tn = 2, 64, 64, 64
    xv = O.f64_to_bf16_bits(rng.standard_normal((N, tn, D)))
    ev = O.Encoded(T, D, 4, D, np.ones(D, np.int8), None, None, None, np.zeros((N, T, D)), None, None)
    buf = _write_block(ev, N, tn, D, T, None, None, None, xv=xv.tobytes())
    assert len(buf) == O.block_bytes(N, tn, D, T, T, D, 4, D)
    got = O.parse_block(buf, ev, N, tn, D)
    assert np.array_equal(got.Xv, O.bf16_bits_to_f64(xv))
    e = _frozen(rng, N, T, D, 8, 8, 2)
    L = _f16(rng, (tn, 8))
    codes = np.zeros((N, tn, D), np.int64)
    scales = O.f32_round(np.ones((N, tn, 1)))
    buf = bytearray(_write_block(e, N, tn, D, T, L, codes, scales))
    import struct
    off_codes = struct.unpack_from("<Q", buf, 56)[0]
    buf[off_codes] = 0b11100100
    got = O.parse_block(bytes(buf), e, N, tn, D)
    assert list(got.codes.reshape(-1)[:5]) == [0, 1, -2, -1, 0]
