"""Oracle for the JoLT candidate-table engine: a plain, slow, fp64 CPU implementation.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
this module; only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP library: the two meet only at the seeded
inputs (``kvsynth``) and at the documented record byte layout, which this module
parses with its own code.

Sources (the web pages about arXiv:2607.12550, "A JoLT for the KV cache"), cited by
page title and section:

* [JTRA] "Joint Tucker-rank and residual-bit KV allocator" -- Formulas (four
  displays: residual/decoded cache; normalised distortion; Lagrangian; byte cost),
  Mathematical statement, Implementation notes.
* [RTR]  "Rotated Tucker residual for outlier-resistant KV quantization" --
  Mathematical statement, Key formulas (rotation, block quantizer Q_b, decode,
  MSE_KV), Implementation notes (normalized Hadamard, blocks of 64/128 values).
* [TS]   "Technical Summary: A JOLT for the KV Cache" -- Methodology 1 (partial
  Tucker via ST-HOSVD), 2 (rotated residual, b in {0,2,4,8}), 3 (joint Lagrangian
  allocation), 4 (FlashJoLT randomized token-mode SVD).
* [ABS]  arXiv abstract as reproduced on the aiqbench news page (partial Tucker
  over token and feature axes only; random orthogonal rotation; one Lagrangian
  dual over one byte budget).

Readings taken where the pages are silent (each one is listed with its reason in
the design notes of the repository):

* ST-HOSVD order: feature mode first (on X), then token mode on the projected
  tensor Y(r_d) = X x_d U_d[:, :r_d]^T; one token problem per r_d.
* r_T = T / r_d = D mean the identity factor (nothing stored); (T, D) stores X.
* Factors and core are stored as fp16 (RNE); the candidate distortion is the
  distortion of the stored representation.  Scales are stored as fp32.
* Rotation Q = H_D diag(sigma) / sqrt(D) with the Sylvester Hadamard matrix
  H[i, j] = (-1)^popcount(i & j), applied to every length-D row.
* A quantization block is one rotated row of D values; ``round`` is
  round-half-to-even.
* Byte cost: exact record bytes with 256-byte header and 256-byte alignment.
* Allocation: lambda+ = inf{lambda : sum C(z*(lambda)) <= B}; ties in D + lambda*C
  go to the lower cost, then the lower candidate index.
* Streaming admission: an incoming token block keeps the frozen feature factor and
  cores; its token rows are the minimum-norm least-squares fit against the frozen
  reconstruction operator (singular values below 1e-6 of the largest dropped).

Parity pins for every function live in ``tests/test_oracle_*.py``.  No function
here is "parity unpinned".
"""
from __future__ import annotations

import math
import struct
from dataclasses import dataclass, field
from fractions import Fraction
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

KMAX = 32  # largest truncated rank on the grid {4, 8, 16, 32, full}


# ============================================================== number formats
def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (a bf16 is the top half of an fp32)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 directly to bf16: nearest, ties to even, on the bit pattern.

    Only the bf16 normal range (and zero) is supported; anything else raises."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    b64 = x.view(np.uint64)
    sign = (b64 >> np.uint64(63)).astype(np.uint64)
    e11 = ((b64 >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    e8 = e11 - 1023 + 127
    zero = (b64 & np.uint64(0x7FFFFFFFFFFFFFFF)) == 0
    if np.any(~zero & ((e8 < 1) | (e8 > 254))):
        raise OverflowError("value outside the bf16 normal range")
    e8 = np.where(zero, 0, e8).astype(np.uint64)
    mant7 = (b64 >> np.uint64(45)) & np.uint64(0x7F)
    rem = b64 & np.uint64((1 << 45) - 1)
    half = np.uint64(1 << 44)
    mag = (e8 << np.uint64(7)) | mant7
    up = (rem > half) | ((rem == half) & ((mag & np.uint64(1)) == 1))
    mag = mag + up.astype(np.uint64)
    mag = np.where(zero, np.uint64(0), mag)
    return ((sign << np.uint64(15)) | mag).astype(np.uint16)


def fp16_round(x: np.ndarray) -> np.ndarray:
    """Storage rounding of factors and core: fp64 -> fp16 (RNE) -> fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def f32_round(x):
    return np.float64(np.float32(x)) if np.isscalar(x) else np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


# ============================================================== rotation [RTR]
def hadamard(D: int) -> np.ndarray:
    """Sylvester Hadamard matrix: H[i, j] = (-1)^popcount(i & j) (unnormalised)."""
    if D <= 0 or D & (D - 1):
        raise ValueError("Hadamard rotation needs a power-of-two width")
    i = np.arange(D)
    parity = np.zeros((D, D), dtype=np.int64)
    a = i[:, None] & i[None, :]
    while a.any():
        parity ^= a & 1
        a = a >> 1
    return np.where(parity == 1, -1.0, 1.0)


def rotation_matrix(sigma: np.ndarray) -> np.ndarray:
    """Dense Q = H diag(sigma) / sqrt(D) ([RTR] Implementation notes: normalized
    Hadamard for power-of-two widths; random signs make it a random rotation)."""
    D = sigma.shape[0]
    return hadamard(D) * np.asarray(sigma, np.float64)[None, :] / math.sqrt(D)


def rotate_rows(R: np.ndarray, sigma: np.ndarray) -> np.ndarray:
    """Y = Q r for every length-D row r of R ([RTR] Key formulas, Y = QR)."""
    Q = rotation_matrix(sigma)
    return R @ Q.T


def unrotate_rows(Y: np.ndarray, sigma: np.ndarray) -> np.ndarray:
    """r = Q^T y for every row ([JTRA] Formulas, first display: Q^T Q = I)."""
    Q = rotation_matrix(sigma)
    return Y @ Q


# ============================================================== quantizer [RTR]
def quant_scale(Yb: np.ndarray, b: int) -> np.ndarray:
    """Block scale s = max|Y| / (2^(b-1) - 1), stored (and therefore used) as fp32.

    ``Yb`` has the block on its last axis."""
    qmax = (1 << (b - 1)) - 1
    m = np.max(np.abs(Yb), axis=-1)
    return f32_round(m / qmax)


def quant_codes(Yb: np.ndarray, s: np.ndarray, b: int) -> np.ndarray:
    """q = clip(round(Y/s), -2^(b-1), 2^(b-1)-1), round half to even; s = 0 gives q = 0."""
    lo, hi = -(1 << (b - 1)), (1 << (b - 1)) - 1
    s_ = s[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(s_ > 0, Yb / np.where(s_ > 0, s_, 1.0), 0.0)
    return np.clip(np.rint(u), lo, hi).astype(np.int64)


def quantize_blocks(Y: np.ndarray, b: int, blk: int):
    """Q_b applied blockwise along the last axis (blocks of ``blk`` consecutive values).

    Returns (codes [..., D] int64, scales [..., D/blk] fp64-of-fp32, Yhat [..., D])."""
    D = Y.shape[-1]
    if D % blk:
        raise ValueError("block size must divide the row width")
    Yb = Y.reshape(Y.shape[:-1] + (D // blk, blk))
    if b == 0:
        z = np.zeros_like(Y)
        return None, None, z
    s = quant_scale(Yb, b)
    q = quant_codes(Yb, s, b)
    Yhat = (q * s[..., None]).reshape(Y.shape)
    return q.reshape(Y.shape), s, Yhat


# ============================================================== eigen helpers
def sign_normalise(U: np.ndarray) -> np.ndarray:
    """Make the largest-magnitude entry of every column positive (first index on ties)."""
    U = U.copy()
    idx = np.argmax(np.abs(U), axis=0)
    sgn = np.sign(U[idx, np.arange(U.shape[1])])
    sgn[sgn == 0] = 1.0
    return U * sgn[None, :]


def eigh_desc(M: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Eigenpairs of a symmetric matrix, eigenvalues descending, sign-normalised vectors."""
    w, V = np.linalg.eigh(M)
    order = np.argsort(-w, kind="stable")
    return w[order], sign_normalise(V[:, order])


# ============================================================== partial Tucker [TS 1]
def feature_factor(X: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Mode-d factor of ST-HOSVD: eigenvectors of the feature Gram sum_n X_n^T X_n
    (equivalently right singular vectors of the feature unfolding)."""
    N, T, D = X.shape
    Xf = X.reshape(N * T, D)
    G = Xf.T @ Xf
    return eigh_desc(G)


def token_unfolding(Yr: np.ndarray) -> np.ndarray:
    """A[t, n*r + j] = Yr[n, t, j]: the token unfolding with slices side by side."""
    N, T, r = Yr.shape
    return Yr.transpose(1, 0, 2).reshape(T, N * r)


def token_factor_exact(A: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k eigenpairs of the token Gram A A^T (sequential SVD on the token unfolding)."""
    lam, U = eigh_desc(A @ A.T)
    return lam, U[:, :k]


def orth(M: np.ndarray) -> np.ndarray:
    """Orthonormal basis of the column space (Householder QR)."""
    Q, _ = np.linalg.qr(M, mode="reduced")
    return Q


def token_factor_randomized(A: np.ndarray, omega: np.ndarray, power_iters: int, k: int) -> np.ndarray:
    """FlashJoLT token factor ([TS] Methodology 4): randomized range finder with the given
    Gaussian test matrix, ``power_iters`` rounds of subspace iteration (re-orthonormalised
    after every product with A^T and with A), then the small SVD of B = Q^T A."""
    Q = orth(A @ omega)
    for _ in range(power_iters):
        Qt = orth(A.T @ Q)
        Q = orth(A @ Qt)
    B = Q.T @ A
    UB, _, _ = np.linalg.svd(B, full_matrices=False)
    return sign_normalise(Q @ UB[:, :k])


def token_spectrum_randomized(A: np.ndarray, omega: np.ndarray, power_iters: int, k: int) -> np.ndarray:
    """The top-k squared singular values of FlashJoLT's B = Q^T A (the same range finder as
    token_factor_randomized): the energies its token factor captures, descending."""
    Q = orth(A @ omega)
    for _ in range(power_iters):
        Qt = orth(A.T @ Q)
        Q = orth(A @ Qt)
    sv = np.linalg.svd(Q.T @ A, compute_uv=False)
    return (sv * sv)[:k]


# ============================================================== byte cost [JTRA]
HDR_BYTES = 256
ALIGN = 256


def pad(x: int, a: int = ALIGN) -> int:
    return -(-int(x) // a) * a


def candidate_cost(N: int, T: int, D: int, rT: int, rd: int, b: int, blk: int,
                   s: int = 2, align: int = ALIGN, hdr: int = HDR_BYTES) -> int:
    """Storage-exact bytes of one compressed record ([JTRA] Formulas, cost display, and
    Implementation notes: count factors, core, codes, scales, transform metadata and
    alignment padding).  Factors are shared by the N slices of the group."""
    p = lambda x: -(-int(x) // align) * align
    if rT == T and rd == D:
        tucker = p(s * N * T * D)
    else:
        tucker = (p(s * T * rT) if rT < T else 0) + (p(s * D * rd) if rd < D else 0) + p(s * N * rT * rd)
    resid = 0
    if b > 0:
        resid = p(-(-(b * N * T * D) // 8)) + p(4 * N * T * (D // blk))
    return hdr + tucker + resid


def candidate_list(T: int, D: int, rT: Sequence[int], rd: Sequence[int], bits: Sequence[int]):
    """Candidate index i = (i_rT * len(rd) + i_rd) * len(bits) + i_b."""
    return [(a, c, b) for a in rT for c in rd for b in bits]


def cost_table(N, T, D, rT, rd, bits, blk, s=2, align=ALIGN, hdr=HDR_BYTES) -> np.ndarray:
    return np.array([candidate_cost(N, T, D, a, c, b, blk, s, align, hdr)
                     for (a, c, b) in candidate_list(T, D, rT, rd, bits)], dtype=np.uint64)


# ============================================================== per-table build
@dataclass
class TableResult:
    D: np.ndarray            # [n_cand] normalised distortion of the stored representation
    C: np.ndarray            # [n_cand] bytes
    xnorm2: float
    energy_gap: np.ndarray   # [n_cand] ||R||^2 - ||QR||^2 (should be ~0)
    lam_d: np.ndarray = None
    Ud: np.ndarray = None
    UT: Dict[int, np.ndarray] = field(default_factory=dict)


def _factors_for(X, Ud, UT_r, rT, rd, round_fp16=True):
    """Stored factors for one (r_T, r_d): (Ut~ or None, Ud~ or None, G~)."""
    N, T, D = X.shape
    rnd = fp16_round if round_fp16 else (lambda a: np.asarray(a, np.float64))
    Yr = X if rd == D else X @ Ud[:, :rd]
    if rT == T:
        G = Yr
        Ut = None
    else:
        U = UT_r[:, :rT]
        G = np.einsum("tk,ntj->nkj", U, Yr)
        Ut = rnd(U)
    if round_fp16 and np.max(np.abs(G)) >= 65504.0:
        raise OverflowError("core exceeds the fp16 range")
    return Ut, (None if rd == D else rnd(Ud[:, :rd])), rnd(G)


def reconstruct(Ut, Ud, G):
    """X~_n = U_T G_n U_d^T with identity factors where None ([JTRA] Mathematical statement)."""
    Xt = G
    if Ud is not None:
        Xt = Xt @ Ud.T
    if Ut is not None:
        Xt = np.einsum("tk,nkd->ntd", Ut, Xt)
    return Xt


def score_residual(X, Xt, sigma, bits, blk, n_chunk=16):
    """For every b: sum over blocks of ||Y - Q_b(Y)||^2 with Y = Q (X - X~) row-wise
    ([JTRA] Formulas, distortion display; computed in the rotated domain, which is
    exact because Q is orthogonal).  Also returns ||R||^2 - ||Y||^2."""
    N = X.shape[0]
    err = {b: 0.0 for b in bits}
    gap = 0.0
    for n0 in range(0, N, n_chunk):
        R = X[n0:n0 + n_chunk] - (Xt[n0:n0 + n_chunk] if Xt is not None else 0.0)
        Y = rotate_rows(R, sigma)
        r2 = float(np.sum(R * R))
        y2 = float(np.sum(Y * Y))
        gap += r2 - y2
        for b in bits:
            _, _, Yhat = quantize_blocks(Y, b, blk)
            d = Y - Yhat
            err[b] += float(np.sum(d * d))
    return err, gap


def build_table(X: np.ndarray, sigma: np.ndarray, rT: Sequence[int], rd: Sequence[int],
                bits: Sequence[int], blk: int, token_mode: str = "exact",
                omegas: Optional[Dict[int, np.ndarray]] = None, power_iters: int = 2,
                s_bytes: int = 2, round_fp16: bool = True, keep_factors: bool = False) -> TableResult:
    """Candidate table of one (group, K/V) tensor ([JTRA] Implementation notes:
    enumerate the grid, partial Tucker, residual, fixed orthogonal transform, quantize,
    measure normalised Frobenius distortion, store (D, C) pairs).

    X is the fp64 value of the bf16 input, shape [N, T, D]."""
    N, T, D = X.shape
    cands = candidate_list(T, D, rT, rd, bits)
    Ctab = cost_table(N, T, D, rT, rd, bits, blk, s_bytes)
    xn2 = float(np.sum(X * X))
    if not np.isfinite(xn2):
        raise FloatingPointError("non-finite input")
    Dtab = np.zeros(len(cands))
    gaps = np.zeros(len(cands))
    lam_d, Ud = feature_factor(X)
    res = TableResult(D=Dtab, C=Ctab, xnorm2=xn2, energy_gap=gaps,
                      lam_d=lam_d if keep_factors else None, Ud=Ud if keep_factors else None)
    kt = max([a for a in rT if a < T], default=0)
    for j, r_d in enumerate(rd):
        Yr = X if r_d == D else X @ Ud[:, :r_d]
        A = token_unfolding(Yr)
        if kt == 0:
            UT_r = None
        elif token_mode == "exact":
            _, UT_r = token_factor_exact(A, kt)
        else:
            UT_r = token_factor_randomized(A, bf16_bits_to_f64(omegas[r_d]), power_iters, kt)
        if keep_factors:
            res.UT[r_d] = UT_r
        for i, r_T in enumerate(rT):
            base = (i * len(rd) + j) * len(bits)
            if r_T == T and r_d == D:
                continue  # X stored verbatim: D = 0 for every b
            Ut, Udr, G = _factors_for(X, Ud, UT_r, r_T, r_d, round_fp16)
            Xt = reconstruct(Ut, Udr, G)
            err, gap = score_residual(X, Xt, sigma, bits, blk)
            for k, b in enumerate(bits):
                Dtab[base + k] = err[b] / xn2 if xn2 > 0 else 0.0
                gaps[base + k] = gap
    return res


# ============================================================== modelled tables [TS 4], referee notes
def gaussian_eps2(G: np.ndarray, bits: Sequence[int]) -> Dict[int, float]:
    """Calibration of the separable error model: eps^2(b) = sum ||g - Q_b(g)||^2 / sum ||g||^2
    over Gaussian rows g (one quantization block per row), eps^2(0) = 1 (no residual).  The
    pages calibrate eps^2(b) on a Gaussian round trip (the referee's notes on their Eq. (2))."""
    G = np.asarray(G, np.float64)
    e0 = float(np.sum(G * G))
    out = {}
    for b in bits:
        if b == 0:
            out[b] = 1.0
            continue
        _, _, Gh = quantize_blocks(G, b, G.shape[-1])
        out[b] = float(np.sum((G - Gh) ** 2)) / e0
    return out


def model_table(X: np.ndarray, rT: Sequence[int], rd: Sequence[int], bits: Sequence[int], eps2: Dict[int, float],
                token_mode: str = "exact", omegas: Optional[Dict[int, np.ndarray]] = None,
                power_iters: int = 2) -> np.ndarray:
    """Modelled candidate table D(z) = eps^2(b) tau(r_T, r_d) from spectra only (the pages'
    separable model e ~ eps^2(b) tau; no reconstruction, no residual pass).  tau is the energy
    outside the partial Tucker approximation, relative to ||X||^2: ||X||^2 less the energy of
    the top r_T token eigen-directions of Y(r_d) (ST-HOSVD: the core's energy), or of the top
    r_d feature directions when r_T = T; 0 for (T, D).  In randomized mode the captured
    energies are those of B = Q^T A, and everything the sketch misses counts as residual (the
    FlashJoLT tail-mass accounting).  Storage rounding is not modelled."""
    N, T, D = X.shape
    xn2 = float(np.sum(X * X))
    lam_d, Ud = feature_factor(X)
    kt = max([a for a in rT if a < T], default=0)
    out = np.zeros(len(rT) * len(rd) * len(bits))
    for j, r_d in enumerate(rd):
        Yr = X if r_d == D else X @ Ud[:, :r_d]
        total = xn2 if r_d == D else float(np.sum(lam_d[:r_d]))
        if kt:
            A = token_unfolding(Yr)
            if token_mode == "exact":
                lam_t = eigh_desc(A @ A.T)[0][:kt]
            else:
                lam_t = token_spectrum_randomized(A, bf16_bits_to_f64(omegas[r_d]), power_iters, kt)
        for i, r_T in enumerate(rT):
            captured = total if r_T == T else float(np.sum(lam_t[:r_T]))
            tau = 0.0 if (r_T == T and r_d == D) else max(0.0, (xn2 - captured) / xn2) if xn2 > 0 else 0.0
            for k, b in enumerate(bits):
                out[(i * len(rd) + j) * len(bits) + k] = eps2[b] * tau
    return out


# ============================================================== allocation [JTRA], [TS 3]
@dataclass
class Allocation:
    choice: np.ndarray      # [n_tables] candidate index per table
    lam: float              # lambda+ (byte price)
    total: int              # sum of chosen costs
    margin: np.ndarray      # [n_tables] (L2 - L1)/|L1| at lambda+ (0 for the critical table)


def _choose_at(Dt, Ct, lam: Fraction):
    """argmin D + lam*C; ties to lower C then lower index (exact arithmetic)."""
    best = None
    for i in range(len(Dt)):
        key = (Fraction(float(Dt[i])) + lam * int(Ct[i]), int(Ct[i]), i)
        if best is None or key < best:
            best = key
    return best[2]


def _hull(Dt, Ct):
    """Lower convex hull of the (C, D) points from the cheapest point up to the
    minimum-distortion point (ties in D resolved to the lower C).  Returns the vertices
    (ascending C) and the prices between consecutive vertices, descending."""
    best = {}
    for i in range(len(Dt)):
        c, d = int(Ct[i]), Fraction(float(Dt[i]))
        if c not in best or d < best[c]:
            best[c] = d
    P = sorted(best.items())  # ascending cost
    hull = []
    for c, d in P:
        while len(hull) >= 2:
            (c1, d1), (c2, d2) = hull[-2], hull[-1]
            # drop the middle point unless it lies strictly below the chord
            if (d2 - d1) * (c - c1) >= (d - d1) * (c2 - c1):
                hull.pop()
            else:
                break
        hull.append((c, d))
    k = min(range(len(hull)), key=lambda i: (hull[i][1], hull[i][0]))
    hull = hull[:k + 1]
    bps = [(d1 - d2) / (c2 - c1) for (c1, d1), (c2, d2) in zip(hull[:-1], hull[1:])]
    return hull, bps


def _vertex_index(Dt, Ct, vertex):
    c, d = vertex
    for i in range(len(Dt)):
        if int(Ct[i]) == c and Fraction(float(Dt[i])) == d:
            return i
    raise AssertionError("hull vertex not found")


def allocate(Dtab: np.ndarray, Ctab: np.ndarray, budget: int) -> Allocation:
    """Budget-feasible allocation at the smallest feasible byte price ([JTRA] Mathematical
    statement: for a fixed price every table independently takes argmin D + lambda*C; the
    price is searched so that the total fits B).  The price returned is
    lambda+ = inf{lambda : sum C(z*(lambda)) <= B}, found exactly by walking the
    breakpoints of every table's lower convex hull in rational arithmetic."""
    Dtab = np.asarray(Dtab, np.float64)
    Ctab = np.asarray(Ctab, np.uint64)
    nt, nc = Dtab.shape
    if int(sum(int(Ctab[t].min()) for t in range(nt))) > budget:
        raise ValueError("infeasible budget")
    hulls = [_hull(Dtab[t], Ctab[t]) for t in range(nt)]
    prices = {Fraction(0)}
    for _, bps in hulls:
        prices.update(bps)
    lam_star = None
    choice = None
    for lam in sorted(prices):
        ch = []
        for t in range(nt):
            hull, bps = hulls[t]
            j = sum(1 for bp in bps if bp > lam)  # vertex: cheaper end at a tie
            ch.append(_vertex_index(Dtab[t], Ctab[t], hull[j]))
        tot = sum(int(Ctab[t][ch[t]]) for t in range(nt))
        if tot <= budget:
            lam_star, choice = lam, ch
            break
    assert choice is not None
    margin = np.zeros(nt)
    for t in range(nt):
        assert _choose_at(Dtab[t], Ctab[t], lam_star) == choice[t]
        L = [Fraction(float(Dtab[t][i])) + lam_star * int(Ctab[t][i]) for i in range(nc)]
        L1 = L[choice[t]]
        others = [L[i] for i in range(nc) if i != choice[t]]
        L2 = min(others) if others else L1
        margin[t] = float((L2 - L1) / abs(L1)) if L1 != 0 else (float("inf") if L2 > L1 else 0.0)
    tot = sum(int(Ctab[t][choice[t]]) for t in range(nt))
    return Allocation(choice=np.array(choice, np.int32), lam=float(lam_star), total=tot, margin=margin)


def refine_swap(Dtab: np.ndarray, Ctab: np.ndarray, budget: int, choice,
                trace: Optional[list] = None) -> Tuple[np.ndarray, int]:
    """Greedy improvement of a budget-feasible allocation ([JTRA] Implementation notes:
    after the price search, optionally swap candidates with the best distortion reduction
    per added byte).

    A move replaces one table's candidate by another of strictly lower distortion such
    that the total cost still fits B.  Each round applies the best move and repeats until
    none is left.  Moves that add no bytes rank first (by the larger reduction); the others
    rank by (D_cur - D_new) / (C_new - C_cur), evaluated in fp64 as written.  Ties go to
    the lower table, then the lower candidate index.  Returns (choice, total bytes); the
    moves, as (table, candidate) pairs, are appended to ``trace`` when given."""
    Dtab = np.asarray(Dtab, np.float64)
    Ctab = np.asarray(Ctab, np.uint64)
    nt, nc = Dtab.shape
    ch = [int(c) for c in choice]
    total = sum(int(Ctab[t][ch[t]]) for t in range(nt))
    if total > budget:
        raise ValueError("starting allocation exceeds the budget")
    while True:
        best = None  # (free, score, table, cand) compared by the ranking above
        for t in range(nt):
            dc, cc = float(Dtab[t][ch[t]]), int(Ctab[t][ch[t]])
            for i in range(nc):
                dn, cn = float(Dtab[t][i]), int(Ctab[t][i])
                if not dn < dc or total - cc + cn > budget:
                    continue
                free = cn <= cc
                score = (dc - dn) if free else (dc - dn) / float(cn - cc)
                better = (best is None or (free and not best[0]) or
                          (free == best[0] and score > best[1]))
                if better:
                    best = (free, score, t, i)
        if best is None:
            break
        _, _, t, i = best
        total += int(Ctab[t][i]) - int(Ctab[t][ch[t]])
        ch[t] = i
        if trace is not None:
            trace.append((t, i))
    return np.array(ch, np.int32), total


def allocate_common(Dtab: np.ndarray, Ctab: np.ndarray, budget: int, allowed=None) -> int:
    """The fixed baselines of [JTRA] Implementation notes (fixed-rank or fixed-bit
    allocations; the pages' own toy baseline gives every group the same (r_T, r_d, b)):
    one candidate index shared by every table, the allowed candidate of least total
    distortion whose total cost fits B.  Ties go to the lower total cost, then the lower
    index.  ``allowed`` is a boolean mask over candidates (all when None)."""
    Dtab = np.asarray(Dtab, np.float64)
    Ctab = np.asarray(Ctab, np.uint64)
    nt, nc = Dtab.shape
    best = None
    for i in range(nc):
        if allowed is not None and not allowed[i]:
            continue
        cost = sum(int(Ctab[t][i]) for t in range(nt))
        if cost > budget:
            continue
        dist = math.fsum(float(Dtab[t][i]) for t in range(nt))
        key = (dist, cost, i)
        if best is None or key < best:
            best = key
    if best is None:
        raise ValueError("no allowed common candidate fits the budget")
    return best[2]


def lagrangian_choice(Dtab, Ctab, lam: float) -> np.ndarray:
    """z*(lambda) per table in fp64 (used by the monotonicity and Everett pins)."""
    lamf = Fraction(lam)
    return np.array([_choose_at(Dtab[t], Ctab[t], lamf) for t in range(Dtab.shape[0])], np.int32)


# ============================================================== encode / decode [RTR]
@dataclass
class Encoded:
    rT: int
    rd: int
    b: int
    blk: int
    sigma: np.ndarray
    Ut: Optional[np.ndarray]     # fp16 values [T, rT] or None
    Ud: Optional[np.ndarray]     # fp16 values [D, rd] or None
    G: Optional[np.ndarray]      # fp16 values [N, rT', rd'] or None (verbatim case)
    Xv: Optional[np.ndarray]     # verbatim X values (T, D case)
    codes: Optional[np.ndarray]  # int [N, T, D]
    scales: Optional[np.ndarray] # fp32 values [N, T, D/blk]


def encode_with_factors(X, sigma, Ut, Ud, G, b, blk, verbatim=False):
    """Residual codes for given stored factors ([RTR] Implementation notes: partition the
    rotated residual into blocks, store the scale and the integer codes)."""
    N, T, D = X.shape
    if verbatim:
        return None, None, np.zeros_like(X)
    Xt = reconstruct(Ut, Ud, G)
    if b == 0:
        return None, None, Xt
    Y = rotate_rows(X - Xt, sigma)
    q, s, _ = quantize_blocks(Y, b, blk)
    return q, s, Xt


def encode(X, sigma, rT, rd, b, blk, token_mode="exact", omegas=None, power_iters=2) -> Encoded:
    """Full encode of one table at z = (r_T, r_d, b) with the oracle's own factors."""
    N, T, D = X.shape
    if rT == T and rd == D:
        return Encoded(rT, rd, b, blk, sigma, None, None, None, X.copy(),
                       np.zeros((N, T, D), np.int64) if b else None,
                       np.zeros((N, T, D // blk)) if b else None)
    _, Udf = feature_factor(X)
    Yr = X if rd == D else X @ Udf[:, :rd]
    UT_r = None
    if rT < T:
        A = token_unfolding(Yr)
        if token_mode == "exact":
            _, UT_r = token_factor_exact(A, KMAX)
        else:
            UT_r = token_factor_randomized(A, bf16_bits_to_f64(omegas[rd]), power_iters, KMAX)
    Ut, Udr, G = _factors_for(X, Udf, UT_r, rT, rd)
    q, s, _ = encode_with_factors(X, sigma, Ut, Udr, G, b, blk)
    return Encoded(rT, rd, b, blk, sigma, Ut, Udr, G, None, q, s)


def decode_f64(e: Encoded) -> np.ndarray:
    """X^ = X~ + Q^T Q_b(QR) in fp64 ([JTRA] Formulas, first display; b = 0 gives X~)."""
    if e.Xv is not None:
        return e.Xv.copy()
    Xt = reconstruct(e.Ut, e.Ud, e.G)
    if e.b == 0:
        return Xt
    N, T, D = Xt.shape
    Yhat = (e.codes.reshape(N, T, D // e.blk, e.blk) * e.scales[..., None]).reshape(N, T, D)
    return Xt + unrotate_rows(Yhat, e.sigma)


def decode_bf16(e: Encoded) -> np.ndarray:
    return f64_to_bf16_bits(decode_f64(e))


# ============================================================== record byte layout
MAGIC = 0x544C4F4A  # "JOLT"


def attention(Khat: np.ndarray, Vhat: np.ndarray, Q: np.ndarray, scale: float) -> np.ndarray:
    """Attention over a decoded K/V cache ([JTRA] Implementation notes: reconstruct the
    low-rank part and residual immediately before attention), per slice n in fp64:
    O[n, i] = sum_t softmax_t(scale * Q[n, i] . K[n, t]) V[n, t].
    Khat, Vhat [N, T, D]; Q [N, nq, D]."""
    S = np.einsum("nid,ntd->nit", Q, Khat) * scale
    S = S - S.max(axis=2, keepdims=True)
    P = np.exp(S)
    P = P / P.sum(axis=2, keepdims=True)
    return np.einsum("nit,ntd->nid", P, Vhat)


def parse_record(buf: bytes, N: int, T: int, D: int) -> Encoded:
    """Read a compressed record in the library's documented byte layout (header of 256
    bytes, then 256-byte aligned sections: U_T fp16 [T, r_T], U_d fp16 [D, r_d], core
    fp16 [N, r_T, r_d] or verbatim bf16 X, packed b-bit two's-complement codes in
    row-major element order, fp32 scales [N, T, D/blk])."""
    mv = memoryview(buf)
    magic, ver, n, t, d, rT, rd, b, blk, flags = struct.unpack_from("<IIiiiiiiii", mv, 0)
    if magic != MAGIC or ver != 1 or (n, t, d) != (N, T, D):
        raise ValueError("bad record header")
    total, off_ut, off_ud, off_core, off_codes, off_scales = struct.unpack_from("<QQQQQQ", mv, 40)
    sbits = np.frombuffer(bytes(mv[128:128 + (D + 7) // 8]), dtype=np.uint8)
    neg = np.unpackbits(sbits, bitorder="little")[:D]
    sigma = np.where(neg == 1, -1, 1).astype(np.int8)
    f16 = lambda off, cnt: np.frombuffer(bytes(mv[off:off + 2 * cnt]), dtype=np.float16).astype(np.float64)
    if rT == T and rd == D:
        xv = bf16_bits_to_f64(np.frombuffer(bytes(mv[off_core:off_core + 2 * N * T * D]), np.uint16)).reshape(N, T, D)
        return Encoded(rT, rd, b, blk, sigma, None, None, None, xv, None, None)
    Ut = f16(off_ut, T * rT).reshape(T, rT) if rT < T else None
    Ud = f16(off_ud, D * rd).reshape(D, rd) if rd < D else None
    G = f16(off_core, N * rT * rd).reshape(N, rT, rd)
    codes = scales = None
    if b > 0:
        nel = N * T * D
        raw = np.frombuffer(bytes(mv[off_codes:off_codes + -(-(b * nel) // 8)]), np.uint8)
        per = 8 // b
        # element i sits in byte i // per at bit offset (i % per) * b, two's complement
        fields = [(raw >> np.uint8(j * b)) & np.uint8((1 << b) - 1) for j in range(per)]
        u = np.stack(fields, axis=1).reshape(-1)[:nel].astype(np.int16)
        codes = np.where(u >= (1 << (b - 1)), u - (1 << b), u).astype(np.int8).reshape(N, T, D)
        scales = np.frombuffer(bytes(mv[off_scales:off_scales + 4 * N * T * (D // blk)]), np.float32)
        scales = scales.astype(np.float64).reshape(N, T, D // blk)
    return Encoded(rT, rd, b, blk, sigma, Ut, Ud, G, None, codes, scales)


# ============================================================== row-sampled decode/encode
def reconstruct_rows(e: Encoded, n_idx: np.ndarray, t_idx: np.ndarray) -> np.ndarray:
    """X~[n, t, :] for selected (n, t) rows only ([JTRA] Mathematical statement: the
    reconstruction is U_T G_n U_d^T row by row)."""
    if e.Xv is not None:
        return e.Xv[n_idx, t_idx, :].copy()
    G = e.G[n_idx]                         # [S, rT', rd']
    if e.Ud is not None:
        G = G @ e.Ud.T                     # [S, rT', D]
    if e.Ut is None:
        return G[np.arange(len(t_idx)), t_idx, :]
    return np.einsum("sk,skd->sd", e.Ut[t_idx], G)


def decode_rows_f64(e: Encoded, n_idx: np.ndarray, t_idx: np.ndarray) -> np.ndarray:
    """Decoded rows X^ = X~ + Q^T Q_b(QR) for selected rows (fp64)."""
    Xt = reconstruct_rows(e, n_idx, t_idx)
    if e.Xv is not None or e.b == 0:
        return Xt
    D = Xt.shape[1]
    Yhat = (e.codes[n_idx, t_idx].reshape(-1, D // e.blk, e.blk) * e.scales[n_idx, t_idx][..., None]).reshape(-1, D)
    return Xt + unrotate_rows(Yhat, e.sigma)


def decode_eval_bound(e: Encoded, n_idx: np.ndarray, t_idx: np.ndarray) -> np.ndarray:
    """Bound on the error of X^ evaluated in fp32 for selected rows ([JTRA] Formulas, first
    display, evaluated as the decoded cache is stored: fp32, then one rounding to bf16).
    A decoder that sums the products of the stored fp16 factors and the residual term in
    fp32 is off the exact value by at most u (2K + 8) S per element, u = 2^-24, with S the
    sum of the magnitudes of everything it adds: sum_k |L_tk| sum_j |G_kj| |U_fj| (the
    reconstruction of the chosen chain with absolute values; K = inner dimension) plus the
    magnitude of the residual term.  0 for verbatim records."""
    if e.Xv is not None:
        return np.zeros((len(n_idx), e.Xv.shape[2]))
    G = np.abs(e.G[n_idx])                                  # [S, rT', rd']
    if e.Ud is not None:
        G = G @ np.abs(e.Ud).T                              # [S, rT', D]
    if e.Ut is None:
        S = G[np.arange(len(t_idx)), t_idx, :]
        K = e.G.shape[2]
    else:
        S = np.einsum("sk,skd->sd", np.abs(e.Ut[t_idx]), G)
        K = e.Ut.shape[1]
    if e.b > 0:
        D = S.shape[1]
        Yhat = (e.codes[n_idx, t_idx].reshape(-1, D // e.blk, e.blk) * e.scales[n_idx, t_idx][..., None]).reshape(-1, D)
        S = S + np.abs(unrotate_rows(Yhat, e.sigma))
    return 2.0 ** -24 * (2 * K + 8) * S


def bf16_consistent(got_bits: np.ndarray, x: np.ndarray, bound: np.ndarray) -> np.ndarray:
    """Acceptance of a bf16 value computed from the exact x (fp64) with an evaluation error
    of at most `bound`: True where got is within one bf16 ulp of bf16(x) (round to nearest
    even), or lies between the roundings of x - bound and x + bound."""
    def ordered(b):
        b = np.asarray(b).astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    x = np.asarray(x, np.float64)
    g, w = ordered(got_bits), ordered(f64_to_bf16_bits(x))
    lo, hi = ordered(f64_to_bf16_bits(x - bound)), ordered(f64_to_bf16_bits(x + bound))
    return (np.abs(g - w) <= 1) | ((g >= lo) & (g <= hi))


def encode_rows(X_rows: np.ndarray, e: Encoded, n_idx: np.ndarray, t_idx: np.ndarray):
    """Codes and scales of selected rows given the stored factors of `e`."""
    Xt = reconstruct_rows(e, n_idx, t_idx)
    Y = rotate_rows(X_rows - Xt, e.sigma)
    q, s, _ = quantize_blocks(Y, e.b, e.blk)
    return q, s


# ============================================================== streaming admission [RTR], [JTRA]
# Both pages place the compressor on the cache write path: the selected Tucker factors are
# maintained and every incoming token block is reconstructed and its residual R = X - X~
# rotated and quantized ([RTR] Implementation notes; [JTRA] Implementation notes, admission
# time).  Reading taken here: the feature factor and the cores of the frozen record stay
# fixed; an incoming token has no row in U_T, so its row is the least-squares fit of the
# token against the frozen reconstruction operator.  Singular values below STREAM_RCOND of
# the largest are dropped (minimum-norm solution), so a rank-deficient operator (N r_d < r_T,
# or zero cores) has a unique answer.
STREAM_RCOND = 1e-6
BLOCK_MAGIC = 0x42544C4A  # "JLTB"


def _stream_operator(e: Encoded, N: int, D: int):
    """R_n (K x D) of the frozen record, X~_n = L R_n: G_n U_d^T (U_d = I when r_d = D) for
    r_T < T; U_d^T (the same for every slice) for r_T = T."""
    if e.Ut is None:
        return np.broadcast_to(e.Ud.T, (N,) + e.Ud.T.shape)
    return e.G if e.Ud is None else e.G @ e.Ud.T


def stream_left_factor(e: Encoded, Xn: np.ndarray, round_fp16: bool = True) -> np.ndarray:
    """Left factor of an incoming block X' [N, t', D] against the frozen record e.

    r_T < T: one row per token shared by the slices, as U_T's rows are:
        l_t = argmin sum_n ||X'_n[t] - l_t R_n||^2  ->  L [t', r_T];
    r_T = T (identity token factor): the block's own core rows, slice by slice:
        l_{n,t} = argmin ||X'_n[t] - l_{n,t} U_d^T||^2  ->  L [N, t', r_d].
    Minimum-norm least squares (numpy lstsq) with relative cutoff STREAM_RCOND; stored as
    fp16 (round to nearest even) unless round_fp16 is False."""
    N, tn, D = Xn.shape
    R = _stream_operator(e, N, D)
    rnd = fp16_round if round_fp16 else (lambda a: a)
    if e.Ut is None:
        Ud = e.Ud
        L = np.stack([np.linalg.lstsq(Ud, Xn[n].T, rcond=STREAM_RCOND)[0].T for n in range(N)])
        return rnd(L)
    # stack the slices: [R_0^T; R_1^T; ...] (N D x K) times l^T = [X'_0[t]^T; X'_1[t]^T; ...]
    A = np.concatenate([R[n].T for n in range(N)], axis=0)
    B = np.concatenate([Xn[n].T for n in range(N)], axis=0)
    return rnd(np.linalg.lstsq(A, B, rcond=STREAM_RCOND)[0].T)


def stream_encode(e: Encoded, Xn: np.ndarray, L: Optional[np.ndarray] = None) -> Encoded:
    """Block record contents of X' against the frozen record e: the left factor (the
    oracle's own, or a given stored one for conditional code parity), then the rotated
    residual codes and scales with the frozen rotation ([RTR] Implementation notes)."""
    N, tn, D = Xn.shape
    if e.Xv is not None:  # (T, D): the block is kept verbatim
        return Encoded(e.rT, e.rd, e.b, e.blk, e.sigma, None, None, None, Xn.copy(), None, None)
    if L is None:
        L = stream_left_factor(e, Xn)
    if e.Ut is None:
        Ut, G = None, L
    else:
        Ut, G = L, e.G
    q, s, _ = encode_with_factors(Xn, e.sigma, Ut, e.Ud, G, e.b, e.blk)
    return Encoded(e.rT, e.rd, e.b, e.blk, e.sigma, Ut, e.Ud, G, None, q, s)


def block_distortion(Xn: np.ndarray, blk: Encoded) -> float:
    """||X' - X^'||^2 / ||X'||^2 of a decoded block in fp64 ([JTRA] Formulas, distortion)."""
    x2 = float(np.sum(Xn * Xn))
    return float(np.sum((Xn - decode_f64(blk)) ** 2)) / x2 if x2 > 0 else 0.0


def block_bytes(N: int, tn: int, D: int, T: int, rT: int, rd: int, b: int, blk: int) -> int:
    """Bytes of a block record: 256-byte header, then 256-aligned sections: the left factor
    (fp16 [t', r_T], or [N, t', r_d] when r_T = T; bf16 X' verbatim for (T, D)), packed b-bit
    codes, fp32 scales (one per block of blk values)."""
    out = HDR_BYTES
    if rT == T and rd == D:
        return out + pad(2 * N * tn * D)
    out += pad(2 * tn * rT) if rT < T else pad(2 * N * tn * rd)
    if b > 0:
        out += pad(-(-(b * N * tn * D) // 8)) + pad(4 * N * tn * (D // blk))
    return out


def parse_block(buf: bytes, frozen: Encoded, N: int, tn: int, D: int) -> Encoded:
    """Read a block record (header: magic "JLTB", version, N, t', D, r_T, r_d, b, blk, T of the
    frozen record; then the 64-bit total and the offsets of the left factor, codes and
    scales) and join it to its frozen record."""
    mv = memoryview(buf)
    magic, ver, n, t, d, rT, rd, b, blk, T = struct.unpack_from("<IIiiiiiiii", mv, 0)
    if magic != BLOCK_MAGIC or ver != 1 or (n, t, d) != (N, tn, D):
        raise ValueError("bad block header")
    total, off_l, off_codes, off_scales = struct.unpack_from("<QQQQ", mv, 40)
    f16 = lambda off, cnt: np.frombuffer(bytes(mv[off:off + 2 * cnt]), dtype=np.float16).astype(np.float64)
    if frozen.Xv is not None:
        xv = bf16_bits_to_f64(np.frombuffer(bytes(mv[off_l:off_l + 2 * N * tn * D]), np.uint16)).reshape(N, tn, D)
        return Encoded(rT, rd, b, blk, frozen.sigma, None, None, None, xv, None, None)
    if frozen.Ut is None:
        Ut, G = None, f16(off_l, N * tn * rd).reshape(N, tn, rd)
    else:
        Ut, G = f16(off_l, tn * rT).reshape(tn, rT), frozen.G
    codes = scales = None
    if b > 0:
        nel = N * tn * D
        raw = np.frombuffer(bytes(mv[off_codes:off_codes + -(-(b * nel) // 8)]), np.uint8)
        per = 8 // b
        fields = [(raw >> np.uint8(j * b)) & np.uint8((1 << b) - 1) for j in range(per)]
        u = np.stack(fields, axis=1).reshape(-1)[:nel].astype(np.int16)
        codes = np.where(u >= (1 << (b - 1)), u - (1 << b), u).astype(np.int8).reshape(N, tn, D)
        scales = np.frombuffer(bytes(mv[off_scales:off_scales + 4 * N * tn * (D // blk)]), np.float32)
        scales = scales.astype(np.float64).reshape(N, tn, D // blk)
    return Encoded(rT, rd, b, blk, frozen.sigma, Ut, frozen.Ud, G, None, codes, scales)
