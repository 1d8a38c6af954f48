"""Seeded synthetic KV-cache generator shared by the GPU path, the oracle and the bench.

This module holds no arithmetic of the compression method itself: it only draws
the input tensors (bf16 group tensors X[N,T,D]) and the random numbers the method
consumes (the rotation sign vector and the Gaussian sketch matrices), so that
both implementations see identical bytes.

Generative model (a stand-in for the Mistral-7B / LLaMA-2-13B caches the pages
measure on, which are not available):

    X_n[t, j] = c_j * sum_k sigma_k * a_{n,t,k} * V[j, k]  +  0.02 * eps_{n,t,j}

* V is a Haar-random orthogonal D x D matrix (QR of a Gaussian, sign-fixed),
  one per (group, K/V) table;
* a_{n,.,k} is a stationary AR(1) process over tokens (rho = 0.9, unit variance),
  independent over (n, k);
* keys:   sigma_k = (k+1)^-1.0, c_j = exp(N(0, variance 0.5)) with a few outlier
  channels multiplied by 8;
* values: sigma_k = (k+1)^-0.3 (flat spectrum), c_j = 1;
* eps ~ N(0, 1); the result is rounded to bf16 (fp64 -> fp32 -> bf16, both RNE).

Every table is seeded by ``SeedSequence([config_id, group, kv])``; signs and
sketches use the same prefix plus a stream tag, so any table can be regenerated
alone.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get_workload", "generate_table", "rotation_signs",
    "sketch_omega", "f32_to_bf16_bits", "bf16_bits_to_f32", "bf16_bits_to_f64",
    "fp16_bytes", "generate_low_rank_table", "generate_queries", "gaussian_rows", "generate_block",
    "generate_token_spectrum_table",
]

RHO = 0.9
NOISE = 0.02
SKETCH_COLS_DEFAULT = 40  # q_cap (32) + oversample (8)


@dataclass(frozen=True)
class Workload:
    """Shape and budget description of one synthetic workload."""
    name: str
    config_id: int
    N: int              # slices per table (layers-in-group x KV heads)
    T: int              # cached tokens
    D: int              # head width
    n_groups: int
    kinds: Tuple[int, ...]  # 0 = K, 1 = V
    n_outlier: int      # outlier channels (x8) in K
    token_mode: str     # "exact" | "randomized"
    ratios: Tuple[float, ...]   # budget = floor(fp16 bytes / ratio)
    quant_block: int
    rT: Tuple[int, ...] = field(default=())
    rd: Tuple[int, ...] = field(default=())
    bits: Tuple[int, ...] = (0, 2, 4, 8)
    q_cap: int = 32
    oversample: int = 8
    power_iters: int = 2

    @property
    def n_tables(self) -> int:
        return self.n_groups * len(self.kinds)

    def table_ids(self):
        """(g, c) for table index t = len(kinds)*g + position of c."""
        return [(g, c) for g in range(self.n_groups) for c in self.kinds]

    def budgets(self):
        fb = fp16_bytes(self)
        return [int(fb // r) if float(r).is_integer() else int(np.floor(fb / r)) for r in self.ratios]

    def x_bytes(self) -> int:
        return 2 * self.N * self.T * self.D * self.n_tables


def _wl(name, cid, N, T, D, G, kinds, m, mode, ratios, blk):
    return Workload(name=name, config_id=cid, N=N, T=T, D=D, n_groups=G, kinds=kinds,
                    n_outlier=m, token_mode=mode, ratios=ratios, quant_block=blk,
                    rT=(4, 8, 16, 32, T), rd=(4, 8, 16, 32, D))


WORKLOADS = {
    # tiny exact case: 1 group, keys only
    "tiny": _wl("tiny", 0, 4, 64, 64, 1, (0,), 2, "exact", (2.0,), 64),
    # Mistral-7B shaped GQA cache (32 layers x 8 KV heads, 4 layers per group)
    "mistral_t512": _wl("mistral_t512", 1, 32, 512, 128, 8, (0, 1), 4, "exact", (2.0,), 128),
    "mistral_t1024_flash": _wl("mistral_t1024_flash", 2, 32, 1024, 128, 8, (0, 1), 4, "randomized", (3.0,), 128),
    # LLaMA-2-13B shaped MHA cache (40 layers x 40 heads, 4 layers per group)
    "llama13b_t2048": _wl("llama13b_t2048", 3, 160, 2048, 128, 10, (0, 1), 4, "randomized", (2.0, 3.0), 128),
    # long-context stress: Mistral shape at 32k tokens
    "mistral_t32k": _wl("mistral_t32k", 4, 32, 32768, 128, 8, (0, 1), 4, "randomized", (2.0,), 128),
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def fp16_bytes(w: Workload) -> int:
    return 2 * w.N * w.T * w.D * w.n_tables


# ---------------------------------------------------------------- bf16 helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


# ---------------------------------------------------------------- generators
def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _ar1(rng: np.random.Generator, shape, rho=RHO) -> np.ndarray:
    """Stationary unit-variance AR(1) along axis 1 of `shape` = (N, T, K)."""
    from scipy.signal import lfilter
    eta = rng.standard_normal(shape)
    g = np.sqrt(1.0 - rho * rho)
    eta[:, 0, :] /= g  # so that a_0 = eta_0 exactly
    return lfilter([g], [1.0, -rho], eta, axis=1)


def _mixing(w: Workload, c: int, rng: np.random.Generator) -> np.ndarray:
    """[k, j] = sigma_k V[j, k] c_j of one table (the first draws of its generator)."""
    D = w.D
    Gm = rng.standard_normal((D, D))
    Qm, Rm = np.linalg.qr(Gm)
    Qm = Qm * np.sign(np.diag(Rm))[None, :]
    if c == 0:
        sig = (np.arange(D) + 1.0) ** -1.0
        ch = np.exp(rng.normal(0.0, np.sqrt(0.5), D))
        out = rng.choice(D, size=w.n_outlier, replace=False)
        ch[out] *= 8.0
    else:
        sig = (np.arange(D) + 1.0) ** -0.3
        ch = np.ones(D)
    return (Qm * sig[None, :]).T * ch[None, :]


def generate_table(w: Workload, g: int, c: int, n_chunk: int = 8) -> np.ndarray:
    """bf16 bits [N, T, D] of table (group g, kind c) of workload w."""
    N, T, D = w.N, w.T, w.D
    rng = _rng(w.config_id, g, c)
    mix = _mixing(w, c, rng)
    out_bits = np.empty((N, T, D), dtype=np.uint16)
    for n0 in range(0, N, n_chunk):
        n1 = min(N, n0 + n_chunk)
        a = _ar1(rng, (n1 - n0, T, D))
        x = a @ mix
        x += NOISE * rng.standard_normal((n1 - n0, T, D))
        out_bits[n0:n1] = f32_to_bf16_bits(x.astype(np.float32))
    return out_bits


def generate_block(w: Workload, g: int, c: int, tn: int, tag: int = 0) -> np.ndarray:
    """bf16 bits [N, tn, D]: a block of tn further tokens of table (g, c), i.e. the same
    feature mixing (V, spectrum, channel scales) as generate_table with a fresh stationary
    AR(1) token process and noise (stream tag 3, block `tag`)."""
    mix = _mixing(w, c, _rng(w.config_id, g, c))
    rng = _rng(w.config_id, g, c, 3, tag)
    x = _ar1(rng, (w.N, tn, w.D)) @ mix
    x += NOISE * rng.standard_normal((w.N, tn, w.D))
    return f32_to_bf16_bits(x.astype(np.float32))


def generate_queries(w: Workload, g: int, nq: int) -> np.ndarray:
    """bf16 bits [N, nq, D] of synthetic attention queries for layer group g: nq queries per
    slice (e.g. the query heads sharing one KV head), standard normal entries."""
    rng = _rng(w.config_id, g, 7)
    return f32_to_bf16_bits(rng.standard_normal((w.N, nq, w.D)).astype(np.float32))


def gaussian_rows(D: int, rows: int, seed: int = 0) -> np.ndarray:
    """float32 [rows, D] standard normal rows: the calibration input of the separable error
    model's quantizer factor (one quantization block per row)."""
    rng = np.random.default_rng(np.random.SeedSequence([2000, D, seed]))
    return rng.standard_normal((rows, D)).astype(np.float32)


def generate_low_rank_table(N: int, T: int, D: int, rank: int, noise: float, seed: int) -> np.ndarray:
    """bf16 bits [N, T, D] of a degenerate table: every slice is a combination of the same
    `rank` token and feature directions (one of them dominant) plus `noise` times a
    Gaussian, so the token and feature spectra collapse after `rank` components."""
    rng = np.random.default_rng(np.random.SeedSequence([1000, seed]))
    U = rng.standard_normal((T, rank))
    V = rng.standard_normal((rank, D))
    w = 1.0 / (1.0 + np.arange(rank)) ** 2
    w[0] *= 20.0
    out = np.empty((N, T, D), dtype=np.uint16)
    for n in range(N):
        c = rng.standard_normal(rank) * w
        x = 0.05 * ((U * c[None, :]) @ V + noise * rng.standard_normal((T, D)))
        out[n] = f32_to_bf16_bits(x.astype(np.float32))
    return out


def generate_token_spectrum_table(N: int, T: int, D: int, spectrum: np.ndarray, seed: int) -> np.ndarray:
    """bf16 bits [N, T, D] whose token Gram sum_n X_n X_n^T has the eigenvalues `spectrum`
    (length K <= min(T, N D)) before the bf16 rounding: X_n = U diag(sqrt(spectrum)) W_n with
    U [T, K] orthonormal columns and the K rows of [W_0 | ... | W_{N-1}] orthonormal, both
    seeded Haar-random.  A slowly decaying spectrum makes a hard case for subspace iteration
    on the token Gram."""
    lam = np.asarray(spectrum, np.float64)
    K = lam.shape[0]
    if K > T or K > N * D:
        raise ValueError("spectrum longer than the token or slice-feature dimension")
    rng = np.random.default_rng(np.random.SeedSequence([3000, seed]))
    U, _ = np.linalg.qr(rng.standard_normal((T, K)))
    W, _ = np.linalg.qr(rng.standard_normal((N * D, K)))
    W = W.T.reshape(K, N, D)
    x = np.einsum("tk,knd->ntd", U * np.sqrt(lam)[None, :], W, optimize=True)
    return f32_to_bf16_bits(x.astype(np.float32))


def rotation_signs(w: Workload, g: int, c: int) -> np.ndarray:
    """int8 vector of +-1 of length D: the random signs of the rotation of table (g, c)."""
    rng = _rng(w.config_id, g, c, 1)
    bits = rng.integers(0, 2, size=w.D)
    return np.where(bits == 1, -1, 1).astype(np.int8)


def sketch_omega(w: Workload, g: int, c: int, rd: int, cols: int = SKETCH_COLS_DEFAULT) -> np.ndarray:
    """bf16 bits [N*rd, cols]: Gaussian test matrix for the token-mode range finder of
    table (g, c) at feature rank rd (rd == D means the unprojected tensor)."""
    rng = _rng(w.config_id, g, c, 2, rd)
    om = rng.standard_normal((w.N * rd, cols))
    return f32_to_bf16_bits(om.astype(np.float32))
