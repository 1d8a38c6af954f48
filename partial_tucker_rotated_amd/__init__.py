"""Python binding of the JoLT KV-cache candidate-table engine (libjolt.so, gfx950).

Argument marshalling only: every step of the computation runs in the HIP library.
Device buffers are anything with ``data_ptr()`` (torch tensors); the stream defaults
to torch's current stream.  The C declarations and their semantics are in
``include/jolt.h``.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "JoltError", "JoltConfig", "load", "default_config", "workspace_size", "cost_table",
    "record_bytes", "build_tables", "model_tables", "allocate", "encode", "encode_built", "decode", "N_CAND",
    "last_build_info",
    "TOKEN_EXACT", "TOKEN_RANDOMIZED", "EXPORTED_SYMBOLS",
]

N_CAND = 100
TOKEN_EXACT, TOKEN_RANDOMIZED = 0, 1
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libjolt.so")

EXPORTED_SYMBOLS = (
    "jolt_default_config", "jolt_status_string", "jolt_workspace_size", "jolt_cost_table",
    "jolt_build_tables", "jolt_model_tables", "jolt_allocate", "jolt_refine_swap", "jolt_allocate_common", "jolt_record_bytes",
    "jolt_encode", "jolt_encode_built", "jolt_decode", "jolt_attend_workspace_size", "jolt_attend",
    "jolt_stream_state_bytes", "jolt_stream_block_bytes", "jolt_stream_workspace_size", "jolt_stream_prepare",
    "jolt_stream_encode", "jolt_stream_decode", "jolt_last_build_info", "jolt_stream_encode_noalloc",
)

_STATUS = {0: "JOLT_OK", -1: "JOLT_EINVAL", -2: "JOLT_ENOMEM", -3: "JOLT_EDEVICE",
           -4: "JOLT_EINFEASIBLE", -5: "JOLT_ERANGE", -6: "JOLT_ENONFINITE"}


class JoltError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        self.name = _STATUS.get(code, str(code))
        super().__init__(f"{where}: {self.name}")


class JoltConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "N", "T", "D", "n_tables", "quant_block", "s_bytes", "align_bytes", "token_mode",
        "q_cap", "oversample", "power_iters", "exact_iters", "factor_precision", "exact_max_iters")]


class FactorInfo(ctypes.Structure):
    _fields_ = [("iterations", ctypes.c_int32), ("converged", ctypes.c_int32), ("max_residual", ctypes.c_double)]


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m partial_tucker_rotated_amd._build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
    cfgp = ctypes.POINTER(JoltConfig)
    lib.jolt_default_config.argtypes = [cfgp, i32, i32, i32, i32]
    lib.jolt_default_config.restype = None
    lib.jolt_status_string.argtypes = [i32]
    lib.jolt_status_string.restype = ctypes.c_char_p
    lib.jolt_workspace_size.argtypes = [cfgp, ctypes.POINTER(sz)]
    lib.jolt_cost_table.argtypes = [cfgp, P]
    lib.jolt_record_bytes.argtypes = [cfgp, i32, ctypes.POINTER(u64)]
    lib.jolt_build_tables.argtypes = [cfgp, P, P, P, P, P, P, P, sz, P]
    lib.jolt_model_tables.argtypes = [cfgp, P, P, P, P, i32, P, P, P, P, P, sz, P]
    lib.jolt_allocate.argtypes = [P, P, i32, i32, u64, P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(u64)]
    lib.jolt_refine_swap.argtypes = [P, P, i32, i32, u64, P, ctypes.POINTER(u64), ctypes.POINTER(i32)]
    lib.jolt_allocate_common.argtypes = [P, P, i32, i32, u64, P, ctypes.POINTER(i32), ctypes.POINTER(u64),
                                         ctypes.POINTER(ctypes.c_double)]
    lib.jolt_encode.argtypes = [cfgp, P, P, P, P, P, P, sz, P]
    lib.jolt_encode_built.argtypes = [cfgp, P, P, P, P, P, sz, P]
    lib.jolt_decode.argtypes = [cfgp, P, P, P, P]
    lib.jolt_last_build_info.argtypes = [P, ctypes.POINTER(FactorInfo)]
    lib.jolt_attend_workspace_size.argtypes = [cfgp, i32, i32, ctypes.POINTER(sz)]
    lib.jolt_attend.argtypes = [cfgp, i32, P, P, P, P, P, i32, ctypes.c_float, P, P, sz, P]
    lib.jolt_stream_state_bytes.argtypes = [ctypes.POINTER(sz)]
    lib.jolt_stream_block_bytes.argtypes = [cfgp, i32, i32, ctypes.POINTER(u64)]
    lib.jolt_stream_workspace_size.argtypes = [cfgp, i32, ctypes.POINTER(sz)]
    lib.jolt_stream_prepare.argtypes = [cfgp, P, P, P, P]
    lib.jolt_stream_encode.argtypes = [cfgp, P, P, P, P, i32, P, P, P, sz, P]
    lib.jolt_stream_decode.argtypes = [cfgp, P, P, P, i32, P, P]
    lib.jolt_stream_encode_noalloc.argtypes = [cfgp, P, P, P, P, i32, P, P, P]
    lib.jolt_debug_timer_enable.argtypes = [i32, i32]
    lib.jolt_debug_timer_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]
    lib.jolt_debug_read.argtypes = [cfgp, P, i32, P, sz]
    for f in ("jolt_workspace_size", "jolt_cost_table", "jolt_record_bytes", "jolt_build_tables", "jolt_model_tables",
              "jolt_allocate", "jolt_refine_swap", "jolt_allocate_common", "jolt_encode", "jolt_encode_built",
              "jolt_decode", "jolt_attend_workspace_size", "jolt_attend", "jolt_stream_state_bytes",
              "jolt_stream_block_bytes", "jolt_stream_workspace_size", "jolt_stream_prepare", "jolt_stream_encode",
              "jolt_stream_decode", "jolt_debug_timer_enable", "jolt_last_build_info", "jolt_stream_encode_noalloc",
              "jolt_debug_timer_read", "jolt_debug_read"):
        getattr(lib, f).restype = i32
    _lib = lib
    return lib


def _check(code: int, where: str):
    if code != 0:
        raise JoltError(code, where)


def default_config(N: int, T: int, D: int, n_tables: int, token_mode: int = TOKEN_EXACT,
                   exact_iters: Optional[int] = None, power_iters: int = 2, factor_precision: int = 0,
                   exact_max_iters: Optional[int] = None) -> JoltConfig:
    """jolt_default_config, then the given overrides (None keeps the library's default)."""
    cfg = JoltConfig()
    load().jolt_default_config(ctypes.byref(cfg), N, T, D, n_tables)
    cfg.token_mode = token_mode
    if exact_iters is not None:
        cfg.exact_iters = exact_iters
    if exact_max_iters is not None:
        cfg.exact_max_iters = exact_max_iters
    cfg.power_iters = power_iters
    cfg.factor_precision = factor_precision
    return cfg


def last_build_info(workspace) -> dict:
    """jolt_last_build_info: how the last factor computation in `workspace` obtained its
    token factors (iterations, converged, max_residual)."""
    info = FactorInfo()
    _check(load().jolt_last_build_info(workspace.data_ptr(), ctypes.byref(info)), "jolt_last_build_info")
    return {"iterations": int(info.iterations), "converged": bool(info.converged),
            "max_residual": float(info.max_residual)}


def workspace_size(cfg: JoltConfig) -> int:
    out = ctypes.c_size_t(0)
    _check(load().jolt_workspace_size(ctypes.byref(cfg), ctypes.byref(out)), "jolt_workspace_size")
    return int(out.value)


def cost_table(cfg: JoltConfig) -> np.ndarray:
    C = np.zeros(N_CAND, dtype=np.uint64)
    _check(load().jolt_cost_table(ctypes.byref(cfg), C.ctypes.data), "jolt_cost_table")
    return C


def record_bytes(cfg: JoltConfig, cand: int) -> int:
    out = ctypes.c_uint64(0)
    _check(load().jolt_record_bytes(ctypes.byref(cfg), int(cand), ctypes.byref(out)), "jolt_record_bytes")
    return int(out.value)


def _need(t, nbytes: int, what: str):
    """A contiguous device tensor of at least `nbytes` bytes (the C side derives every
    layout from cfg and the candidate, so a short buffer would be read or written past its
    end)."""
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{what}: a device tensor is required")
    if not t.is_contiguous():
        raise ValueError(f"{what}: the tensor must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{what}: {have} bytes, at least {nbytes} needed")


def _need_all(ts, nbytes, what: str, count: int):
    if ts is None or len(ts) != count:
        raise ValueError(f"{what}: one tensor per table expected ({count})")
    for k, t in enumerate(ts):
        _need(t, nbytes(k) if callable(nbytes) else nbytes, f"{what}[{k}]")


def _x_bytes(cfg, T=None) -> int:
    return 2 * cfg.N * (cfg.T if T is None else T) * cfg.D


def _omega_bytes(cfg) -> int:
    return 2 * cfg.N * (4 + 8 + 16 + 32 + cfg.D) * (cfg.q_cap + cfg.oversample)


def _check_inputs(cfg, xs, signs, omegas):
    _need_all(xs, _x_bytes(cfg), "xs", cfg.n_tables)
    _need(signs, cfg.n_tables * cfg.D, "signs")
    if cfg.token_mode == TOKEN_RANDOMIZED:
        _need_all(omegas, _omega_bytes(cfg), "omegas", cfg.n_tables)


def _ptr_array(bufs: Optional[Sequence]) -> Optional[ctypes.Array]:
    if bufs is None:
        return None
    return (ctypes.c_void_p * len(bufs))(*[b.data_ptr() for b in bufs])


def _stream(stream) -> int:
    if stream is not None:
        return int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def build_tables(cfg: JoltConfig, xs: Sequence, signs, omegas: Optional[Sequence], workspace, stream=None):
    """Candidate tables of every table: returns (D [n_tables, 100] float64,
    C [n_tables, 100] uint64, xnorm2 [n_tables] float64)."""
    nt = cfg.n_tables
    if len(xs) != nt or (omegas is not None and len(omegas) != nt):
        raise ValueError("one input (and sketch) per table expected")
    _check_inputs(cfg, xs, signs, omegas)
    D = np.zeros((nt, N_CAND), np.float64)
    C = np.zeros((nt, N_CAND), np.uint64)
    xn = np.zeros(nt, np.float64)
    xa, oa = _ptr_array(xs), _ptr_array(omegas)
    code = load().jolt_build_tables(ctypes.byref(cfg), xa, signs.data_ptr(), oa, D.ctypes.data, C.ctypes.data,
                                    xn.ctypes.data, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                    _stream(stream))
    _check(code, "jolt_build_tables")
    return D, C, xn


def model_tables(cfg: JoltConfig, xs: Sequence, signs, omegas: Optional[Sequence], gauss, workspace, stream=None):
    """Modelled candidate tables from the spectra (jolt_model_tables): returns (D [n_tables, 100]
    float64, C [n_tables, 100] uint64, xnorm2 [n_tables] float64, eps2 [4] float64 for
    b = 0, 2, 4, 8).  `gauss` is a device fp32 tensor [rows, D] of standard normal rows."""
    nt = cfg.n_tables
    if len(xs) != nt or (omegas is not None and len(omegas) != nt):
        raise ValueError("one input (and sketch) per table expected")
    if (gauss.dim() != 2 or gauss.shape[1] != cfg.D or not gauss.is_floating_point() or gauss.element_size() != 4
            or not gauss.is_contiguous()):
        raise ValueError("gauss must be a contiguous float32 [rows, D] tensor")
    _check_inputs(cfg, xs, signs, omegas)
    D = np.zeros((nt, N_CAND), np.float64)
    C = np.zeros((nt, N_CAND), np.uint64)
    xn = np.zeros(nt, np.float64)
    e2 = np.zeros(4, np.float64)
    xa, oa = _ptr_array(xs), _ptr_array(omegas)
    code = load().jolt_model_tables(ctypes.byref(cfg), xa, signs.data_ptr(), oa, gauss.data_ptr(), int(gauss.shape[0]),
                                    D.ctypes.data, C.ctypes.data, xn.ctypes.data, e2.ctypes.data,
                                    workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                    _stream(stream))
    _check(code, "jolt_model_tables")
    return D, C, xn, e2


def allocate(D: np.ndarray, C: np.ndarray, budget: int):
    """(choice int32 [n_tables], lambda, total bytes) by bisection on the byte price."""
    D = np.ascontiguousarray(D, np.float64)
    C = np.ascontiguousarray(C, np.uint64)
    nt, nc = D.shape
    ch = np.zeros(nt, np.int32)
    lam = ctypes.c_double(0.0)
    tot = ctypes.c_uint64(0)
    _check(load().jolt_allocate(D.ctypes.data, C.ctypes.data, nt, nc, int(budget), ch.ctypes.data,
                                ctypes.byref(lam), ctypes.byref(tot)), "jolt_allocate")
    return ch, float(lam.value), int(tot.value)


def refine_swap(D, C, budget: int, choice):
    """jolt_refine_swap: (choice int32 [n_tables], total bytes, moves) after the greedy swap
    from the starting allocation `choice`."""
    D = np.ascontiguousarray(D, np.float64)
    C = np.ascontiguousarray(C, np.uint64)
    nt, nc = D.shape
    ch = np.array(choice, np.int32, copy=True)
    tot = ctypes.c_uint64(0)
    moves = ctypes.c_int32(0)
    _check(load().jolt_refine_swap(D.ctypes.data, C.ctypes.data, nt, nc, int(budget), ch.ctypes.data,
                                   ctypes.byref(tot), ctypes.byref(moves)), "jolt_refine_swap")
    return ch, int(tot.value), int(moves.value)


def allocate_common(D, C, budget: int, allowed=None):
    """jolt_allocate_common: (candidate index, total bytes, total distortion) of the best
    candidate shared by every table among the allowed ones (mask over candidates)."""
    D = np.ascontiguousarray(D, np.float64)
    C = np.ascontiguousarray(C, np.uint64)
    nt, nc = D.shape
    mask = None
    if allowed is not None:
        mask = np.ascontiguousarray(np.asarray(allowed, bool).astype(np.uint8))
        if mask.shape != (nc,):
            raise ValueError("allowed must be a mask over the candidates")
    cand = ctypes.c_int32(0)
    tot = ctypes.c_uint64(0)
    dist = ctypes.c_double(0.0)
    _check(load().jolt_allocate_common(D.ctypes.data, C.ctypes.data, nt, nc, int(budget),
                                       mask.ctypes.data if mask is not None else None, ctypes.byref(cand),
                                       ctypes.byref(tot), ctypes.byref(dist)), "jolt_allocate_common")
    return int(cand.value), int(tot.value), float(dist.value)


def encode(cfg: JoltConfig, xs: Sequence, signs, omegas: Optional[Sequence], choice: np.ndarray, recs: Sequence,
           workspace, stream=None):
    """jolt_encode: records of the chosen candidates, factors recomputed."""
    ch = np.ascontiguousarray(choice, np.int32)
    _check_inputs(cfg, xs, signs, omegas)
    _check_records(cfg, recs, ch)
    code = load().jolt_encode(ctypes.byref(cfg), _ptr_array(xs), signs.data_ptr(), _ptr_array(omegas),
                              ch.ctypes.data, _ptr_array(recs), workspace.data_ptr(),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    _check(code, "jolt_encode")


def encode_built(cfg: JoltConfig, xs: Sequence, signs, choice: np.ndarray, recs: Sequence, workspace,
                 stream=None):
    """jolt_encode_built: the same records from the factors the last build_tables left in
    `workspace` (same cfg, inputs and workspace)."""
    ch = np.ascontiguousarray(choice, np.int32)
    _need_all(xs, _x_bytes(cfg), "xs", cfg.n_tables)
    _check_records(cfg, recs, ch)
    code = load().jolt_encode_built(ctypes.byref(cfg), _ptr_array(xs), signs.data_ptr(), ch.ctypes.data,
                                    _ptr_array(recs), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream(stream))
    _check(code, "jolt_encode_built")


TIMER_SCORE = 0  # kernel id of the fused score pass for the launch timer


def timer_enable(kernel: int, enable: bool):
    """jolt_debug_timer_enable: time every later launch of `kernel` with HIP events."""
    _check(load().jolt_debug_timer_enable(kernel, 1 if enable else 0), "jolt_debug_timer_enable")


def debug_read(cfg: JoltConfig, workspace, which: int, nbytes: int) -> np.ndarray:
    """jolt_debug_read: the first `nbytes` bytes of workspace region `which` (after a build) as uint8."""
    out = np.empty(nbytes, np.uint8)
    _check(load().jolt_debug_read(ctypes.byref(cfg), workspace.data_ptr(), which, out.ctypes.data, nbytes),
           "jolt_debug_read")
    return out


def timer_read(kernel: int):
    """jolt_debug_timer_read: (summed launch milliseconds, launches) since the last read."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int32(0)
    _check(load().jolt_debug_timer_read(kernel, ctypes.byref(ms), ctypes.byref(n)), "jolt_debug_timer_read")
    return float(ms.value), int(n.value)


def _check_records(cfg, recs, ch):
    if ch.shape != (cfg.n_tables,):
        raise ValueError("one candidate per table expected")
    _need_all(recs, lambda k: record_bytes(cfg, int(ch[k])), "records", cfg.n_tables)


def decode(cfg: JoltConfig, recs: Sequence, choice: np.ndarray, xhats: Sequence, stream=None):
    ch = np.ascontiguousarray(choice, np.int32)
    _check_records(cfg, recs, ch)
    _need_all(xhats, _x_bytes(cfg), "xhats", cfg.n_tables)
    code = load().jolt_decode(ctypes.byref(cfg), _ptr_array(recs), ch.ctypes.data, _ptr_array(xhats),
                              _stream(stream))
    _check(code, "jolt_decode")


def attend_workspace_size(cfg: JoltConfig, n_groups: int, nq: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().jolt_attend_workspace_size(ctypes.byref(cfg), int(n_groups), int(nq), ctypes.byref(n)),
           "jolt_attend_workspace_size")
    return int(n.value)


def attend(cfg: JoltConfig, recs_k: Sequence, cands_k, recs_v: Sequence, cands_v, qs: Sequence, outs: Sequence,
           workspace, scale=None, stream=None):
    """jolt_attend over len(recs_k) layer groups: outs[g] (fp32 [N, nq, D]) =
    softmax(scale Q_g K_g^T) V_g with K_g, V_g decoded from the two records inside the attention
    kernel.  qs[g]: bf16 bits as a device int16 tensor [N, nq, D]."""
    ng = len(recs_k)
    nq = int(qs[0].shape[1])
    if scale is None:
        scale = 1.0 / float(cfg.D) ** 0.5
    ck = np.ascontiguousarray(cands_k, np.int32)
    cv = np.ascontiguousarray(cands_v, np.int32)
    if ck.shape != (ng,) or cv.shape != (ng,):
        raise ValueError("one K and one V candidate per group expected")
    _need_all(recs_k, lambda g: record_bytes(cfg, int(ck[g])), "recs_k", ng)
    _need_all(recs_v, lambda g: record_bytes(cfg, int(cv[g])), "recs_v", ng)
    _need_all(qs, 2 * cfg.N * nq * cfg.D, "qs", ng)
    _need_all(outs, 4 * cfg.N * nq * cfg.D, "outs", ng)
    code = load().jolt_attend(ctypes.byref(cfg), ng, _ptr_array(recs_k), ck.ctypes.data, _ptr_array(recs_v),
                              cv.ctypes.data, _ptr_array(qs), nq, ctypes.c_float(scale), _ptr_array(outs),
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(code, "jolt_attend")


# ---------------------------------------------------------------- streaming admission
def stream_state_bytes() -> int:
    n = ctypes.c_size_t(0)
    _check(load().jolt_stream_state_bytes(ctypes.byref(n)), "jolt_stream_state_bytes")
    return int(n.value)


def stream_block_bytes(cfg: JoltConfig, cand: int, t_new: int) -> int:
    n = ctypes.c_uint64(0)
    _check(load().jolt_stream_block_bytes(ctypes.byref(cfg), int(cand), int(t_new), ctypes.byref(n)),
           "jolt_stream_block_bytes")
    return int(n.value)


def stream_workspace_size(cfg: JoltConfig, t_new: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().jolt_stream_workspace_size(ctypes.byref(cfg), int(t_new), ctypes.byref(n)),
           "jolt_stream_workspace_size")
    return int(n.value)


def stream_prepare(cfg: JoltConfig, recs: Sequence, choice, states: Sequence, stream=None):
    """jolt_stream_prepare: freeze every table's record (states[t]: device tensors of
    stream_state_bytes() bytes)."""
    ch = np.ascontiguousarray(choice, np.int32)
    _check_records(cfg, recs, ch)
    _need_all(states, stream_state_bytes(), "states", cfg.n_tables)
    _check(load().jolt_stream_prepare(ctypes.byref(cfg), _ptr_array(recs), ch.ctypes.data, _ptr_array(states),
                                      _stream(stream)), "jolt_stream_prepare")


def stream_encode(cfg: JoltConfig, recs: Sequence, choice, states: Sequence, xnews: Sequence, t_new: int,
                  blocks: Sequence, workspace, dist=None, stream=None):
    """jolt_stream_encode: block records of the incoming blocks xnews[t] (bf16 bits as device
    int16 [N, t_new, D]) against the frozen records; dist (device float64 [n_tables]) receives
    each block's distortion when given."""
    ch = np.ascontiguousarray(choice, np.int32)
    _check_stream(cfg, recs, ch, blocks, t_new)
    _need_all(states, stream_state_bytes(), "states", cfg.n_tables)
    _need_all(xnews, _x_bytes(cfg, t_new), "xnews", cfg.n_tables)
    if dist is not None:
        _need(dist, 8 * cfg.n_tables, "dist")
    code = load().jolt_stream_encode(ctypes.byref(cfg), _ptr_array(recs), ch.ctypes.data, _ptr_array(states),
                                     _ptr_array(xnews), int(t_new), _ptr_array(blocks),
                                     dist.data_ptr() if dist is not None else None, workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(), _stream(stream))
    _check(code, "jolt_stream_encode")


NOALLOC_SCRATCH_BYTES = 32 << 20  # JOLT_NOALLOC_SCRATCH_BYTES


def stream_encode_noalloc(cfg: JoltConfig, recs: Sequence, choice, states: Sequence, xnews: Sequence, t_new: int,
                          blocks: Sequence, dist=None, stream=None):
    """jolt_stream_encode_noalloc: stream_encode with the library's per-device scratch instead
    of a caller workspace (no device allocation; calls overlapping on one device race)."""
    ch = np.ascontiguousarray(choice, np.int32)
    _check_stream(cfg, recs, ch, blocks, t_new)
    _need_all(states, stream_state_bytes(), "states", cfg.n_tables)
    _need_all(xnews, _x_bytes(cfg, t_new), "xnews", cfg.n_tables)
    if dist is not None:
        _need(dist, 8 * cfg.n_tables, "dist")
    code = load().jolt_stream_encode_noalloc(ctypes.byref(cfg), _ptr_array(recs), ch.ctypes.data,
                                             _ptr_array(states), _ptr_array(xnews), int(t_new), _ptr_array(blocks),
                                             dist.data_ptr() if dist is not None else None, _stream(stream))
    _check(code, "jolt_stream_encode_noalloc")


def _check_stream(cfg, recs, ch, blocks, t_new):
    _check_records(cfg, recs, ch)
    _need_all(blocks, lambda k: stream_block_bytes(cfg, int(ch[k]), t_new), "blocks", cfg.n_tables)


def stream_decode(cfg: JoltConfig, recs: Sequence, choice, blocks: Sequence, t_new: int, outs: Sequence, stream=None):
    ch = np.ascontiguousarray(choice, np.int32)
    _check_stream(cfg, recs, ch, blocks, t_new)
    _need_all(outs, _x_bytes(cfg, t_new), "outs", cfg.n_tables)
    _check(load().jolt_stream_decode(ctypes.byref(cfg), _ptr_array(recs), ch.ctypes.data, _ptr_array(blocks),
                                     int(t_new), _ptr_array(outs), _stream(stream)), "jolt_stream_decode")
