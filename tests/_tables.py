"""Seeded input tables of the full-size workloads for the GPU tests, generated in child
processes started when the test session begins (before any test touches the GPU), and the
oracle's stored tables (tests/golden/oracle_tables_*.json, written by
tests/golden/make_oracle_tables.py from the oracle alone)."""
from __future__ import annotations

import json
import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# workloads whose tables the full-size tests need, started at session start
PREGEN = ("mistral_t32k", "llama13b_t2048")

_pool = None
_futs = {}


def _gen(name, t):
    import kvsynth as ks
    w = ks.get_workload(name)
    g, c = w.table_ids()[t]
    return ks.generate_table(w, g, c)


def start(names=PREGEN, workers=8):
    """Queue the generation of every table of `names` in spawned worker processes."""
    global _pool
    if _pool is not None:
        return
    import kvsynth as ks
    workers = max(1, min(workers, len(os.sched_getaffinity(0))))
    _pool = ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"))
    for name in names:
        w = ks.get_workload(name)
        for t in range(w.n_tables):
            _futs[(name, t)] = _pool.submit(_gen, name, t)


def stop():
    global _pool
    if _pool is not None:
        _pool.shutdown(wait=False, cancel_futures=True)
        _pool = None
        _futs.clear()


def table(name, t):
    """bf16 bits [N, T, D] of table t of workload `name` (from the pool when queued)."""
    f = _futs.pop((name, t), None)
    if f is not None:
        return f.result()
    return _gen(name, t)


def golden(name, mode, part=None):
    """The oracle's stored tables of a workload (None when the file is absent)."""
    fn = f"oracle_tables_{name}_{mode}" + (f".part{part:03d}" if part is not None else "") + ".json"
    path = os.path.join(GOLDEN, fn)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        return json.load(f)
