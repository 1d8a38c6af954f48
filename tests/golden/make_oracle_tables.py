"""Write the oracle's candidate tables and allocations of the seeded workloads to
tests/golden/oracle_tables_<workload>.json, for the full-size GPU parity tests.

Calls only the oracle (oracle/jolt_oracle.py) and the seeded input generator (kvsynth):
for every table of the workload it stores the SHA-256 of the bf16 input bytes, the
oracle's D(z) and C(z) over the 100 candidates and ||X||^2; for every budget of the
workload, the oracle's allocation (choice, price, total bytes, Lagrangian margin per
table).  Floats are written with repr(), which round-trips exactly.

    python tests/golden/make_oracle_tables.py --workload mistral_t512 [--token-mode exact]
        [--jobs 4] [--tables 0,1,2]

A run with --tables writes only those tables (no allocation) to a partial file, so a
long workload can be computed in pieces and joined with --join.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)


def _one(name, mode, t):
    import numpy as np
    import kvsynth as ks
    from oracle import jolt_oracle as O
    w = ks.get_workload(name)
    g, c = w.table_ids()[t]
    t0 = time.time()
    xb = ks.generate_table(w, g, c)
    sha = hashlib.sha256(np.ascontiguousarray(xb).tobytes()).hexdigest()
    X = O.bf16_bits_to_f64(xb)
    del xb
    om = {r: ks.sketch_omega(w, g, c, r) for r in w.rd} if mode == "randomized" else None
    res = O.build_table(X, ks.rotation_signs(w, g, c), w.rT, w.rd, w.bits, w.quant_block, mode,
                        omegas=om, power_iters=w.power_iters)
    return {"table": t, "g": g, "c": c, "sha256": sha, "xnorm2": repr(res.xnorm2),
            "D": [repr(float(v)) for v in res.D], "C": [int(v) for v in res.C],
            "seconds": round(time.time() - t0, 1)}


def _path(name, mode, suffix=""):
    return os.path.join(HERE, f"oracle_tables_{name}_{mode}{suffix}.json")


def _allocations(w, tables):
    import numpy as np
    from oracle import jolt_oracle as O
    Dt = np.array([[float(v) for v in t["D"]] for t in tables])
    Ct = np.array([t["C"] for t in tables], dtype=np.uint64)
    out = []
    for B in w.budgets():
        a = O.allocate(Dt, Ct, B)
        out.append({"budget": int(B), "choice": [int(v) for v in a.choice], "lam": repr(a.lam),
                    "total": int(a.total), "margin": [repr(float(m)) for m in a.margin]})
    return out


def main():
    import kvsynth as ks
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--token-mode", choices=("exact", "randomized"), default=None)
    ap.add_argument("--jobs", type=int, default=1)
    ap.add_argument("--tables", default=None, help="comma-separated table indices (partial file)")
    ap.add_argument("--join", action="store_true", help="join the partial files into the full one")
    args = ap.parse_args()
    w = ks.get_workload(args.workload)
    mode = args.token_mode or w.token_mode
    if args.join:
        tables = {}
        for f in sorted(os.listdir(HERE)):
            if f.startswith(f"oracle_tables_{w.name}_{mode}.part"):
                for t in json.load(open(os.path.join(HERE, f)))["tables"]:
                    tables[t["table"]] = t
        assert sorted(tables) == list(range(w.n_tables)), sorted(tables)
        tabs = [tables[i] for i in range(w.n_tables)]
    else:
        idx = list(range(w.n_tables)) if args.tables is None else [int(v) for v in args.tables.split(",")]
        if args.jobs > 1:
            import multiprocessing as mp
            from concurrent.futures import ProcessPoolExecutor
            with ProcessPoolExecutor(args.jobs, mp_context=mp.get_context("spawn")) as ex:
                tabs = list(ex.map(_one, [w.name] * len(idx), [mode] * len(idx), idx))
        else:
            tabs = [_one(w.name, mode, t) for t in idx]
        for t in tabs:
            print(f"{w.name} table {t['table']}: {t['seconds']} s", flush=True)
        if args.tables is not None:
            path = _path(w.name, mode, f".part{idx[0]:03d}")
            json.dump({"workload": w.name, "token_mode": mode, "tables": tabs}, open(path, "w"), indent=0)
            print("wrote", path)
            return
    out = {"workload": w.name, "token_mode": mode, "N": w.N, "T": w.T, "D": w.D,
           "power_iters": w.power_iters if mode == "randomized" else None,
           "generator": "kvsynth.generate_table; oracle.jolt_oracle.build_table and allocate",
           "tables": tabs, "allocations": _allocations(w, tabs)}
    path = _path(w.name, mode)
    json.dump(out, open(path, "w"), indent=0)
    print("wrote", path)


if __name__ == "__main__":
    main()
