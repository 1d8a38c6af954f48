"""Benchmark of the JoLT candidate-table hot path on one MI355X.

One step = the whole path on one batch of synthetic KV cache: candidate tables of
every (layer group, K/V) tensor (jolt_build_tables), the lambda allocation under
the byte budget (jolt_allocate) and its greedy swap refinement (jolt_refine_swap),
the compressed records from the factors the build computed (jolt_encode_built) and
the decoded cache (jolt_decode).  Inputs are resident in HBM before timing starts.

The default workload is the long-context cache: Mistral-7B shape (32 layers x 8 KV
heads, D = 128) at 32768 tokens, 8 groups of 4 layers, K and V: 16 tables of bf16
[32, 32768, 128] (4.3 GB), randomized token mode, budget 2x.

Prints one JSON line.  `value` = KV bytes (bf16 input) / mean step time.

`--copy-calibration` runs only a device-to-device copy of known size (the reference
kernel for scaling the HBM byte counters of a profiler run) and exits.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# fp32 VALU issue rate with packed fp32 instructions disabled:
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3e12 lane-operations per second
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# VALU lane-operations of the fused score pass per input element, counted from its
# arithmetic: rotation (sign + 7 butterfly stages) once, then for each of the 24
# (r_T, r_d) pairs 11.5 ops (abs-max 0.5, e0 1, e2 2, e4 4, e8 4)
SCORE_OPS_PER_ELEM = 8 + 24 * 11.5
# (r_T, r_d) passes one score launch stands for: every pair except the lossless (T, D);
# one pass reads the table once (2 N T D bytes), which is the algorithmic unit
SCORE_PASSES = 24
SCORE_SRC = os.path.join(ROOT, "partial_tucker_rotated_amd", "csrc", "score.hip")
COPY_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="mistral_t32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tables", type=int, default=1, help="tables the oracle baseline processes")
    ap.add_argument("--cpu-slices", type=int, default=0,
                    help="slices of each sampled table the oracle baseline processes (0: all; "
                         "default 4 at T >= 8192)")
    ap.add_argument("--no-mode-compare", action="store_true",
                    help="skip the exact-vs-randomized build comparison at 1024 tokens")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--token-mode", choices=("exact", "randomized"), default=None,
                    help="override the workload's token-factor mode (exact needs T <= 2048)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the path has no multi-GPU part (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        import torch
        _copy_calibration(torch)
        return
    import kvsynth as ks

    w = ks.get_workload(args.workload)
    ids = w.table_ids()
    xb = _generate(w, ids)  # before the GPU is touched (worker processes)
    import torch
    import partial_tucker_rotated_amd as J
    dev = "cuda"
    xs = [torch.from_numpy(b.view(np.int16)).to(dev) for b in xb]
    signs = torch.from_numpy(np.stack([ks.rotation_signs(w, g, c) for g, c in ids])).to(dev)
    oms = None
    token_mode = args.token_mode or w.token_mode
    mode = J.TOKEN_EXACT if token_mode == "exact" else J.TOKEN_RANDOMIZED
    if mode == J.TOKEN_RANDOMIZED:
        oms = [torch.from_numpy(np.concatenate([ks.sketch_omega(w, g, c, r).reshape(-1) for r in w.rd])
                                .view(np.int16)).to(dev) for g, c in ids]
    cfg = J.default_config(w.N, w.T, w.D, len(ids), mode)
    ws = torch.empty(J.workspace_size(cfg), dtype=torch.uint8, device=dev)
    budget = w.budgets()[0]
    C = J.cost_table(cfg)
    max_rec = int(C.max())
    recs = [torch.empty(max_rec, dtype=torch.uint8, device=dev) for _ in ids]
    xh = [torch.empty_like(x) for x in xs]
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        D, Cc, _ = J.build_tables(cfg, xs, signs, oms, ws)
        if ev:
            ev[1].record(stream)
        ch, lam, tot = J.allocate(D, Cc, budget)
        ch, tot, _ = J.refine_swap(D, Cc, budget, ch)
        J.encode_built(cfg, xs, signs, ch, recs, ws)
        if ev:
            ev[2].record(stream)
        J.decode(cfg, recs, ch, xh)
        if ev:
            ev[3].record(stream)
        return ch, tot, D, Cc

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    J.timer_enable(J.TIMER_SCORE, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ch, tot, Dlast, Clast = step(evs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    J.timer_enable(J.TIMER_SCORE, False)
    score_total_ms, score_launches = J.timer_read(J.TIMER_SCORE)
    ms = (t1 - t0) * 1e3 / args.steps
    build_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    enc_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    dec_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    xbytes = w.x_bytes()
    rec_bytes = int(sum(int(C[c]) for c in ch))

    # dominant kernel: the fused score pass, one launch per build, timed by HIP events the
    # library records around each launch on the stream it is launched on
    score_ms = score_total_ms / max(score_launches, 1)
    score_ops = SCORE_OPS_PER_ELEM * w.N * w.T * w.D * len(ids)
    valu_tops = score_ops / (score_ms * 1e-3) / 1e12
    # algorithmic bytes per launch: 24 (r_T, r_d) passes, each reading every table once
    score_bytes = SCORE_PASSES * xbytes
    achieved = score_bytes / (score_ms * 1e-3) / 1e9
    counters = _score_counters(w.name)
    valu = {"achieved": valu_tops, "peak": VALU_PEAK_TOPS, "unit": "T lane-ops/s", "frac": valu_tops / VALU_PEAK_TOPS,
            "ops_per_element": SCORE_OPS_PER_ELEM,
            "note": "VALU lane-operations counted from the arithmetic (FMA = 1) over the launch time; "
                    "peak = 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (no packed fp32)"}
    if counters.get("valu_insts_per_launch"):
        # SQ_INSTS_VALU counts the MFMA instructions too; they run on the matrix cores
        vector_insts = counters["valu_insts_per_launch"] - counters.get("mfma_insts_per_launch", 0)
        issued = vector_insts * 64 / (score_ms * 1e-3) / 1e12
        valu["counter_issued"] = issued
        valu["counter_frac"] = issued / VALU_PEAK_TOPS
        valu["counter_note"] = ("(SQ_INSTS_VALU - SQ_INSTS_MFMA) x 64 lanes per launch (profiles/) over this run's "
                                "launch time")
    out = {
        "metric": "KV GB/s through 100-candidate JoLT table build; decode GB/s; % HBM peak",
        "value": xbytes / (ms * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "dtype_note": "input and decoded cache bf16; score pass and factor products fp32 (fp16 hi/lo split MFMA, "
                      "fp64 block sums); eigensolver fp64; encoder X~ and residual fp64, rotation and quantizer fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "tables": len(ids), "N": w.N, "T": w.T, "D": w.D,
                   "token_mode": token_mode, "budget_bytes": budget, "kv_bytes": xbytes},
        "build_ms": build_ms,
        "build_gbps": xbytes / (build_ms * 1e-3) / 1e9,
        "encode_ms": enc_ms,
        "decode_ms": dec_ms,
        "decode_gbps": xbytes / (dec_ms * 1e-3) / 1e9,
        "decode_hbm_frac": (xbytes + rec_bytes) / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "decode_record_bytes": rec_bytes,
        "allocated_bytes": int(tot),
        "roofline": {"kernel": "k_score", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": counters.get("traffic_bytes_per_launch"), "launch_ms": score_ms,
                     "launches": score_launches, "algorithmic_bytes_per_launch": score_bytes,
                     "valu": valu,
                     "note": "algorithmic bytes = 24 (r_T, r_d) passes x 2 N T D bytes per table x tables, over "
                             "the launch time (HIP events on the launch stream); the fused kernel reads each "
                             "table once, so traffic (HBM bytes per launch from FETCH_SIZE + WRITE_SIZE) is "
                             "far below it and its bound is the VALU issue rate (valu)"},
    }
    out["allocation"] = _allocation_quality(J, w, Dlast, Clast)
    out["fused_attention"] = _fused_attention(J, torch, w, cfg, ids, xs, signs, ws, ch, stream, args)
    out["streaming"] = _streaming(J, torch, w, cfg, ids, xs, signs, ws, ch, Dlast, stream, args)
    # last: it leaves the workspace without the cores that jolt_encode_built reads
    out["model_tables"] = _model_tables(J, torch, w, cfg, xs, signs, oms, ws, Dlast, Clast, args)
    if not args.no_mode_compare:
        del xs, xh, recs, ws
        torch.cuda.empty_cache()
        out["flash_vs_exact"] = _flash_vs_exact(J, torch, args)
    if not args.no_cpu_baseline:
        slices = args.cpu_slices or (4 if w.T >= 8192 else w.N)
        out["cpu_baseline"] = _cpu_baseline(w, xb, args.cpu_tables, slices)
    print(json.dumps(out), flush=True)


def _fused_attention(J, torch, w, cfg, ids, xs, signs, ws, choice, stream, args):
    """jolt_attend over every layer group (K table 2g, V table 2g + 1) at the last step's
    allocation, nq = 4 queries per KV head (32 query heads over 8 KV heads), timed with HIP
    events on the launch stream, beside jolt_decode of the same records (the unfused path
    still has to run attention over the decoded caches after that)."""
    import kvsynth as ks
    nq = 4
    groups = sorted({g for g, _ in ids})
    recs = [torch.empty(int(J.record_bytes(cfg, int(c))), dtype=torch.uint8, device="cuda") for c in choice]
    J.encode_built(cfg, xs, signs, choice, recs, ws)
    qs = {g: torch.from_numpy(ks.generate_queries(w, g, nq).view(np.int16)).cuda() for g in groups}
    outs = {g: torch.empty((w.N, nq, w.D), dtype=torch.float32, device="cuda") for g in groups}
    aws = torch.empty(J.attend_workspace_size(cfg, len(groups), nq), dtype=torch.uint8, device="cuda")
    pos = {gc: k for k, gc in enumerate(ids)}
    kk = [pos[(g, 0)] for g in groups]
    kv = [pos[(g, 1)] for g in groups]

    def run():
        J.attend(cfg, [recs[i] for i in kk], [int(choice[i]) for i in kk], [recs[i] for i in kv],
                 [int(choice[i]) for i in kv], [qs[g] for g in groups], [outs[g] for g in groups], aws)

    xh = [torch.empty_like(x) for x in xs]
    run()
    J.decode(cfg, recs, choice, xh)
    torch.cuda.synchronize()
    # median over repetitions, each bracketed by HIP events on the launch stream
    reps = max(10, 2 * args.steps)
    ea = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    ed = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for r in range(reps):
        ea[r][0].record(stream)
        run()
        ea[r][1].record(stream)
    for r in range(reps):
        ed[r][0].record(stream)
        J.decode(cfg, recs, choice, xh)
        ed[r][1].record(stream)
    # the unfused path's attention over the decoded bf16 caches: torch batched products with
    # contiguous right operands (scores K Q^T, softmax in fp32, P V)
    qts = {g: qs[g].view(torch.bfloat16).transpose(1, 2).contiguous() for g in groups}

    def torch_attention():
        for g in groups:
            k = xh[pos[(g, 0)]].view(torch.bfloat16)
            v = xh[pos[(g, 1)]].view(torch.bfloat16)
            s = torch.bmm(k, qts[g]).float() * float(1.0 / np.sqrt(w.D))  # [N, T, nq]
            pt = torch.softmax(s, dim=1).to(torch.bfloat16).transpose(1, 2).contiguous()  # [N, nq, T]
            torch.bmm(pt, v)

    torch_attention()
    et = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for r in range(reps):
        et[r][0].record(stream)
        torch_attention()
        et[r][1].record(stream)
    torch.cuda.synchronize()
    att_ms = float(np.median([a.elapsed_time(b) for a, b in ea]))
    dec_ms = float(np.median([a.elapsed_time(b) for a, b in ed]))
    tat_ms = float(np.median([a.elapsed_time(b) for a, b in et]))
    rec_bytes = int(sum(int(r.numel()) for r in recs))
    kv_bytes = w.x_bytes()
    return {"nq": nq, "groups": len(groups), "ms": att_ms, "record_bytes": rec_bytes,
            "record_gbps": rec_bytes / (att_ms * 1e-3) / 1e9, "kv_equiv_gbps": kv_bytes / (att_ms * 1e-3) / 1e9,
            "hbm_frac": (rec_bytes + 2 * w.N * nq * w.D * len(groups) * 3) / (att_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "decode_only_ms": dec_ms, "unfused_attention_ms": tat_ms, "unfused_total_ms": dec_ms + tat_ms,
            "note": "kv_equiv_gbps = bf16 K+V bytes attended per second; decode_only_ms = jolt_decode of "
                    "the same records; unfused_attention_ms = torch batched-product attention over the "
                    "decoded bf16 caches; unfused_total_ms = the two, the path the fused kernel replaces"}


def _streaming(J, torch, w, cfg, ids, xs, signs, ws, choice, Dmeas, stream, args):
    """Admission of a further 256-token block per table against the records frozen at the
    step's allocation (jolt_stream_prepare once, then jolt_stream_encode per block), timed
    with HIP events on the launch stream over repeated encodes of the same blocks; the
    blocks are new tokens of the same generative model (kvsynth.generate_block)."""
    import kvsynth as ks
    tn = 256
    recs = [torch.empty(int(J.record_bytes(cfg, int(c))), dtype=torch.uint8, device="cuda") for c in choice]
    J.encode_built(cfg, xs, signs, choice, recs, ws)
    states = [torch.empty(J.stream_state_bytes(), dtype=torch.uint8, device="cuda") for _ in ids]
    blocks = [torch.empty(J.stream_block_bytes(cfg, int(c), tn), dtype=torch.uint8, device="cuda") for c in choice]
    xn = [torch.from_numpy(ks.generate_block(w, g, c, tn).view(np.int16)).cuda() for g, c in ids]
    sws = torch.empty(J.stream_workspace_size(cfg, tn), dtype=torch.uint8, device="cuda")
    dist = torch.empty(len(ids), dtype=torch.float64, device="cuda")
    outs = [torch.empty_like(x) for x in xn]
    e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    J.stream_prepare(cfg, recs, choice, states)  # first launch of each kernel outside the timing
    J.stream_encode(cfg, recs, choice, states, xn, tn, blocks, sws, dist=dist)
    J.stream_decode(cfg, recs, choice, blocks, tn, outs)
    torch.cuda.synchronize()
    reps = max(10, 4 * args.steps)
    e[0].record(stream)
    J.stream_prepare(cfg, recs, choice, states)
    e[1].record(stream)
    for _ in range(reps):
        J.stream_encode(cfg, recs, choice, states, xn, tn, blocks, sws, dist=dist)
    e[2].record(stream)
    for _ in range(reps):
        J.stream_decode(cfg, recs, choice, blocks, tn, outs)
    e[3].record(stream)
    torch.cuda.synchronize()
    prep_ms = e[0].elapsed_time(e[1])
    enc_ms = e[1].elapsed_time(e[2]) / reps
    dec_ms = e[2].elapsed_time(e[3]) / reps
    d = dist.cpu().numpy()
    xbytes = 2 * w.N * tn * w.D * len(ids)
    bbytes = int(sum(int(b.numel()) for b in blocks))
    rows = np.arange(len(ids))
    return {"t_new": tn, "tables": len(ids), "prepare_ms": prep_ms, "encode_ms": enc_ms, "decode_ms": dec_ms,
            "kv_gbps": xbytes / (enc_ms * 1e-3) / 1e9,
            "encode_hbm_frac": (xbytes + bbytes) / (enc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "block_bytes": bbytes, "bf16_bytes": xbytes, "block_dist_sum": float(d.sum()),
            "block_dist_max": float(d.max()), "frozen_dist_sum": float(Dmeas[rows, choice].sum()),
            "note": "encode_ms per 256-token block of every table (fold-in, residual codes, distortion); "
                    "block_dist_sum = sum over tables of the new block's distortion, frozen_dist_sum = the "
                    "same at the frozen tokens"}


def _model_tables(J, torch, w, cfg, xs, signs, oms, ws, Dmeas, Cmeas, args):
    """jolt_model_tables (the separable model eps^2(b) tau from the spectra: no cores,
    reconstruction or residual pass) on the same tables, wall-clock per call (it synchronises
    to hand its table to the host), and what allocating from the model costs: the measured
    distortion at the model's allocation (price search + swap) against the measured-table
    allocation, at each budget."""
    import kvsynth as ks
    G = torch.from_numpy(ks.gaussian_rows(w.D, 4096)).cuda()
    Dm, Cm, _, eps2 = J.model_tables(cfg, xs, signs, oms, G, ws)
    torch.cuda.synchronize()
    reps = max(3, args.steps)
    t0 = time.perf_counter()
    for _ in range(reps):
        Dm, Cm, _, eps2 = J.model_tables(cfg, xs, signs, oms, G, ws)
    ms = (time.perf_counter() - t0) * 1e3 / reps
    rows = np.arange(Dmeas.shape[0])
    per_budget = []
    for B in w.budgets():
        ch, _, _ = J.allocate(Dm, Cm, B)
        ch, tot, _ = J.refine_swap(Dm, Cm, B, ch)
        chm, _, _ = J.allocate(Dmeas, Cmeas, B)
        chm, _, _ = J.refine_swap(Dmeas, Cmeas, B, chm)
        per_budget.append({"budget_bytes": int(B), "model_alloc_measured": float(Dmeas[rows, ch].sum()),
                           "measured_alloc": float(Dmeas[rows, chm].sum()), "model_alloc_bytes": int(tot),
                           "same_choice_tables": int(np.sum(ch == chm))})
    return {"ms": ms, "kv_gbps": w.x_bytes() / (ms * 1e-3) / 1e9,
            "eps2": {str(b): float(e) for b, e in zip((0, 2, 4, 8), eps2)}, "budgets": per_budget,
            "note": "wall-clock per jolt_model_tables call incl. the host copy of the spectra; "
                    "model_alloc_measured = measured D summed at the allocation made from the model"}


def _allocation_quality(J, w, D, C):
    """Sum of normalised distortion over the tables of the last step at each budget of the
    workload: the price search alone, with the greedy swap, and the shared-candidate
    baselines (best shared candidate; shared candidate with b fixed at 4; pure Tucker, b = 0),
    plus the host time of the price search + swap."""
    cands = [(a, c, b) for a in w.rT for c in w.rd for b in w.bits]
    res = {"unit": "sum over tables of D(z)", "budgets": []}
    for B in w.budgets():
        t0 = time.perf_counter()
        ch0, _, tot0 = J.allocate(D, C, B)
        ch, tot, moves = J.refine_swap(D, C, B, ch0)
        host_ms = (time.perf_counter() - t0) * 1e3
        rows = np.arange(D.shape[0])
        entry = {"budget_bytes": int(B), "joint": float(D[rows, ch0].sum()), "joint_bytes": int(tot0),
                 "joint_swap": float(D[rows, ch].sum()), "joint_swap_bytes": int(tot), "swap_moves": moves,
                 "host_ms": host_ms}
        for name, mask in (("common_best", None), ("common_b4", [c[2] == 4 for c in cands]),
                           ("common_b0", [c[2] == 0 for c in cands])):
            try:
                i, ctot, dist = J.allocate_common(D, C, B, mask)
                entry[name] = dist
                entry[name + "_z"] = list(cands[i])
            except J.JoltError:
                entry[name] = None
        res["budgets"].append(entry)
    return res


def _gen_one(name, g, c):
    import kvsynth as ks
    return ks.generate_table(ks.get_workload(name), g, c)


def _generate(w, ids):
    """Seeded bf16 tables of the workload; large workloads in a spawned process pool, with
    a progress line per table on stderr."""
    import kvsynth as ks
    if w.x_bytes() < (256 << 20):
        return [ks.generate_table(w, g, c) for g, c in ids]
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    workers = max(1, min(8, len(os.sched_getaffinity(0)), len(ids)))
    out = [None] * len(ids)
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
        futs = {ex.submit(_gen_one, w.name, g, c): k for k, (g, c) in enumerate(ids)}
        for done, f in enumerate(__import__("concurrent.futures").futures.as_completed(futs), 1):
            out[futs[f]] = f.result()
            print(f"generated table {done}/{len(ids)} of {w.name}", file=sys.stderr, flush=True)
    return out


def _copy_calibration(torch):
    """A plain device-to-device copy of COPY_BYTES, three times."""
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}), flush=True)


def _source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _score_counters(workload):
    """Per-launch counter figures of the score kernel from the committed summary of this
    workload (profiles/k_score_<workload>_counters.txt): HBM bytes (FETCH_SIZE + WRITE_SIZE,
    copy-calibrated) and issued VALU / MFMA instructions.  Empty when there is no summary or
    the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"k_score_{workload}_counters.txt")
    if not os.path.exists(path):
        return {}
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != _source_hash(SCORE_SRC):
        return {}
    out = {}
    for k in ("traffic_bytes_per_launch", "valu_insts_per_launch", "mfma_insts_per_launch"):
        try:
            out[k] = float(vals[k])
        except (KeyError, ValueError):
            pass
    return out


def _flash_vs_exact(J, torch, args):
    """Build time of the 16 Mistral-shaped tables at 1024 tokens ([32, 1024, 128]) with the
    exact token mode (subspace iteration to the Ritz-residual tolerance) and with the
    randomized range finder (FlashJoLT), median of repeated builds bracketed by HIP events on
    the launch stream; the tables of both are the same bytes."""
    import kvsynth as ks
    w = ks.get_workload("mistral_t1024_flash")
    ids = w.table_ids()
    xs = [torch.from_numpy(ks.generate_table(w, g, c).view(np.int16)).cuda() for g, c in ids]
    signs = torch.from_numpy(np.stack([ks.rotation_signs(w, g, c) for g, c in ids])).cuda()
    oms = [torch.from_numpy(np.concatenate([ks.sketch_omega(w, g, c, r).reshape(-1) for r in w.rd])
                            .view(np.int16)).cuda() for g, c in ids]
    stream = torch.cuda.current_stream()
    res = {"workload": "16 tables of bf16 [32, 1024, 128] (mistral_t1024_flash inputs)"}
    for name, mode, om in (("exact", J.TOKEN_EXACT, None), ("randomized", J.TOKEN_RANDOMIZED, oms)):
        cfg = J.default_config(w.N, w.T, w.D, len(ids), mode)
        ws = torch.empty(J.workspace_size(cfg), dtype=torch.uint8, device="cuda")
        J.build_tables(cfg, xs, signs, om, ws)
        reps = max(3, args.steps)
        t = []
        for _ in range(reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            J.build_tables(cfg, xs, signs, om, ws)
            e[1].record(stream)
            torch.cuda.synchronize()
            t.append(e[0].elapsed_time(e[1]))
        res[name + "_build_ms"] = float(np.median(t))
        if mode == J.TOKEN_EXACT:
            res["exact_iterations"] = J.last_build_info(ws)["iterations"]
        del ws
        torch.cuda.empty_cache()
    res["exact_over_randomized"] = res["exact_build_ms"] / res["randomized_build_ms"]
    return res


def _cpu_baseline(w, xb, ntab, nslices):
    """The oracle (fp64 NumPy, untuned) on a bounded sample: the first `ntab` tables, each
    cut to its first `nslices` slices (all T tokens, so the token-mode problem keeps its
    length), in the workload's token mode.  cores = BLAS threads of the oracle's NumPy
    (threadpoolctl, read after the run, once the library is loaded); the sample string also
    gives the process CPU time over wall time, the parallelism the run actually reached."""
    import resource
    import kvsynth as ks
    from oracle import jolt_oracle as O
    ids = w.table_ids()[:ntab]
    ns = min(nslices, w.N)
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    for k, (g, c) in enumerate(ids):
        X = O.bf16_bits_to_f64(xb[k][:ns])
        om = None
        if w.token_mode == "randomized":
            om = {r: ks.sketch_omega(w, g, c, r)[: ns * r] for r in w.rd}
        O.build_table(X, ks.rotation_signs(w, g, c), w.rT, w.rd, w.bits, w.quant_block, w.token_mode,
                      omegas=om)
    dt = time.perf_counter() - t0
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max(blas) if blas else 1
    except Exception:  # threadpoolctl missing: the process's CPU affinity
        cores = len(os.sched_getaffinity(0))
    nbytes = 2 * ns * w.T * w.D * len(ids)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"100-candidate table build of {len(ids)} of {w.n_tables} tables cut to {ns} of {w.N} "
                      f"slices (bf16 [{ns}, {w.T}, {w.D}], {nbytes} KV bytes, {w.token_mode} token mode), "
                      f"{dt:.1f} s wall, {cpu / dt:.1f} cores busy on average"}


if __name__ == "__main__":
    main()
