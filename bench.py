#!/usr/bin/env python3
"""Benchmark of the FlashLoop loop step on one MI355X.

One step = every loop of one workload, in order: the full early loops (commit
the base or a dense delta layer, full causal attention with column mass) and
the lazy loops (token selection, key selection, delta commit of the
active tokens, mass-corrected attention), i.e. every step of the hot path
over one batch of synthetic input already resident in HBM.  Deltas are
stored as 4-bit codes with one binary16 scale per 32 elements unless
--delta-bits / --group ask for 2-bit codes or 64-element groups.

Metric: active-token loop-steps per second = (sum over the step's loops of the
rows that loop computes: N in a full loop, n_active in a lazy loop) / step
time, over K steps without instrumentation.  The JSON line also carries the
lazy-loop rate, KV bytes per second, the roofline position of the dominant
kernel (from hipEvent pairs around every launch, over a second run of the
same K steps) and the CPU oracle timed on the host.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_VECTOR_PEAK_TFLOPS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="single_layer",
                    help="tiny | single_layer | long_prefill | decode | deep")
    ap.add_argument("--cpu-baseline", type=int, default=1, help="0 skips the host oracle timing")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--delta-bits", type=int, default=4, choices=(2, 4),
                    help="bits per stored delta element of the lazy loops' KV versions")
    ap.add_argument("--group", type=int, default=32, choices=(32, 64),
                    help="delta elements sharing one binary16 scale (must divide head_dim)")
    ap.add_argument("--exit-threshold", type=float, default=None,
                    help="instead of the benchmark line: step time with early exit at this threshold against "
                         "the full loop count, and the loops each sequence ran")
    ap.add_argument("--quality", action="store_true",
                    help="instead of timing: error of every lazy loop against the dense loop, for the output "
                         "formulas and key policies")
    return ap.parse_args()


# --------------------------------------------------------------------------- work model
def _pairs(rows, keys_sorted):
    """sum over rows i of |{j in keys : j <= i}| for ascending key lists."""
    import numpy as np
    return int(np.searchsorted(keys_sorted, rows, side="right").sum())


def work_model(wl, run):
    """Algorithmic flops / bytes of one step, per kernel family: 4d flops per visible
    (row, key) pair in full loops and 8d in lazy ones (6d for the mixture formula),
    2d (4d lazy) for the column mass, and the bytes each HBM-bound kernel must move."""
    import numpy as np
    H, d, N = wl.n_heads, wl.head_dim, wl.n_tokens
    es = 2 if wl.dtype == "bf16" else 4
    rec = d * wl.delta_bits // 8 + 2 * (d // wl.group)   # bytes of one delta record (one head row)
    w = {"attn_full_flops": 0, "attn_lazy_flops": 0, "colmass_full_flops": 0, "colmass_lazy_flops": 0,
         "select_bytes": 0, "commit_bytes": 0, "kv_bytes": 0, "lazy_rows": 0, "rows": 0}
    if wl.decode:
        S = wl.n_seq
        w["decode_full_bytes"] = w["decode_lazy_bytes"] = 0
        for l in range(1, wl.n_loops + 1):
            w["rows"] += S
            if l == 1:
                p = S * H * N
                w["attn_full_flops"] += 4 * d * p
                w["decode_full_bytes"] += S * H * N * d * es * 2
            else:
                keys = run.keys.cpu().numpy()
                p = S * H * wl.n_keys
                w["attn_lazy_flops"] += 8 * d * p
                w["lazy_rows"] += S
                # chain reads of the selected keys: base + one record per present layer, K and V
                layers_present = 0
                for s in range(S):
                    for lp in range(2, l + 1):
                        present = set(run.ctx[lp][s].cpu().numpy().tolist()) | {N - 1}
                        layers_present += sum(int(j in present) for j in keys[s, 0])
                w["decode_lazy_bytes"] += 2 * H * (S * wl.n_keys * d * es + layers_present * rec)
        w["kv_bytes"] = w["decode_full_bytes"] + w["decode_lazy_bytes"]
        return w
    for l in range(1, wl.n_loops + 1):
        if l <= wl.n_full:
            p = H * N * (N + 1) // 2
            w["rows"] += N
            w["attn_full_flops"] += 4 * d * p
            w["colmass_full_flops"] += 2 * d * p
            w["commit_bytes"] += 2 * H * N * (d * es + (d * es + (l - 1) * rec if l > 1 else d * es))
        else:
            act = run.act[l].cpu().numpy()
            keys = run.keys_l[l].cpu().numpy()
            na = act.size
            w["rows"] += na
            w["lazy_rows"] += na
            p = sum(_pairs(act, keys[h]) for h in range(H))
            w["attn_lazy_flops"] += 8 * d * p
            w["colmass_lazy_flops"] += 4 * d * p
            cand = N if l == wl.n_full + 1 else wl.n_active(l - 1)
            w["select_bytes"] += cand * H * d * es * 2 + N * 8 + N * 8 + H * N * 4 + H * wl.n_keys * 4
            chain = 2 * H * na * (d * es + (l - 2) * rec)        # upper bound: every earlier layer present
            w["commit_bytes"] += 2 * H * na * d * es + chain + 2 * H * na * rec
            w["kv_bytes"] += chain + 2 * H * na * rec
    return w


KERNEL_WORK = {
    # kernel name -> (work key, unit, bound)
    "rows_attend_full": ("attn_full_flops", "TFLOP/s", "alu"),
    "rows_attend_lazy": ("attn_lazy_flops", "TFLOP/s", "alu"),
    "rows_attend_commit_lazy": ("attn_lazy_flops", "TFLOP/s", "alu"),
    "rows_colmass": ("colmass_full_flops", "TFLOP/s", "alu"),
    "mfma_fwd_full": ("attn_full_flops", "TFLOP/s", "mfma"),
    "mfma_fwd_lazy": ("attn_lazy_flops", "TFLOP/s", "mfma"),
    "mfma_colmass_full": ("colmass_full_flops", "TFLOP/s", "mfma"),
    "mfma_colmass_lazy": ("colmass_lazy_flops", "TFLOP/s", "mfma"),
    "delta_norm": ("select_bytes", "GB/s", "hbm"),
    "commit_delta": ("commit_bytes", "GB/s", "hbm"),
}
# the decode workload's per-row kernels stream the stored context: HBM-bound
KERNEL_WORK_DECODE = dict(KERNEL_WORK, **{
    "rows_attend_full": ("decode_full_bytes", "GB/s", "hbm"),
    "rows_attend_commit_lazy": ("decode_lazy_bytes", "GB/s", "hbm"),
    "rows_attend_lazy": ("decode_lazy_bytes", "GB/s", "hbm"),
})


def measured_traffic(timer, workload):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary of
    this kernel and workload; null when there is none or the library sources
    changed since the counters were taken."""
    from sparse_loop_attention_amd import profiling
    now = profiling.source_hash()
    for rec in profiling.load_traffic_records(os.path.join(ROOT, "profiles")):
        if rec["timer"] == timer and rec["workload"] == workload:
            if rec["source_hash"] != now:
                return {"traffic": None, "traffic_note": f"{rec['file']} is stale (sources changed)"}
            return {"traffic": rec["traffic_bytes"], "traffic_unit": "bytes per launch",
                    "traffic_source": rec["file"]}
    return {}


def roofline(timings, work, steps, decode=False, workload="", kernel=None):
    """Roofline of `kernel`, or of the kernel with the largest share of the step."""
    table = KERNEL_WORK_DECODE if decode else KERNEL_WORK
    if kernel is None:
        name, (ms, launches) = max(timings.items(), key=lambda kv: kv[1][0])
    elif kernel in timings:
        name, (ms, launches) = kernel, timings[kernel]
    else:
        return None
    avg_ms = ms / max(launches, 1)
    entry = {"kernel": name, "launches_per_step": launches / steps, "avg_launch_ms": avg_ms}
    if name in table:
        key, unit, bound = table[name]
        per_step = work[key]
        secs = ms / 1e3 / steps
        if unit == "GB/s":
            achieved = per_step / secs / 1e9
            peak = HBM_PEAK_GBPS
        else:
            achieved = per_step / secs / 1e12
            peak = MFMA_BF16_PEAK_TFLOPS if bound == "mfma" else FP32_VECTOR_PEAK_TFLOPS
        entry.update({"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                      "frac": achieved / peak, "traffic": None})
        entry.update(measured_traffic(name, workload))
    else:
        entry.update({"bound": None, "achieved": None, "peak": None, "unit": None, "frac": None, "traffic": None})
    return entry


# --------------------------------------------------------------------------- CPU oracle
def cpu_baseline(wl, target_s):
    """The oracle, as it stands, on a bounded sample of the same workload.

    Decode: the T loops of one sequence over its built context (the context
    build is outside the timed work, as on the GPU).  Prefill: whole steps;
    when one step of all heads would take well over the target, whole steps
    of the same workload with fewer heads (same N, schedule and key count),
    scaled by the head fraction (every part of a step is per head or
    proportional to the hidden width).
    """
    import copy
    from threadpoolctl import threadpool_info
    import oracle
    from sparse_loop_attention_amd import configs
    from sparse_loop_attention_amd.synth import SyntheticLoops
    cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    if wl.decode:
        syn = SyntheticLoops(wl, seqs=(0,))
        data = {l: {k: v.copy() for k, v in x.items()} for l, x in syn}
        ctx = {l: syn.context_active_sets(l)[0] for l in range(2, wl.n_loops + 1)}
        store = oracle.build_decode_context(wl, 0, ctx, data)
        n, busy = 0, 0.0
        while busy < target_s:
            st = copy.deepcopy(store)
            t0 = time.perf_counter()
            oracle.run_decode_loops(wl, st, 0, data)
            busy += time.perf_counter() - t0
            n += 1
            print(f"[bench] oracle decode run {n}: {busy:.1f} s", file=sys.stderr, flush=True)
        return {"value": n * wl.n_loops / busy, "unit": "active-token loop-steps/s", "cores": cores,
                "kind": "oracle",
                "sample": f"{n} run(s) of the {wl.n_loops} decode loops of 1 of {wl.n_seq} sequences "
                          f"over its built context, {busy:.1f} s"}

    def steps_of(w, budget):
        data = [(l, {k: v.copy() for k, v in x.items()}) for l, x in SyntheticLoops(w)]
        n, busy = 0, 0.0
        while True:
            t0 = time.perf_counter()
            oracle.run_prefill(w, iter(data))
            busy += time.perf_counter() - t0
            n += 1
            print(f"[bench] oracle step {n} ({w.n_heads} heads): {busy:.1f} s", file=sys.stderr, flush=True)
            if busy >= budget:
                return n, busy

    H = wl.n_heads
    rows_per_step = sum(wl.n_active(l) for l in range(1, wl.n_loops + 1))
    probe = configs.scaled(wl, wl.n_tokens, n_heads=1)
    n1, t1 = steps_of(probe, 0.0)
    hs = H if t1 * H <= 1.5 * target_s else max(1, min(H, int(target_s // t1)))
    if hs == 1 and t1 >= 0.5 * target_s:
        n, dt = n1, t1
    else:
        n, dt = steps_of(wl if hs == H else configs.scaled(wl, wl.n_tokens, n_heads=hs), target_s)
    what = "all heads" if hs == H else f"{hs} of its {H} heads, scaled by {hs}/{H}"
    return {"value": n * rows_per_step / dt * hs / H, "unit": "active-token loop-steps/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{n} whole step(s) of the workload ({wl.n_loops} loops, N = {wl.n_tokens}) with {what}, "
                      f"{dt:.1f} s"}


# --------------------------------------------------------------------------- quality
def quality(wl):
    """Lazy loops against the dense loop they stand in for.

    After each lazy loop l the dense reference is full causal attention of
    every row (the effective queries) over the store's version l, computed by
    the library's full mode; the error is ||o - o_dense|| / ||o_dense|| over
    all rows and over the loop's active rows, for each output formula and key
    policy.
    """
    import torch
    from sparse_loop_attention_amd import abi, driver
    from sparse_loop_attention_amd.synth import SyntheticLoops
    inputs = driver.upload_loops(wl, SyntheticLoops(wl), "cuda")
    n, H, d = wl.n_tokens, wl.n_heads, wl.head_dim
    o_ref = torch.empty(n, H, d, dtype=torch.float32, device="cuda")
    lse_ref = torch.empty(n, H, dtype=torch.float32, device="cuda")
    c_ref = torch.empty(H, n, dtype=torch.float32, device="cuda")
    out = {}
    for formula in ("column", "mixture"):
        for freeze in (False, True):
            run = driver.PrefillRun(wl, inputs, "cuda", formula=formula, freeze_keys=freeze)
            rows = []
            q_eff = None                   # every row's query as of its last active loop
            for l in range(1, wl.n_loops + 1):
                if l <= wl.n_full:
                    run.full_loop(l)
                    cand = None
                    q_eff = inputs[l]["q"][0].clone()
                    continue
                act = run.lazy_loop(l, cand)
                cand = act
                q_eff.index_copy_(0, act.long(), inputs[l]["q"][0].index_select(0, act.long()))
                abi.attend(abi.attend_args(run.kv, abi.FL_ATTEND_FULL, l, q_eff, None, None, n, None,
                                           o_ref, lse_ref, c_ref, run.workspace))
                torch.cuda.synchronize()
                diff = (run.o - o_ref).double()
                ref = o_ref.double()
                idx = act.long()
                rows.append({"loop": l,
                             "rel_err_all": float(diff.norm() / ref.norm()),
                             "rel_err_active": float(diff[idx].norm() / ref[idx].norm())})
            out[f"{formula}{'+frozen' if freeze else ''}"] = rows
            print(f"[bench] quality {formula} frozen={freeze} done", file=sys.stderr, flush=True)
    return out


# --------------------------------------------------------------------------- early exit
def exit_report(wl, tau, steps, warmup):
    """Step time with early exit at threshold tau against the same step without
    it, and the number of loops each sequence ran."""
    import torch
    from sparse_loop_attention_amd import driver
    from sparse_loop_attention_amd.synth import SyntheticLoops
    syn = SyntheticLoops(wl)
    inputs = driver.upload_loops(wl, syn, "cuda")
    ctx = {l: syn.context_active_sets(l) for l in range(2, wl.n_loops + 1)} if wl.decode else None

    def make(thr):
        if wl.decode:
            r = driver.DecodeRun(wl, inputs, ctx, "cuda", exit_threshold=thr)
            r.build_context()
            return r
        return driver.PrefillRun(wl, inputs, "cuda", exit_threshold=thr)

    out = {"workload": wl.name, "threshold": tau, "loops": wl.n_loops, "data": "synthetic"}
    for name, thr in (("no_exit", None), ("exit", tau)):
        run = make(thr)
        for _ in range(warmup):
            run.run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            run.run()
        torch.cuda.synchronize()
        out[f"ms_per_step_{name}"] = (time.perf_counter() - t0) / steps * 1e3
        if thr is not None:
            recs = run.run(record=True)
            torch.cuda.synchronize()
            flags = torch.stack([r.exited for r in recs]).cpu().numpy()      # [loop, seq]
            out["loops_run_per_sequence"] = [int((flags[:, s] == 0).sum()) for s in range(flags.shape[1])]
        print(f"[bench] exit report: {name} done", file=sys.stderr, flush=True)
    return out


# --------------------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1 "
                                   "(the multi-GPU sharding is a design note, not code)"}))
        sys.exit(2)
    import numpy as np
    import torch
    from sparse_loop_attention_amd import abi, configs, driver
    from sparse_loop_attention_amd.synth import SyntheticLoops

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    abi.lib()
    wl = configs.WORKLOADS[args.workload]
    if wl.head_dim % args.group:
        raise SystemExit(f"--group {args.group} does not divide head_dim {wl.head_dim}")
    import dataclasses
    wl = dataclasses.replace(wl, delta_bits=args.delta_bits, group=args.group)
    if args.exit_threshold is not None:
        print(json.dumps(exit_report(wl, args.exit_threshold, args.steps, args.warmup)), flush=True)
        return
    if args.quality:
        if wl.decode:
            raise SystemExit("--quality covers the prefill workloads")
        print(json.dumps({"workload": wl.name, "delta_bits": wl.delta_bits, "group": wl.group,
                          "metric": "relative L2 error of o against the dense loop",
                          "data": "synthetic", "variants": quality(wl)}), flush=True)
        return
    # traffic records name the workload, and the store format when it is not the default
    label = wl.name if (wl.delta_bits, wl.group) == (4, 32) else f"{wl.name}-{wl.delta_bits}b{wl.group}"
    print(f"[bench] workload {label}: generating inputs", file=sys.stderr, flush=True)
    syn = SyntheticLoops(wl)
    if wl.decode:
        ctx_sets = {l: syn.context_active_sets(l) for l in range(2, wl.n_loops + 1)}
        inputs = driver.upload_loops(wl, syn, "cuda")
        run = driver.DecodeRun(wl, inputs, ctx_sets, "cuda")
        run.build_context()
    else:
        inputs = driver.upload_loops(wl, syn, "cuda")
        run = driver.PrefillRun(wl, inputs, "cuda")
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        run.run()
    torch.cuda.synchronize()
    # timed region: K steps as a caller runs them (no instrumentation)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run.run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    # kernel durations: the same K steps again with a hipEvent pair around every
    # launch, on the launch stream (the events add queue gaps between kernels,
    # not kernel time, so the step time above is taken without them)
    print(f"[bench] per-kernel hipEvent timing over {args.steps} steps", file=sys.stderr, flush=True)
    abi.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run.run()
    torch.cuda.synchronize()
    ms_instrumented = (time.perf_counter() - t0) / args.steps * 1e3
    timings = abi.timing_read()
    abi.timing_enable(False)
    work = work_model(wl, run)
    value = work["rows"] * args.steps / elapsed
    lazy_ms = sum(ms for name, (ms, _) in timings.items()
                  if name.endswith("_lazy") or name in ("delta_norm", "topk", "commit_delta", "slot_map",
                                                        "rows_colmass", "colmass_reduce")) / args.steps
    lazy_kernel = next((k for k in ("mfma_fwd_lazy", "rows_attend_commit_lazy", "rows_attend_lazy") if k in timings),
                       None)
    out = {
        "metric": "active-token loop-steps/sec + KV GB/s; % of HBM / bf16-MFMA roofline",
        "value": value,
        "unit": "active-token loop-steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_with_kernel_events": ms_instrumented,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; shapes and change/heavy-key structure of the pages' workloads)",
        "config": {"workload": wl.name, "n_seq": wl.n_seq, "heads": wl.n_heads, "head_dim": wl.head_dim,
                   "seq_len": wl.n_tokens, "loops": wl.n_loops, "full_loops": wl.n_full,
                   "active": list(wl.active), "keys": wl.n_keys,
                   "delta_bits": wl.delta_bits, "group": wl.group},
        "kv_GBps": work["kv_bytes"] / (elapsed / args.steps) / 1e9,
        "lazy_active_token_steps_per_s": (work["lazy_rows"] / (lazy_ms / 1e3)) if lazy_ms > 0 else None,
        "kernels_ms_per_step": {k: round(v[0] / args.steps, 4) for k, v in sorted(timings.items())},
        "roofline": roofline(timings, work, args.steps, wl.decode, label),
        # the lazy loops' attention on its own: the gathered-tile MFMA kernel
        # (prefill) or the chain read (decode), loops after the full ones
        "roofline_lazy_attention": (roofline(timings, work, args.steps, wl.decode, label, kernel=lazy_kernel)
                                    if lazy_kernel else None),
    }
    if args.cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
