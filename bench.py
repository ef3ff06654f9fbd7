#!/usr/bin/env python3
"""Benchmark of the FlashLoop loop step on one MI355X.

One step = every loop of one workload, in order: the full early loops (commit
the base or a dense delta layer, full causal attention with column mass) and
the lazy loops (token selection, key selection, delta commit of the active
tokens, mass-corrected attention), i.e. every step of the hot path over one
batch of synthetic input already resident in HBM.  ``ms_per_step`` times K
such steps without instrumentation.

The headline metric is the lazy loops' own rate: active-token loop-steps/s =
(sum over the lazy loops of n_active) / (the lazy loops' time), where the
lazy loops' time is the median, over R repetitions, of a hipEvent pair
bracketing every library call of loops F+1..T, each repetition started from
the same state after the full loops (a device checkpoint restored untimed).
KV GB/s = (chain bytes read by the commit and the attention + delta bytes
written) / the same time.  The JSON line also carries per-call medians (p10,
p90) measured with each call on its own (no second stream), per-kernel
hipEvent times, the roofline of the lazy loops' attention kernel (the
gathered-tile MFMA forward in prefill, the chain read in decode; flops or
bytes counted from the actual index sets) with the full loop's dominant
kernel beside it, and the CPU oracle timed on the host on the same lazy loops.
"""
from __future__ import annotations

import argparse
import copy
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_VECTOR_PEAK_TFLOPS = 157.3
METRIC = "active-token loop-steps/sec + KV GB/s; % of HBM / bf16-MFMA roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed whole steps (every loop)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--reps", type=int, default=50, help="repetitions of the lazy loops for the medians")
    ap.add_argument("--workload", default="long_prefill",
                    help="long_prefill (default) | single_layer | decode | deep | tiny")
    ap.add_argument("--cpu-baseline", type=int, default=1, help="0 skips the host oracle timing")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of each oracle sample")
    ap.add_argument("--delta-bits", type=int, default=4, choices=(2, 4),
                    help="bits per stored delta element of the lazy loops' KV versions")
    ap.add_argument("--group", type=int, default=32, choices=(32, 64),
                    help="delta elements sharing one binary16 scale (must divide head_dim)")
    ap.add_argument("--exit-threshold", type=float, default=None,
                    help="instead of the benchmark line: step time with early exit at this threshold against "
                         "the full loop count, and the loops each sequence ran")
    ap.add_argument("--quality", action="store_true",
                    help="instead of timing: error of every lazy loop against the dense loop, for the output "
                         "formulas and key policies, and the cost of bf16 attention operands")
    return ap.parse_args()


def _pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, np.float64), q))


def _stats(xs):
    return {"median": _pct(xs, 50), "p10": _pct(xs, 10), "p90": _pct(xs, 90), "n": len(xs)}


# --------------------------------------------------------------------------- work model
def _pairs(rows, keys_sorted):
    """sum over rows i of |{j in keys : j <= i}| for ascending key lists."""
    import numpy as np
    return int(np.searchsorted(keys_sorted, rows, side="right").sum())


def work_model(wl, run):
    """Algorithmic work of each lazy loop, counted from the run's actual index
    sets: 8d flops per visible (row, selected key) pair in the attention (6d
    for the mixture formula), 4d in its column-mass pass; chain bytes read by
    the commit (the active tokens' previous version) and by the attention (the
    selected keys' versions l-1 and l: base row + the records present in
    layers 2..l-1, the layer-l version of an active key being derived from its
    new row), delta records written.  Full loops: 4d flops per causal pair.
    Decode: the lazy kernel reads each selected key's base rows and every
    record it holds up to layer l (the context's layers are stored before the
    loops run)."""
    import numpy as np
    H, d, N = wl.n_heads, wl.head_dim, wl.n_tokens
    es = 2 if wl.dtype == "bf16" else 4
    rec = d * wl.delta_bits // 8 + 2 * (d // wl.group)   # bytes of one delta record (one head row)
    fl = 6 if getattr(run, "formula", "column") == "mixture" else 8
    out = {"loops": {}, "full": {}}
    if wl.decode:
        S = wl.n_seq
        present = {}
        for l in range(2, wl.n_loops + 1):
            m = np.zeros((S, N), bool)
            ctx = run.ctx[l].cpu().numpy()
            for s in range(S):
                m[s, ctx[s]] = True
            m[:, N - 1] = True                               # the new token writes a record every loop
            present[l] = m
        out["full"][1] = {"flops": 4 * d * S * H * N, "bytes": 2 * S * H * N * d * es}
        keys = run.keys.cpu().numpy()                        # the last lazy loop's keys (per-loop sets: see run)
        for l in range(2, wl.n_loops + 1):
            ks = run.keys_by_loop[l] if hasattr(run, "keys_by_loop") else keys
            n_rec = sum(int(np.take_along_axis(present[lp][:, None, :].repeat(H, 1), ks, 2).sum())
                        for lp in range(2, l + 1))
            attend = 2 * (S * H * ks.shape[-1] * d * es + n_rec * rec)
            commit = 2 * H * S * (d * es + (l - 2) * rec)          # the new token has a record in every layer
            out["loops"][l] = {"rows": S, "pairs": S * H * ks.shape[-1], "attn_flops": fl * d * S * H * ks.shape[-1],
                               "attend_bytes": attend, "commit_chain_bytes": commit, "delta_bytes": 2 * H * S * rec}
        return out
    present = {}
    for l in range(2, wl.n_loops + 1):
        m = np.zeros(N, bool)
        if l <= wl.n_full:
            m[:] = True
        else:
            m[run.act[l].cpu().numpy()] = True
        present[l] = m
    for l in range(1, wl.n_full + 1):
        p = H * N * (N + 1) // 2
        out["full"][l] = {"flops": 4 * d * p, "colmass_flops": 2 * d * p}
    for l in range(wl.n_full + 1, wl.n_loops + 1):
        act = run.act[l].cpu().numpy()
        keys = run.keys_l[l].cpu().numpy()
        p = sum(_pairs(act, keys[h]) for h in range(H))
        chain_rec = lambda idx: sum(int(present[lp][idx].sum()) for lp in range(2, l))
        commit = 2 * H * (act.size * d * es + chain_rec(act) * rec)
        attend = 2 * sum(keys[h].size * d * es + chain_rec(keys[h]) * rec for h in range(H))
        cand = N if l == wl.n_full + 1 else wl.n_active(l - 1)
        out["loops"][l] = {"rows": int(act.size), "pairs": p, "attn_flops": fl * d * p, "colmass_flops": 4 * d * p,
                           "attend_bytes": attend, "commit_chain_bytes": commit,
                           "delta_bytes": 2 * H * act.size * rec,
                           "select_bytes": cand * H * d * es * 2 + N * 8 + N * 8 + H * N * 4 + H * wl.n_keys * 4}
    return out


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
    return {"traffic": None}


def roofline_entry(kernel, work, ms, launches, unit, bound, label):
    """Work per launch / average launch time, against MI355X's published peak."""
    avg = ms / max(launches, 1)
    if unit == "GB/s":
        achieved, peak = work / launches / (avg / 1e3) / 1e9, HBM_PEAK_GBPS
    else:
        achieved = work / launches / (avg / 1e3) / 1e12
        peak = MFMA_BF16_PEAK_TFLOPS if bound == "mfma" else FP32_VECTOR_PEAK_TFLOPS
    e = {"kernel": kernel, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
         "avg_launch_ms": avg, "launches": launches, "work_per_launch": work / launches}
    e.update(measured_traffic(kernel, label))
    return e


# --------------------------------------------------------------------------- CPU oracle
def _threads():
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])


def cpu_baseline(wl, target_s):
    """The oracle, as it stands, on the same lazy loops the metric times.

    The full loops run first, untimed (the checkpoint the lazy loops start
    from, as on the GPU).  Prefill: with N above 4096 the oracle runs one head
    of every per-head step (key selection, commit, attention) while the token
    selection scores every token's whole hidden row; the per-head part is
    scaled by the head count (every step but the token selection is per head).
    Decode: the lazy loops of one sequence over its built context.  Timed with
    the BLAS thread pool at its default size and again with one thread.
    """
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from sparse_loop_attention_amd.synth import SyntheticLoops
    lazy = list(range(wl.n_full + 1, wl.n_loops + 1))
    if wl.decode:
        syn = SyntheticLoops(wl, seqs=(0,))
        data = {l: {k: v.copy() for k, v in x.items()} for l, x in syn}
        ctx = {l: syn.context_active_sets(l)[0] for l in range(2, wl.n_loops + 1)}
        store = oracle.build_decode_context(wl, 0, ctx, data)
        head = oracle.run_decode_loops(wl, store, 0, data, upto=1)           # loop 1, untimed

        def once():
            st = copy.deepcopy(store)
            t0 = time.perf_counter()
            oracle.run_decode_loops(wl, st, 0, data, start=2, state=head[-1])
            return time.perf_counter() - t0
        rows = len(lazy)
        what = f"the {len(lazy)} lazy decode loops of 1 of {wl.n_seq} sequences over its built context"
        t_sel, hs = 0.0, wl.n_heads
    else:
        hs = wl.n_heads if wl.n_tokens <= 4096 else 1
        raw = [(l, {k: v.copy() for k, v in x.items()}) for l, x in SyntheticLoops(wl)]
        data = [(l, {k: (v if k == "h" else np.ascontiguousarray(v[:, :, :hs])) for k, v in x.items()})
                for l, x in raw]
        wl_s = dataclasses.replace(wl, n_heads=hs)
        t0 = time.perf_counter()
        ck = oracle.run_prefill(wl_s, iter(data), upto=wl.n_full)           # full loops, untimed
        print(f"[bench] oracle full loops ({hs} heads, untimed): {time.perf_counter() - t0:.1f} s",
              file=sys.stderr, flush=True)
        hx = {l: x["h"][0] for l, x in raw}

        def once():
            t0 = time.perf_counter()
            oracle.run_prefill(wl_s, iter(data), resume=ck)
            return time.perf_counter() - t0

        def selection():                   # the part that is not per head: every token's whole hidden row
            t0 = time.perf_counter()
            for l in lazy:
                oracle.topk_ascending(oracle.token_scores(hx[l - 1], hx[l - 2]), wl.n_active(l))
            return time.perf_counter() - t0
        rows = sum(wl.n_active(l) for l in lazy)
        what = (f"lazy loops {lazy[0]}-{lazy[-1]} (N = {wl.n_tokens}) after the untimed full loops, "
                + ("all heads" if hs == wl.n_heads else
                   f"{hs} of {wl.n_heads} heads for the per-head steps, scaled by {wl.n_heads}/{hs}, "
                   f"token selection over the whole hidden row"))
    out = {}
    for threads in (None, 1):
        with threadpool_limits(limits=threads):
            cores = _threads()
            n, busy = 0, 0.0
            while busy < (target_s if threads is None else 0.5 * target_s) or n == 0:
                busy += once()
                n += 1
            t_run = busy / n
            t_sel = 0.0
            if not wl.decode and hs < wl.n_heads:
                t_sel = min(selection(), t_run)
            t_step = t_sel + (t_run - t_sel) * wl.n_heads / hs
        print(f"[bench] oracle, {cores} thread(s): {n} run(s), {t_run:.2f} s each", file=sys.stderr, flush=True)
        out[threads] = {"value": rows / t_step, "unit": "active-token loop-steps/s", "cores": cores,
                        "kind": "oracle", "sample": f"{n} run(s) of {what}; {t_run:.2f} s per run"
                        + (f", of which {t_sel:.2f} s token selection" if t_sel else "")}
    res = out[None]
    res["single_thread"] = out[1]
    return res


# --------------------------------------------------------------------------- quality
def quality(wl):
    """Lazy loops against the dense loop they stand in for.

    After each lazy loop l the dense reference is full causal attention of
    every row (the effective queries) over the store's version l, computed by
    the library's full mode; the error is ||o - o_dense|| / ||o_dense|| over
    all rows and over the loop's active rows, for each output formula and key
    policy.  Also, at a size the oracle finishes in seconds (at most 1024
    tokens and 4 heads), the GPU's largest error against the oracle with
    attention's K^, V^ rounded to bf16 (the parity reference) and against the
    oracle that attends to the float32 reconstruction: what bf16 operands cost.
    """
    import numpy as np
    import torch
    import oracle
    from sparse_loop_attention_amd import abi, configs, driver
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
    small = configs.scaled(wl, min(n, 1024), n_heads=min(H, 4))
    run = driver.PrefillRun(small, driver.upload_loops(small, SyntheticLoops(small), "cuda"), "cuda")
    recs = run.run(record=True)
    torch.cuda.synchronize()
    ops = {}
    for od in (None, "fp32"):
        _, hist = oracle.run_prefill(small, iter(SyntheticLoops(small)), keep=True, operand_dtype=od)
        per = []
        for l in range(1, small.n_loops + 1):
            want = hist[l - 1].o
            got = recs[l - 1].o.cpu().numpy().astype(np.float64)
            per.append({"loop": l, "max_abs_err_over_rms": float(np.abs(got - want).max() / np.sqrt(np.mean(want ** 2)))})
        ops["bf16_operands" if od is None else "fp32_operands"] = per
    out["gpu_vs_oracle_operands"] = {"workload": f"{small.name} scaled to N = {small.n_tokens}, {small.n_heads} heads",
                                     **ops}
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


# --------------------------------------------------------------------------- GPU timing
# the lazy loops' attention kernel and the full loop's dominant kernel, by workload kind
LAZY_KERNEL = {"prefill": ("mfma_fwd_lazy", "attn_flops", "TFLOP/s", "mfma"),
               "decode": ("rows_attend_commit_lazy", "attend_bytes", "GB/s", "hbm"),
               "fp32": ("rows_attend_commit_lazy", "attn_flops", "TFLOP/s", "alu")}
FULL_KERNEL = {"prefill": ("mfma_fwd_full", "flops", "TFLOP/s", "mfma"),
               "decode": ("rows_attend_full", "bytes", "GB/s", "hbm"),
               "fp32": ("rows_attend_full", "flops", "TFLOP/s", "alu")}


def make_run(wl, inputs, syn, overlap=None):
    from sparse_loop_attention_amd import driver
    if wl.decode:
        ctx_sets = {l: syn.context_active_sets(l) for l in range(2, wl.n_loops + 1)}
        run = driver.DecodeRun(wl, inputs, ctx_sets, "cuda")
        run.build_context()
        return run
    return driver.PrefillRun(wl, inputs, "cuda", overlap=overlap)


def time_lazy_loops(run, wl, reps):
    """Median (p10, p90) over `reps` of the lazy loops' time, each repetition
    from the state after the full loops (restored untimed).  The lazy loops
    rewrite their own layers and index sets, so the restored outputs (o, lse,
    column mass) are all a repetition needs."""
    import torch
    first = wl.n_full + 1
    run.run(upto=wl.n_full)
    snap = run.snapshot(arena=False)
    times = []
    for _ in range(reps):
        run.restore(snap)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run.run(start=first)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    return times, snap


def per_call_and_kernel_times(run, wl, snap, reps):
    """Each library call of the lazy loops on its own (one stream): hipEvent
    medians per call; and per lazy loop, the kernels' hipEvent times (a
    second pass, so the kernel events do not add to the call times)."""
    import torch
    from sparse_loop_attention_amd import abi, driver
    first = wl.n_full + 1
    timer = driver.CallTimer()
    run.timer = timer
    for _ in range(reps):
        run.restore(snap)
        run.run(start=first)
    calls = timer.ms()
    run.timer = driver._NO_TIMER
    per_loop = {l: {} for l in range(first, wl.n_loops + 1)}
    keys_by_loop = {}
    for _ in range(max(3, reps // 5)):
        run.restore(snap)
        for l in range(first, wl.n_loops + 1):
            abi.timing_enable(True)
            run.run(start=l, upto=l)
            t = abi.timing_read()
            abi.timing_enable(False)
            for k, (ms, n) in t.items():
                acc = per_loop[l].setdefault(k, [0.0, 0])
                acc[0] += ms
                acc[1] += n
            if wl.decode:
                keys_by_loop[l] = run.keys.cpu().numpy()
    torch.cuda.synchronize()
    return {k: _stats(v) for k, v in sorted(calls.items())}, per_loop, keys_by_loop


# --------------------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus must be 1 "
                                   "(the multi-GPU sharding is a design note, not code)"}))
        sys.exit(2)
    import torch
    from sparse_loop_attention_amd import abi, configs, driver
    from sparse_loop_attention_amd.synth import SyntheticLoops

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    abi.lib()
    wl = configs.WORKLOADS[args.workload]
    if wl.head_dim % args.group:
        raise SystemExit(f"--group {args.group} does not divide head_dim {wl.head_dim}")
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
    kind = "decode" if wl.decode else ("prefill" if wl.dtype == "bf16" else "fp32")
    print(f"[bench] workload {label}: generating inputs", file=sys.stderr, flush=True)
    syn = SyntheticLoops(wl)
    inputs = driver.upload_loops(wl, syn, "cuda")
    run = make_run(wl, inputs, syn)
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        run.run()
    torch.cuda.synchronize()
    # whole steps (every loop) as a caller runs them, no instrumentation
    print(f"[bench] timing {args.steps} whole steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run.run()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) / args.steps * 1e3
    # per-kernel hipEvent times over the same K whole steps
    print(f"[bench] per-kernel hipEvent timing over {args.steps} whole steps", file=sys.stderr, flush=True)
    abi.timing_enable(True)
    for _ in range(args.steps):
        run.run()
    torch.cuda.synchronize()
    step_kernels = abi.timing_read()
    abi.timing_enable(False)
    # the metric: the lazy loops from the checkpoint after the full loops
    print(f"[bench] lazy loops: {args.reps} repetitions", file=sys.stderr, flush=True)
    lazy_times, snap = time_lazy_loops(run, wl, args.reps)
    # each call on its own, then each loop's kernels (one stream)
    print("[bench] per-call and per-kernel timing of the lazy loops", file=sys.stderr, flush=True)
    solo = run if wl.decode else make_run(wl, inputs, syn, overlap=False)
    if solo is not run:
        solo.run(upto=wl.n_full)
        solo.restore(snap)
    calls, per_loop, keys_by_loop = per_call_and_kernel_times(solo, wl, snap, args.reps)
    if wl.decode:
        run.keys_by_loop = keys_by_loop
    work = work_model(wl, run)
    lazy = sorted(work["loops"])
    lazy_ms = _pct(lazy_times, 50)
    rows = sum(work["loops"][l]["rows"] for l in lazy)
    kv_bytes = sum(work["loops"][l]["attend_bytes"] + work["loops"][l]["commit_chain_bytes"]
                   + work["loops"][l]["delta_bytes"] for l in lazy)
    # roofline of the lazy loops' attention kernel, over all lazy loops and per loop
    kname, wkey, unit, bound = LAZY_KERNEL[kind]
    tot_ms = sum(per_loop[l].get(kname, [0.0, 0])[0] for l in lazy)
    tot_n = sum(per_loop[l].get(kname, [0.0, 0])[1] for l in lazy)
    reps_k = max(3, args.reps // 5)
    tot_work = sum(work["loops"][l][wkey] for l in lazy) * reps_k
    roof = roofline_entry(kname, tot_work, tot_ms, tot_n, unit, bound, label) if tot_n else None
    if roof:
        # HBM traffic: each loop's launch is its own kernel instance, with its own
        # counter record (timer "<kernel>@<loop>"); per launch over the loops
        traffic = [measured_traffic(f"{kname}@{l}", label) for l in lazy]
        roof["traffic"] = (sum(t["traffic"] for t in traffic) / len(lazy)
                           if all(t.get("traffic") is not None for t in traffic) else None)
        roof["traffic_sources"] = [t.get("traffic_source") or t.get("traffic_note") for t in traffic]
        roof.pop("traffic_source", None)
        roof.pop("traffic_unit", None)
        roof["scope"] = f"lazy loops {lazy[0]}-{lazy[-1]}: work summed over the loops / kernel time summed"
        roof["per_loop"] = {}
        for l, t in zip(lazy, traffic):
            ms, n = per_loop[l].get(kname, [0.0, 0])
            if n:
                e = roofline_entry(kname, work["loops"][l][wkey] * reps_k, ms, n, unit, bound, label)
                roof["per_loop"][str(l)] = {k: e[k] for k in ("achieved", "frac", "avg_launch_ms", "work_per_launch")}
                roof["per_loop"][str(l)]["traffic"] = t.get("traffic")
    fname, fkey, funit, fbound = FULL_KERNEL[kind]
    full_roof = None
    if fname in step_kernels:
        ms, n = step_kernels[fname]
        fwork = sum(work["full"][l][fkey] for l in work["full"]) * args.steps
        full_roof = roofline_entry(fname, fwork, ms, n, funit, fbound, label)
    out = {
        "metric": METRIC,
        "value": rows / (lazy_ms / 1e3),
        "unit": "active-token loop-steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; shapes and change/heavy-key structure of the pages' workloads)",
        "config": {"workload": wl.name, "n_seq": wl.n_seq, "heads": wl.n_heads, "head_dim": wl.head_dim,
                   "seq_len": wl.n_tokens, "loops": wl.n_loops, "full_loops": wl.n_full,
                   "active": list(wl.active), "keys": wl.n_keys, "delta_bits": wl.delta_bits, "group": wl.group},
        "value_definition": "sum of n_active over the lazy loops / median time of the lazy loops' library calls "
                            "(hipEvents, from the state after the full loops)",
        "lazy_loops_ms": _stats(lazy_times),
        "kv_GBps": kv_bytes / (lazy_ms / 1e3) / 1e9,
        "kv_bytes_per_step": kv_bytes,
        "abi_calls_ms": calls,
        "kernels_ms_per_step": {k: round(v[0] / args.steps, 4) for k, v in sorted(step_kernels.items())},
        "kernels_ms_per_lazy_loop": {str(l): {k: round(v[0] / reps_k, 4) for k, v in sorted(per_loop[l].items())}
                                     for l in lazy},
        "roofline": roof,
        "roofline_full_loop": full_roof,
        "work_per_lazy_loop": {str(l): {k: v for k, v in work["loops"][l].items()} for l in lazy},
    }
    if wl.decode:
        # the same lazy loops as one flashloop_decode_loops launch (every loop's
        # key selection, commit and attention in one kernel), from the same state
        print(f"[bench] lazy loops in one launch: {args.reps} repetitions", file=sys.stderr, flush=True)
        one = driver.DecodeRun(wl, inputs, {l: syn.context_active_sets(l) for l in range(2, wl.n_loops + 1)},
                               "cuda", single_launch=True)
        one.build_context()
        one_times, _ = time_lazy_loops(one, wl, args.reps)
        abi.timing_enable(True)
        for _ in range(reps_k):
            one.restore(snap)
            one.run(start=wl.n_full + 1)
        torch.cuda.synchronize()
        t1 = abi.timing_read()
        abi.timing_enable(False)
        ms1, n1 = t1.get("decode_loops", (0.0, 0))
        attend_bytes = sum(work["loops"][l]["attend_bytes"] for l in lazy)
        out["single_launch"] = {
            "lazy_loops_ms": _stats(one_times),
            "value": rows / (_pct(one_times, 50) / 1e3),
            "kernel": "decode_loops", "avg_launch_ms": ms1 / max(n1, 1),
            "achieved_GBps": attend_bytes / (ms1 / max(n1, 1) / 1e3) / 1e9 if n1 else None,
            "note": "the lazy loops' chain reads (attend_bytes summed over the loops) per launch of the one kernel",
        }
    if args.cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
