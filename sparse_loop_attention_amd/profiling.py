"""Profiler helpers: a copy kernel of known size for counter calibration, and
text summaries of rocprofv3 output (kernel statistics, HBM traffic).

    python -m sparse_loop_attention_amd.profiling copy [--gib 1] [--reps 3]
        one torch copy of a known size per rep, to calibrate FETCH_SIZE and
        WRITE_SIZE against bytes actually moved;
    python -m sparse_loop_attention_amd.profiling stats STATS_CSV --title T --command C
        markdown table of a `rocprofv3 --kernel-trace --stats` summary;
    python -m sparse_loop_attention_amd.profiling traffic --fetch DIR --write DIR
            --cal-fetch DIR --cal-write DIR --kernel SUBSTR --timer NAME
            --workload NAME --command C [--cal-bytes B]
        per-dispatch HBM bytes of one kernel from two `--pmc` runs, each
        counter scaled by what it reads for the copy kernel; the result
        carries a hash of the library sources so that a reader can tell
        whether the kernel changed since the counters were taken.

    python -m sparse_loop_attention_amd.profiling counters --dir DIR [--dir DIR ...]
            --kernel LABEL=SUBSTR [--kernel ...] --title T --command C
        per-dispatch averages of every counter found in one or more
        `rocprofv3 --pmc` runs, per kernel, with derived ratios (MFMA busy
        share of the CUs' busy SIMD cycles, MFMA operations against the
        kernel's algorithmic flops, LDS bank-conflict share, VALU and
        transcendental instructions per MFMA).

Traffic summaries are markdown files under profiles/ holding one line
`traffic-record: {json}` that bench.py reads.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)


def source_hash() -> str:
    """Hash of everything the kernels are built from."""
    files = sorted(glob.glob(os.path.join(PKG, "csrc", "*"))) + [os.path.join(ROOT, "include", "flashloop.h"),
                                                                 os.path.join(PKG, "build.py")]
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic_records(profiles_dir: str):
    """Every `traffic-record:` line of the markdown files under profiles/."""
    out = []
    for f in sorted(glob.glob(os.path.join(profiles_dir, "*.md"))):
        with open(f) as fh:
            for line in fh:
                if line.startswith("traffic-record:"):
                    rec = json.loads(line[len("traffic-record:"):])
                    rec["file"] = os.path.relpath(f, ROOT)
                    out.append(rec)
    return out


def _counter_csv(d: str) -> str:
    hits = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if len(hits) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {d}, found {len(hits)}")
    return hits[0]


def per_dispatch(d: str, counter: str, kernel_substr: str):
    """Values of `counter` per dispatch of kernels whose name contains kernel_substr."""
    vals = collections.defaultdict(float)
    names = {}
    with open(_counter_csv(d)) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter or kernel_substr not in r["Kernel_Name"]:
                continue
            k = int(r["Dispatch_Id"])
            vals[k] += float(r["Counter_Value"])
            names[k] = r["Kernel_Name"]
    return [vals[k] for k in sorted(vals)], sorted(set(names.values()))


def cmd_copy(a):
    import torch
    n = int(a.gib * (1 << 30)) // 4
    x = torch.empty(n, dtype=torch.float32, device="cuda")
    x.fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(a.reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(f"copied {a.reps} x {n * 4} bytes", flush=True)


def cmd_stats(a):
    with open(a.stats_csv) as fh:
        rows = list(csv.DictReader(fh))
    # per-dispatch durations from the trace beside the statistics, for the
    # minimum, the median and the mean of each kernel's last `solo_last`
    # dispatches (bench.py's one-stream timing passes come last)
    trace = os.path.join(os.path.dirname(a.stats_csv), os.path.basename(a.stats_csv).replace("kernel_stats", "kernel_trace"))
    durs = collections.defaultdict(list)
    if os.path.exists(trace):
        with open(trace) as fh:
            for r in csv.DictReader(fh):
                durs[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    solo = f" | last {a.solo_last} avg us" if a.solo_last else ""
    out = [f"# {a.title}", "", "Command (from the repository root, one MI355X):", "", "```", a.command, "```", ""]
    if a.solo_last:
        out += [f"The last {a.solo_last} dispatches of each lazy-loop kernel are bench.py's one-stream timing passes "
                "(per call, then per kernel); earlier dispatches of the lazy loops ran beside the token selection "
                "on the second stream.", ""]
    out += [f"| kernel | calls | total ms | avg us | min us | median us{solo} | % |",
            "|---|---|---|---|---|---|" + ("---|" if a.solo_last else "") + "---|"]
    for r in rows[:a.top]:
        name = r["Name"]
        d = sorted(durs.get(name, []))
        mn = f"{d[0]:.1f}" if d else "-"
        md = f"{d[len(d) // 2]:.1f}" if d else "-"
        extra = ""
        if a.solo_last:
            seq = [x for x in durs.get(name, [])][-a.solo_last:]
            extra = f" | {sum(seq) / len(seq):.1f}" if seq else " | -"
        short = name if len(name) <= 96 else name[:93] + "..."
        out.append(f"| `{short}` | {r['Calls']} | {int(r['TotalDurationNs']) / 1e6:.3f} | "
                   f"{float(r['AverageNs']) / 1e3:.1f} | {mn} | {md}{extra} | {float(r['Percentage']):.2f} |")
    print("\n".join(out))


def cmd_traffic(a):
    fetch, names = per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    write, _ = per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    cal_f, _ = per_dispatch(a.cal_fetch, "FETCH_SIZE", a.cal_kernel)
    cal_w, _ = per_dispatch(a.cal_write, "WRITE_SIZE", a.cal_kernel)
    if not (fetch and write and cal_f and cal_w):
        raise SystemExit("missing dispatches")
    kib = 1024.0
    # bytes moved per KiB the counter reports, from the copy of known size
    f_factor = a.cal_bytes / (sum(cal_f) / len(cal_f) * kib)
    w_factor = a.cal_bytes / (sum(cal_w) / len(cal_w) * kib)
    f_avg = sum(fetch) / len(fetch)
    w_avg = sum(write) / len(write)
    traffic = f_avg * kib * f_factor + w_avg * kib * w_factor
    rec = {"timer": a.timer, "workload": a.workload, "kernel": names[0] if names else a.kernel,
           "dispatches": len(fetch), "fetch_kib": f_avg, "write_kib": w_avg,
           "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4),
           "traffic_bytes": traffic, "source_hash": source_hash()}
    out = [f"# HBM traffic of `{a.timer}` on the {a.workload} workload", "",
           "Commands (from the repository root, one MI355X; each counter in a run of its own):", "", "```",
           a.command, "```", "",
           f"* kernel: `{rec['kernel'][:120]}`, {len(fetch)} dispatch(es) averaged",
           f"* FETCH_SIZE {f_avg:.0f} KiB/dispatch x {f_factor:.3f} (copy calibration) = "
           f"{f_avg * kib * f_factor / 1e6:.1f} MB",
           f"* WRITE_SIZE {w_avg:.0f} KiB/dispatch x {w_factor:.3f} (copy calibration) = "
           f"{w_avg * kib * w_factor / 1e6:.1f} MB",
           f"* copy calibration: {a.cal_bytes} bytes read and written per dispatch; FETCH_SIZE reads "
           f"{sum(cal_f) / len(cal_f):.0f} KiB, WRITE_SIZE {sum(cal_w) / len(cal_w):.0f} KiB",
           f"* sources hash {rec['source_hash']} (the record is stale once the library sources change)",
           "", "traffic-record: " + json.dumps(rec)]
    print("\n".join(out))


def all_counters(d: str, kernel_substr: str):
    """{counter: [value per dispatch]} of kernels whose name contains kernel_substr."""
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    names = set()
    with open(_counter_csv(d)) as fh:
        for r in csv.DictReader(fh):
            if kernel_substr not in r["Kernel_Name"]:
                continue
            vals[r["Counter_Name"]][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
            names.add(r["Kernel_Name"])
    return {c: [v[k] for k in sorted(v)] for c, v in vals.items()}, sorted(names)


def cmd_counters(a):
    out = [f"# {a.title}", "", "Commands (from the repository root, one MI355X; one `--pmc` set per run):", "",
           "```", a.command, "```", ""]
    for spec in a.kernel:
        label, sub = spec.split("=", 1)
        merged, names = {}, set()
        for d in a.dir:
            c, n = all_counters(d, sub)
            names.update(n)
            for k, v in c.items():
                merged[k] = sum(v) / len(v)
        if not merged:
            out += [f"## {label}", "", f"no dispatch of `{sub}`", ""]
            continue
        out += [f"## {label}", "", f"kernel: `{sorted(names)[0][:140]}`", "", "| counter | per dispatch |", "|---|---|"]
        for k in sorted(merged):
            out.append(f"| {k} | {merged[k]:.4g} |")
        g = merged.get
        derived = []
        # Units, from the counters' own consistency on this chip: GRBM_GUI_ACTIVE
        # is summed over the 8 XCDs (per XCD it matches the kernel time at
        # 1.8-2.1 GHz), SQ_BUSY_CU_CYCLES over the 256 CUs and
        # SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs (MOPS x 512 / 1024 flops per
        # cycle reproduces it)
        if g("SQ_BUSY_CU_CYCLES") and g("GRBM_GUI_ACTIVE"):
            derived.append(("CU busy fraction: SQ_BUSY_CU_CYCLES / (256 x GRBM_GUI_ACTIVE / 8)",
                            g("SQ_BUSY_CU_CYCLES") / (256 * g("GRBM_GUI_ACTIVE") / 8)))
        if g("SQ_VALU_MFMA_BUSY_CYCLES") and g("SQ_BUSY_CU_CYCLES"):
            derived.append(("MFMA busy while the CU is busy: SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES)",
                            g("SQ_VALU_MFMA_BUSY_CYCLES") / (4 * g("SQ_BUSY_CU_CYCLES"))))
        if g("SQ_VALU_MFMA_BUSY_CYCLES") and g("GRBM_GUI_ACTIVE"):
            derived.append(("MFMA busy over the kernel: SQ_VALU_MFMA_BUSY_CYCLES / (1024 x GRBM_GUI_ACTIVE / 8)",
                            g("SQ_VALU_MFMA_BUSY_CYCLES") / (1024 * g("GRBM_GUI_ACTIVE") / 8)))
        if g("SQ_WAIT_INST_ANY") and g("SQ_WAVE_CYCLES"):
            derived.append(("wave time waiting on a dependency: SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES",
                            g("SQ_WAIT_INST_ANY") / g("SQ_WAVE_CYCLES")))
        if g("SQ_LDS_BANK_CONFLICT") and g("SQ_ACTIVE_INST_LDS"):
            derived.append(("LDS bank-conflict cycles / LDS active cycles",
                            g("SQ_LDS_BANK_CONFLICT") / (4 * g("SQ_ACTIVE_INST_LDS"))))
        if g("SQ_INSTS_MFMA"):
            for k in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS"):
                if g(k):
                    derived.append((f"{k} per MFMA instruction", g(k) / g("SQ_INSTS_MFMA")))
        mops = sum(g(k) or 0.0 for k in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16"))
        if mops:
            derived.append(("MFMA flops (MOPS x 512)", mops * 512))
        if g("SQ_VALU_MFMA_COEXEC_CYCLES") and g("SQ_VALU_MFMA_BUSY_CYCLES"):
            derived.append(("VALU co-issued during MFMA / MFMA busy", g("SQ_VALU_MFMA_COEXEC_CYCLES") / g("SQ_VALU_MFMA_BUSY_CYCLES")))
        if derived:
            out += ["", "| derived | value |", "|---|---|"] + [f"| {k} | {v:.4g} |" for k, v in derived]
        out.append("")
    print("\n".join(out))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--gib", type=float, default=1.0)
    c.add_argument("--reps", type=int, default=3)
    s = sub.add_parser("stats")
    s.add_argument("stats_csv")
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--top", type=int, default=16)
    s.add_argument("--solo-last", type=int, default=0)
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "cal_fetch", "cal_write", "kernel", "timer", "workload", "command"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--cal-kernel", default="copyBuffer")
    t.add_argument("--cal-bytes", type=float, default=float(1 << 30))
    k = sub.add_parser("counters")
    k.add_argument("--dir", action="append", required=True)
    k.add_argument("--kernel", action="append", required=True, help="LABEL=name substring")
    k.add_argument("--title", required=True)
    k.add_argument("--command", required=True)
    a = ap.parse_args(argv)
    {"copy": cmd_copy, "stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    main()
