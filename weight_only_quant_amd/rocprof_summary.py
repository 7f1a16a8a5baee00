"""Summarise rocprofv3 CSV output for the qmat kernels.

    python -m weight_only_quant_amd.rocprof_summary trace <kernel_trace.csv> [--out summary.md]
    python -m weight_only_quant_amd.rocprof_summary traffic --fetch <fetch.csv> --write <write.csv>
        --copy-fetch <copy_fetch.csv> --copy-write <copy_write.csv> --copy-bytes N
        --kernel <substring> --grid <grid size> --workload <name> --alg-bytes N --out traffic.json
    python -m weight_only_quant_amd.rocprof_summary counters <counter_collection.csv> --names A,B,...
        [--kernels <substring>,...] [--out summary.md]

trace:   per (kernel, grid size) dispatch count, mean/median/min duration and the median
         start-to-start period of back-to-back dispatches (graph replays: gap included).
counters: per (kernel, grid) dispatch count and the mean per dispatch of each named counter
         (rocprofv3 --pmc output, one row per dispatch and counter).
traffic: HBM bytes per dispatch of one kernel from FETCH_SIZE and WRITE_SIZE (KiB per
         dispatch), each scaled by what the same counter reports for a device copy of known
         size (the counters need not cover every memory channel).  The JSON also records the
         SHA-256 of the small-T kernels' sources so that a later change to them invalidates it.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import statistics
import sys

# the sources of the small-T product kernels (the benchmark's timed kernels)
KERNEL_SOURCES = [os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", n)
                  for n in ("qmat_kernels.hip", "qmat_device.h", "qmat_kernels.h", "qmat_layout.h")]


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed (so that editing a comment does
    not count as a change of the measured kernels; string literals are not special-cased, which
    is safe for these sources: none holds a comment marker inside a string)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_sha256(sources=None) -> str:
    """SHA-256 over the small-T kernel sources' code (comments and layout ignored)."""
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def _short(name: str) -> str:
    n = name.replace("void qmatk::", "").replace("(qmatk::RunArgs)", "").replace("(qmatk::DequantArgs)", "")
    n = n.replace("void (anonymous namespace)::", "")
    if n.startswith("read_stream_kernel<") and "(" in n:
        n = n[:n.index("(")]  # the read-stream probe: template arguments only
    return n


def trace_summary(path: str):
    """Per (kernel, grid, workgroup): dispatch count, mean / median / min duration, and the
    median start-to-start period of back-to-back dispatches of that kernel (consecutive in the
    trace with nothing in between: the time per launch of a graph replay, dispatch gap included,
    the figure an event-timed replay measures)."""
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    d = collections.defaultdict(list)
    period = collections.defaultdict(list)
    prev = None
    for r in rows:
        grid = r.get("Grid_Size_X") or r.get("Grid_Size")
        key = (_short(r["Kernel_Name"]), grid, r.get("Workgroup_Size_X") or r.get("Workgroup_Size"))
        start = int(r["Start_Timestamp"])
        d[key].append(int(r["End_Timestamp"]) - start)
        if prev is not None and prev[0] == key:
            period[key].append(start - prev[1])
        prev = (key, start)
    out = []
    for (k, g, wg), v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        pv = period.get((k, g, wg))
        out.append({"kernel": k, "grid": int(g), "workgroup": int(wg), "calls": len(v),
                    "mean_us": sum(v) / len(v) / 1e3, "median_us": statistics.median(v) / 1e3, "min_us": min(v) / 1e3,
                    "period_us": statistics.median(pv) / 1e3 if pv else None})
    return out


def counter_mean(path: str, counter: str, kernel: str, grid: str = None) -> float:
    vals = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter or kernel not in r["Kernel_Name"]:
            continue
        if grid is not None and r["Grid_Size"] != str(grid):
            continue
        vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for kernel {kernel!r} grid {grid} in {path}")
    return sum(vals) / len(vals)


def counter_table(path: str, names, kernels=None):
    """{(kernel, grid): {counter: mean per dispatch}} plus each key's dispatch count."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        k = _short(r["Kernel_Name"])
        if r["Counter_Name"] not in names or (kernels and not any(s in k for s in kernels)):
            continue
        vals[(k, int(r["Grid_Size"]))][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = {}
    for key, d in vals.items():
        out[key] = ({n: sum(v) / len(v) for n, v in d.items()}, max(len(v) for v in d.values()))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--out")
    t.add_argument("--command", default="")
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--names", required=True)
    c.add_argument("--kernels", default="")
    c.add_argument("--out")
    c.add_argument("--command", default="")
    f = sub.add_parser("traffic")
    for a in ("fetch", "write", "copy_fetch", "copy_write", "kernel", "grid", "workload", "out"):
        f.add_argument("--" + a.replace("_", "-"), required=True)
    f.add_argument("--copy-bytes", type=int, required=True)
    f.add_argument("--alg-bytes", type=int, required=True)
    f.add_argument("--command", default="")
    args = ap.parse_args(argv)
    if args.cmd == "trace":
        rows = trace_summary(args.csv)
        lines = ["| kernel | grid | workgroup | calls | mean us | median us | min us | period us |",
                 "|---|---|---|---|---|---|---|---|"]
        for r in rows:
            per = f"{r['period_us']:.2f}" if r["period_us"] is not None else ""
            lines.append(f"| {r['kernel']} | {r['grid']} | {r['workgroup']} | {r['calls']} | {r['mean_us']:.2f} | "
                         f"{r['median_us']:.2f} | {r['min_us']:.2f} | {per} |")
        text = "\n".join(lines) + "\n"
        if args.command:
            text = f"Command: `{args.command}`\n\n" + text
        if args.out:
            with open(args.out, "w") as fh:
                fh.write(text)
        print(text)
        return
    if args.cmd == "counters":
        names = args.names.split(",")
        kernels = [k for k in args.kernels.split(",") if k]
        table = counter_table(args.csv, names, kernels)
        lines = ["| kernel | grid | dispatches | " + " | ".join(names) + " |",
                 "|---|---|---|" + "---|" * len(names)]
        for (k, g), (means, n) in sorted(table.items(), key=lambda kv: (kv[0][0], kv[0][1])):
            cells = [f"{means[x]:.4g}" if x in means else "" for x in names]
            short = k if len(k) <= 64 else k[:48] + "..." + k[-12:]
            lines.append(f"| {short} | {g} | {n} | " + " | ".join(cells) + " |")
        text = "\n".join(lines) + "\n"
        if args.command:
            text = f"Command: `{args.command}`\n\n" + text
        if args.out:
            with open(args.out, "w") as fh:
                fh.write(text)
        print(text)
        return
    fetch_kib = counter_mean(args.fetch, "FETCH_SIZE", args.kernel, args.grid)
    write_kib = counter_mean(args.write, "WRITE_SIZE", args.kernel, args.grid)
    copy_fetch_kib = counter_mean(args.copy_fetch, "FETCH_SIZE", "copyBuffer")
    copy_write_kib = counter_mean(args.copy_write, "WRITE_SIZE", "copyBuffer")
    fs = args.copy_bytes / (copy_fetch_kib * 1024)
    ws = args.copy_bytes / (copy_write_kib * 1024)
    traffic = fetch_kib * 1024 * fs + write_kib * 1024 * ws
    rec = {"workload": args.workload, "kernel": args.kernel, "grid": int(args.grid),
           "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib,
           "copy_bytes": args.copy_bytes, "copy_fetch_kib": copy_fetch_kib, "copy_write_kib": copy_write_kib,
           "fetch_scale": fs, "write_scale": ws, "traffic_bytes": traffic, "algorithmic_bytes": args.alg_bytes,
           "traffic_over_algorithmic": traffic / args.alg_bytes, "kernel_source_sha256": kernel_source_sha256(),
           "command": args.command}
    with open(args.out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main(sys.argv[1:])
