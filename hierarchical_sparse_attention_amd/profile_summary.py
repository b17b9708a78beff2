"""Summaries of rocprofv3 output for the repository's profiles/ folder.

  python -m hierarchical_sparse_attention_amd.profile_summary stats \\
      <trace_dir> <bench_json> <out_md> --command "<command that made trace_dir>"
      per-kernel call counts and durations (kernel-trace --stats) next to the
      benchmark line of the same run.

  python -m hierarchical_sparse_attention_amd.profile_summary traffic \\
      <fetch_dir> <write_dir> <copy_fetch_dir> <copy_write_dir> <kernel> <entry> \\
      <workload> <out_json> --command "<commands>"
      HBM bytes per launch of one kernel from FETCH_SIZE and WRITE_SIZE
      (KiB per dispatch), each scaled by what the same counter reads for a
      plain 1 GiB device copy (bench.py --mode copy), stamped with the sha256
      of the kernel's sources so that a later change of the kernel voids it.

Reads CSV files only; runs nothing on the GPU.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _rows(d, name):
    out = []
    for f in glob.glob(os.path.join(d, "**", name), recursive=True):
        out += list(csv.DictReader(open(f)))
    return out


def _short(kernel_name):
    n = kernel_name
    if "::" in n:
        n = n.split("(anonymous namespace)::")[-1]
    return n.split("(")[0]


def stats(args):
    rows = _rows(args.trace_dir, "*kernel_stats.csv")
    bench = json.load(open(args.bench_json))
    lines = ["# Kernel durations: %s" % bench["config"]["workload"], "",
             "Command: `%s`" % args.command, "",
             "rocprofv3 --kernel-trace --stats, all dispatches of the run (warm-up, per-call event "
             "timing, graph replays):", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        if "hs::" not in r["Name"]:
            continue
        lines.append("| `%s` | %s | %.2f | %.2f | %.2f |" % (
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3))
    if "figure" in bench:  # bench.py --mode shared (one figure)
        lines += ["", "Figure of the same run (%s, %d event-timed graph replays each):" % (
            bench["figure"], bench["reps"]), ""]
        lines += ["- %s: %s" % (k, json.dumps(v)) for k, v in bench[bench["figure"]].items()]
        lines.append("")
    else:
        lines += ["", "Benchmark line of the same run:", "",
                  "- ms_per_step (graph replays, %d steps): %.4f" % (bench["steps"],
                                                                    bench["ms_per_step"]),
                  "- value: %.0f %s" % (bench["value"], bench["unit"]),
                  "- per-call event times (ms): %s" % json.dumps(bench["per_call_ms"]),
                  "- roofline: %s" % json.dumps(bench["roofline"]), ""]
    open(args.out_md, "w").write("\n".join(lines))


def _counter_mean(d, counter, match):
    vals = [float(r["Counter_Value"]) for r in _rows(d, "*counter_collection.csv")
            if r["Counter_Name"] == counter and match(r["Kernel_Name"])]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def _largest_kernel_mean(d, counter):
    by = {}
    for r in _rows(d, "*counter_collection.csv"):
        if r["Counter_Name"] == counter:
            by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    name = max(by, key=lambda k: max(by[k]))
    v = by[name]
    return _short(name), sum(v) / len(v), len(v)


def traffic(args):
    sys.path.insert(0, ROOT)
    import bench  # noqa: E402  (source digest shared with the benchmark)

    match = lambda n: args.kernel in n  # noqa: E731
    fetch, nf = _counter_mean(args.fetch_dir, "FETCH_SIZE", match)
    write, nw = _counter_mean(args.write_dir, "WRITE_SIZE", match)
    cname, cfetch, _ = _largest_kernel_mean(args.copy_fetch_dir, "FETCH_SIZE")
    _, cwrite, _ = _largest_kernel_mean(args.copy_write_dir, "WRITE_SIZE")
    gib = float(1 << 30)
    f_fetch = gib / (cfetch * 1024.0)
    f_write = gib / (cwrite * 1024.0)
    rec = {
        "kernel": args.kernel, "entry_point": args.entry, "workload": args.workload,
        "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
        "dispatches": [nf, nw],
        "calibration": {"copy_kernel": cname, "bytes_each_way": int(gib),
                        "fetch_kib": cfetch, "write_kib": cwrite,
                        "fetch_factor": f_fetch, "write_factor": f_write},
        "hbm_bytes_per_launch": fetch * 1024.0 * f_fetch + write * 1024.0 * f_write,
        "source_sha256": bench.source_digest(bench.KERNEL_SOURCES[args.entry]),
        "command": args.command,
    }
    json.dump(rec, open(args.out_json, "w"), indent=2)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("trace_dir")
    a.add_argument("bench_json")
    a.add_argument("out_md")
    a.add_argument("--command", required=True)
    b = sub.add_parser("traffic")
    for n in ("fetch_dir", "write_dir", "copy_fetch_dir", "copy_write_dir", "kernel", "entry",
              "workload", "out_json"):
        b.add_argument(n)
    b.add_argument("--command", required=True)
    args = ap.parse_args(argv)
    (stats if args.what == "stats" else traffic)(args)


if __name__ == "__main__":
    main()
