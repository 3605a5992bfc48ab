"""Summaries of rocprofv3 output for the committed profiles (bench-side tool, not part of the library).

Two uses:

* ``kernel-stats``: turn a ``--kernel-trace --stats`` kernel_stats CSV into a
  short markdown table (calls, total / average / min / max duration).
* ``sweep-table``: turn the JSON line of ``bench.py --workload ragged`` into a
  markdown table (per combination: step time, each kernel's time and rate,
  and its fraction of the roofline that bounds it).
* ``traffic``: from two ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs over
  the benchmark (and the same two counters over a plain copy of known size),
  write the per-launch HBM traffic of one kernel as JSON.  The counters are
  in KiB per dispatch; each is scaled by (bytes the copy really moves) /
  (bytes the counter reports for the copy).  The JSON carries a hash of the
  kernel's sources so ``bench.py`` reports the figure only while the kernel
  is unchanged.

Usage:
  python bench_rocprof.py kernel-stats STATS_CSV OUT_MD --command "..." [--include REGEX]
  python bench_rocprof.py sweep-table BENCH_JSON OUT_MD --command "..."
  python bench_rocprof.py traffic --kernel REGEX --fetch CSV --write CSV \
      --copy-fetch CSV --copy-write CSV --copy-bytes N --out OUT_JSON --command "..."
"""
import argparse
import csv
import hashlib
import json
import os
import re
import statistics

PKG = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mxfp4_block_scaled_cast_amd")
GEMM_SOURCES = [os.path.join(PKG, "csrc", f) for f in ("gemm.hip", "mx_device.h", "mx_host.h")]
CAST_SOURCES = [os.path.join(PKG, "csrc", f) for f in ("cast.hip", "mx_device.h", "mx_host.h")]


def _code_only(text):
    """The source without its comments and blank lines (a comment edit leaves the kernels, and so
    the counters taken on them, unchanged).  String literals holding // or /* are not expected."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def window_average(trace_csv, kernel_regex, start, count):
    """Average duration (us) of dispatches start .. start+count-1, in start order, of the kernels
    matching kernel_regex in a --kernel-trace CSV (e.g. the dispatches of one timed pass)."""
    rows = [r for r in csv.DictReader(open(trace_csv)) if re.search(kernel_regex, r["Kernel_Name"])]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    sel = rows[start:start + count]
    if len(sel) < count:
        raise SystemExit("only %d dispatches of %r after %d" % (len(sel), kernel_regex, start))
    return statistics.mean((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel)


def kernel_stats(csv_path, out_md, command, include=None, trace=None, windows=(), note=None):
    rows = [r for r in csv.DictReader(open(csv_path)) if include is None or re.search(include, r["Name"])]
    lines = ["# rocprofv3 kernel statistics", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | total ms | average us | min us | max us | % |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        name = re.sub(r"\(.*", "", name)
        lines.append("| %s | %s | %.3f | %.1f | %.1f | %.1f | %.1f |" % (
            name, r["Calls"], float(r["TotalDurationNs"]) / 1e6, float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    if windows:
        lines += ["", "| kernel | dispatches (in start order) | average us |", "|---|---|---|"]
        for spec in windows:
            regex, rng = spec.rsplit("@", 1)
            start, count = (int(x) for x in rng.split(":"))
            lines.append("| %s | %d .. %d | %.1f |" % (regex, start, start + count - 1,
                                                       window_average(trace, regex, start, count)))
    if note:
        lines += ["", note]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def sweep_table(json_path, out_md, command):
    d = json.load(open(json_path))
    kinds = list(d["per_combo"][0]["kernels"])  # launch order of the step
    lines = ["# Edge / ragged sweep: one training step per (M, N, K)", "", "Command:", "", "```", command, "```", "",
             "Each cell: kernel time in us, its rate (TFLOP/s for GEMMs, GB/s for casts) and, in brackets, the "
             "fraction of the roofline that bounds it (ideal time at 10.1 PFLOP/s or 8 TB/s, whichever is "
             "longer, over the measured time).", "",
             "Whole sweep: %.2f ms for %.1f TFLOP, %.1f TFLOP/s." % (d["ms_per_step"], d["config"]["step_tflop"],
                                                                    d["value"]), "",
             "| M | N | K | step us | " + " | ".join(kinds) + " |", "|---|---|---|---|" + "---|" * len(kinds)]
    for c in d["per_combo"]:
        cells = []
        for k in kinds:
            x = c["kernels"][k]
            rate = ("%.0f T" % x["tflops"]) if "tflops" in x else ("%.0f GB/s" % x["gbps"])
            cells.append("%.1f, %s (%.2f)" % (x["ms"] * 1e3, rate, x["roofline_frac"]))
        lines.append("| %d | %d | %d | %.1f | %s |" % (c["M"], c["N"], c["K"], c["ms_step"] * 1e3, " | ".join(cells)))
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_dispatch(csv_path, counter, kernel_regex):
    vals = []
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter and re.search(kernel_regex, r["Kernel_Name"]):
            vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit("no %s values for kernels matching %r in %s" % (counter, kernel_regex, csv_path))
    return vals


def traffic(a):
    fetch = _per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    write = _per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    cf = statistics.mean(_per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel))
    cw = statistics.mean(_per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel))
    f_scale = a.copy_bytes / (cf * 1024.0)
    w_scale = a.copy_bytes / (cw * 1024.0)
    fetch_b = statistics.mean(fetch) * 1024.0 * f_scale
    write_b = statistics.mean(write) * 1024.0 * w_scale
    out = {"kernel_regex": a.kernel, "dispatches": len(fetch),
           "fetch_kib_per_dispatch": statistics.mean(fetch), "write_kib_per_dispatch": statistics.mean(write),
           "copy_bytes": a.copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "traffic_bytes_per_launch": fetch_b + write_b,
           "source_hash": source_hash(GEMM_SOURCES if a.sources == "gemm" else CAST_SOURCES),
           "command": a.command}
    with open(a.out, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def main():
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernel-stats")
    k.add_argument("csv")
    k.add_argument("out")
    k.add_argument("--command", required=True)
    k.add_argument("--include", default=None, help="only kernels whose name matches this regex")
    k.add_argument("--trace", default=None, help="the run's kernel_trace CSV (for --window)")
    k.add_argument("--window", action="append", default=[],
                   help="REGEX@START:COUNT: average duration of those dispatches of the matching kernels")
    k.add_argument("--note", default=None, help="text appended to the summary")
    w = sub.add_parser("sweep-table")
    w.add_argument("json")
    w.add_argument("out")
    w.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True)
    # the runtime's copy kernel only: the fill that initialises the source reads nothing
    t.add_argument("--copy-kernel", default="copyBuffer")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--sources", choices=["gemm", "cast"], default="gemm")
    t.add_argument("--out", required=True)
    t.add_argument("--command", required=True)
    a = p.parse_args()
    if a.cmd == "kernel-stats":
        kernel_stats(a.csv, a.out, a.command, a.include, a.trace, a.window, a.note)
    elif a.cmd == "sweep-table":
        sweep_table(a.json, a.out, a.command)
    else:
        traffic(a)


if __name__ == "__main__":
    main()
