"""Condense rocprofv3 --kernel-trace --stats output into a short text summary.

    python -m paged_kv_cache_314_amd.profile_summary <rocprof output dir> "<command>" \\
        [<bench line of the same command without the profiler> [<bench line printed
        inside the profiled run>]]

Reads <dir>/run_kernel_stats.csv (written by rocprofv3 -d <dir> -o run --stats).  Given
the bench.py JSON lines (files), it sets each of the op's kernel durations that
bench.py measured with HIP events beside rocprofv3's average for the same kernel.
"""

import csv
import json
import os
import sys


def _kernel_rows(rows, kind):
    return [r for r in rows if f"::{kind}<" in r["Name"] or f"::{kind}(" in r["Name"]]


def _bench_kernel_us(roof):
    each = roof.get("kernel_us_each")
    if each:
        return dict(each)
    return {roof["kernel"]: roof["kernel_us"]}


def summarize(outdir, command, plain=None, traced=None):
    path = os.path.join(outdir, "run_kernel_stats.csv")
    with open(path) as f:
        rows = list(csv.DictReader(f))
    lines = [f"command: {command}", "",
             f"{'kernel':40s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>7s}"]
    for r in rows:
        lines.append(f"{r['Name'][:40]:40s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.2f} "
                     f"{float(r['MinNs'])/1e3:10.2f} {float(r['MaxNs'])/1e3:10.2f} "
                     f"{float(r['Percentage']):7.2f}")
    lines += ["", "full kernel names:"] + [f"  {r['Name']}" for r in rows]
    for label, path in (("the same bench.py command without the profiler", plain),
                        ("the bench.py line printed inside the profiled run (kernel tracing "
                         "adds per-dispatch work that its event timestamps include)", traced)):
        if path is None:
            continue
        with open(path) as f:
            line = json.loads([x for x in f.read().splitlines() if x.startswith("{")][-1])
        roof = line["roofline"]
        lines += ["", f"{label}:",
                  f"  roofline: achieved {roof['achieved']:.1f} {roof['unit']}, "
                  f"frac {roof['frac']:.4f}, op kernels {roof['kernel_us']:.2f} us "
                  "(each kernel's mean duration from HIP events attached to its dispatch)"]
        for kind, us in _bench_kernel_us(roof).items():
            k = _kernel_rows(rows, kind)
            if not k:
                lines.append(f"  {kind}: {us:.2f} us (not in the trace)")
                continue
            avg = sum(float(r["AverageNs"]) * int(r["Calls"]) for r in k) / \
                sum(int(r["Calls"]) for r in k) / 1e3
            lines.append(f"  {kind}: {us:.2f} us; rocprofv3 average {avg:.2f} us; "
                         f"difference {100 * (us - avg) / avg:+.1f}%")
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    a = sys.argv[1:]
    sys.stdout.write(summarize(a[0], a[1], a[2] if len(a) > 2 else None,
                               a[3] if len(a) > 3 else None))
