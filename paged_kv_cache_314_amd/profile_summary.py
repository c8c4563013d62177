"""Condense rocprofv3 --kernel-trace --stats output into a short text summary.

    python -m paged_kv_cache_314_amd.profile_summary <rocprof output dir> "<command>" > out.txt

Reads <dir>/run_kernel_stats.csv (written by rocprofv3 -d <dir> -o run --stats).
"""

import csv
import os
import sys


def summarize(outdir, command):
    path = os.path.join(outdir, "run_kernel_stats.csv")
    rows = list(csv.DictReader(open(path)))
    lines = [f"command: {command}", "",
             f"{'kernel':40s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>7s}"]
    for r in rows:
        lines.append(f"{r['Name'][:40]:40s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.2f} "
                     f"{float(r['MinNs'])/1e3:10.2f} {float(r['MaxNs'])/1e3:10.2f} "
                     f"{float(r['Percentage']):7.2f}")
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    sys.stdout.write(summarize(sys.argv[1], sys.argv[2]))
