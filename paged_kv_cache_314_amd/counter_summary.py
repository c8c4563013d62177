"""Turn two rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE) into HBM bytes per launch.

    python -m paged_kv_cache_314_amd.counter_summary KIND WORKLOAD \\
        FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR COPY_MIB "<fetch cmd>" "<write cmd>"

KIND is the kernel (decode_kernel | prefill_kernel | append_kernel). Each *_DIR is a `rocprofv3 --pmc ...
-d DIR -o run --output-format csv` output holding run_counter_collection.csv. The copy
runs profile a plain device-to-device copy of COPY_MIB MiB (`bench.py --copy-probe`),
which fixes the factor between each counter's KiB and the bytes actually moved.

Writes profiles/KIND_WORKLOAD_counters.json (read by bench.py for roofline.traffic,
keyed by the kernel source hash) and prints a short text summary.
"""

import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_314_amd", "csrc")
KERNEL_SOURCES = {
    "decode_kernel": ["decode.hip", "pa_device.h"],
    "prefill_kernel": ["prefill.hip", "pa_device.h"],
    "append_kernel": ["append.hip", "pa_device.h"],
}
COPY_KERNEL = "copyBuffer"


def kernel_source_hash(kind):
    """sha256 (first 16 hex digits) of the sources a kernel is built from."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_values(outdir, counter, name_parts):
    """Per-dispatch values (KiB) of `counter` for kernels whose name contains one of
    name_parts (a string or a tuple of strings)."""
    if isinstance(name_parts, str):
        name_parts = (name_parts,)
    path = os.path.join(outdir, "run_counter_collection.csv")
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or not any(n in r["Kernel_Name"] for n in name_parts):
                continue
            d = r["Dispatch_Id"]          # a counter may come in several rows per dispatch
            vals[d] = vals.get(d, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def main(argv):
    kind, workload, fdir, wdir, cfdir, cwdir, copy_mib, fcmd, wcmd = argv
    copy_kib = float(copy_mib) * 1024.0
    cf = counter_values(cfdir, "FETCH_SIZE", COPY_KERNEL)
    cw = counter_values(cwdir, "WRITE_SIZE", COPY_KERNEL)
    # the largest copy dispatch is the probe (torch may launch small copies too)
    fetch_scale = copy_kib / max(cf)
    write_scale = copy_kib / max(cw)
    part = (f"::{kind}<", f"::{kind}(")        # template or plain kernel
    fv = counter_values(fdir, "FETCH_SIZE", part)
    wv = counter_values(wdir, "WRITE_SIZE", part)
    if not fv or not wv:
        raise SystemExit(f"no {kind} dispatches in the counter files")
    fetch = sum(fv) / len(fv)
    write = sum(wv) / len(wv)
    hbm = (fetch * fetch_scale + write * write_scale) * 1024.0
    out = {
        "kernel": kind,
        "workload": workload,
        "source_sha256_16": kernel_source_hash(kind),
        "dispatches": [len(fv), len(wv)],
        "fetch_kib_per_launch": fetch,
        "write_kib_per_launch": write,
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "copy_probe_mib": float(copy_mib),
        "hbm_bytes_per_launch": hbm,
        "commands": [fcmd, wcmd],
    }
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}_counters.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(f"{kind} {workload}: FETCH {fetch:.0f} KiB x {fetch_scale:.3f} + WRITE {write:.0f} KiB "
          f"x {write_scale:.3f} = {hbm / 1e6:.2f} MB per launch -> {path}")


if __name__ == "__main__":
    main(sys.argv[1:])
