"""Condense rocprofv3 counter runs of one kernel on one workload into per-launch figures.

    python -m paged_kv_cache_314_amd.counter_summary traffic KERNEL WORKLOAD \\
        FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR COPY_MIB "<fetch cmd>" "<write cmd>"
    python -m paged_kv_cache_314_amd.counter_summary sq KERNEL WORKLOAD SQ_DIR "<cmd>"

KERNEL is decode_kernel | combine_kernel | prefill_kernel | append_kernel; WORKLOAD is a
workload name, with "@bnnbsd" appended for the head-major cache layout.  Each *_DIR is
a `rocprofv3 --pmc ... -d DIR -o run --output-format csv` output holding
run_counter_collection.csv.

traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what the same
counter reads for a plain device-to-device copy of COPY_MIB MiB (`bench.py
--copy-probe`), give the HBM bytes one launch moves.

sq: the MFMA math operations the kernel executed (SQ_INSTS_VALU_MFMA_MOPS_*, each unit
512 flops), and the fraction of the SIMDs' cycles their MFMA pipes were busy
(SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE per XCD times the SIMD count).

Both merge into profiles/KERNEL_WORKLOAD_counters.json, keyed by the hash of the
kernel's sources and the planner's with comments and blank space left out (bench.py
reads it for roofline.traffic and roofline.executed and ignores it once the code of
either changes), and print a short text summary.
"""

import csv
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_314_amd", "csrc")
# a kernel's counters depend on its code and on the work lists the planner gives it
PLAN_SOURCES = ["plan.cpp", "pa_internal.h"]
KERNEL_SOURCES = {
    "decode_kernel": ["decode.hip", "pa_device.h"] + PLAN_SOURCES,
    "combine_kernel": ["decode.hip", "pa_device.h"] + PLAN_SOURCES,
    "prefill_kernel": ["prefill.hip", "pa_device.h"] + PLAN_SOURCES,
    "append_kernel": ["append.hip", "pa_device.h"] + PLAN_SOURCES,
}
COPY_KERNEL = "copyBuffer"
XCDS = 8                     # MI355X: 8 accelerator complex dies
SIMDS = 256 * 4              # 256 CUs of 4 SIMDs
MOPS_UNIT = 512              # flops per SQ_INSTS_VALU_MFMA_MOPS_* count


def code_text(text):
    """C/C++ source without its comments and with runs of blank space collapsed: what a
    change must touch to change the compiled code (these sources hold no string literal
    with a comment marker in it)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(kind):
    """sha256 (first 16 hex digits) of the code of the sources a kernel and its work lists
    come from (comments and blank space left out)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode("utf-8"))
        h.update(b"\0")
    return h.hexdigest()[:16]


def _name_parts(kind):
    return (f"::{kind}<", f"::{kind}(")        # template or plain kernel


def per_dispatch(outdir, name_parts):
    """{dispatch id: {counter: value summed over its rows, "dur_us": window}} for the
    dispatches whose kernel name contains one of name_parts."""
    if isinstance(name_parts, str):
        name_parts = (name_parts,)
    d = {}
    with open(os.path.join(outdir, "run_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if not any(n in r["Kernel_Name"] for n in name_parts):
                continue
            x = d.setdefault(r["Dispatch_Id"], {})
            # a counter may come in several rows per dispatch (one per die or engine)
            x[r["Counter_Name"]] = x.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            x["dur_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    return d


def counter_values(outdir, counter, name_parts):
    """Per-dispatch values of ``counter`` for kernels whose name contains one of name_parts."""
    return [x[counter] for x in per_dispatch(outdir, name_parts).values() if counter in x]


def _merge(kind, workload, fields):
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}_counters.json")
    out = {}
    if os.path.exists(path):
        with open(path) as f:
            out = json.load(f)
    h = kernel_source_hash(kind)
    if out.get("source_sha256_16") != h:
        out = {}                                 # taken on other sources: start again
    out.update({"kernel": kind, "workload": workload, "source_sha256_16": h})
    out.update(fields)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return path


def traffic(argv):
    kind, workload, fdir, wdir, cfdir, cwdir, copy_mib, fcmd, wcmd = argv
    copy_kib = float(copy_mib) * 1024.0
    cf = counter_values(cfdir, "FETCH_SIZE", COPY_KERNEL)
    cw = counter_values(cwdir, "WRITE_SIZE", COPY_KERNEL)
    # the largest copy dispatch is the probe (torch may launch small copies too)
    fetch_scale = copy_kib / max(cf)
    write_scale = copy_kib / max(cw)
    fv = counter_values(fdir, "FETCH_SIZE", _name_parts(kind))
    wv = counter_values(wdir, "WRITE_SIZE", _name_parts(kind))
    if not fv or not wv:
        raise SystemExit(f"no {kind} dispatches in the counter files")
    fetch = sum(fv) / len(fv)
    write = sum(wv) / len(wv)
    hbm = (fetch * fetch_scale + write * write_scale) * 1024.0
    path = _merge(kind, workload, {
        "dispatches": [len(fv), len(wv)],
        "fetch_kib_per_launch": fetch,
        "write_kib_per_launch": write,
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "copy_probe_mib": float(copy_mib),
        "hbm_bytes_per_launch": hbm,
        "commands": [fcmd, wcmd],
    })
    print(f"{kind} {workload}: FETCH {fetch:.0f} KiB x {fetch_scale:.3f} + WRITE {write:.0f} KiB "
          f"x {write_scale:.3f} = {hbm / 1e6:.2f} MB per launch -> {os.path.relpath(path, ROOT)}")


def sq(argv):
    kind, workload, sdir, cmd = argv
    d = per_dispatch(sdir, _name_parts(kind))
    if not d:
        raise SystemExit(f"no {kind} dispatches in {sdir}")
    keys = sorted(set().union(*d.values()))
    avg = {k: sum(x.get(k, 0.0) for x in d.values()) / len(d) for k in keys}
    mops = sum(v for k, v in avg.items() if k.startswith("SQ_INSTS_VALU_MFMA_MOPS_"))
    flops = mops * MOPS_UNIT
    fields = {"sq_dispatches": len(d), "sq_counters_per_launch": avg, "sq_command": cmd,
              "mfma_flops_per_launch": flops if mops else None}
    lines = [f"{kind} {workload}: {len(d)} launches, counter window {avg['dur_us']:.1f} us",
             f"command: {cmd}"]
    lines += [f"  {k:32s} {v:18.0f}" for k, v in avg.items() if k != "dur_us"]
    if mops:
        lines.append(f"  executed MFMA flops per launch (MOPS x {MOPS_UNIT}): {flops:.4g}")
    if "GRBM_GUI_ACTIVE" in avg:
        cyc = avg["GRBM_GUI_ACTIVE"] / XCDS          # summed over the dies
        lines.append(f"  GRBM_GUI_ACTIVE per XCD {cyc:.0f} cycles = {cyc / avg['dur_us'] / 1e3:.2f} GHz "
                     "over the counter window")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * SIMDS)
            fields["mfma_busy_frac"] = busy
            lines.append(f"  MFMA busy fraction (busy cycles / (GRBM cycles per XCD x {SIMDS} SIMDs)):"
                         f" {busy:.3f}")
        if "SQ_INSTS_MFMA" in avg and "SQ_VALU_MFMA_BUSY_CYCLES" in avg and avg["SQ_INSTS_MFMA"]:
            lines.append(f"  busy cycles per MFMA instruction: "
                         f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / avg['SQ_INSTS_MFMA']:.1f}")
    path = _merge(kind, workload, fields)
    lines.append(f"  -> {os.path.relpath(path, ROOT)}")
    print("\n".join(lines))


if __name__ == "__main__":
    mode, rest = sys.argv[1], sys.argv[2:]
    {"traffic": traffic, "sq": sq}[mode](rest)
