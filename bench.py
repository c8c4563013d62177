"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--kv-layout bnbsh|bnnbsd] [--no-cpu-baseline] [--copy-probe MiB]

A step is one execute of the planned operator (pa_paged_attention): every kernel of
the path, over one batch of seeded synthetic inputs already resident in HBM.  The K timed steps are captured into one HIP
graph and replayed as a single launch (the replay is checked bit for bit against the
eager result); the same K steps launched one by one from the host are reported as
``ms_per_step_eager``.  Without --warmup, the untimed warmup runs for WARMUP_SECONDS
(at least 10 steps) so that the GPU clock has ramped up.  Prints ONE JSON line.

Default (no --workload): the metric on the largest single-GPU configurations.  The
headline ``value`` is the batched decode (bf16, B=64, kvSeqLen ~ U[1024, 8192], H=32,
Hkv=8, D=128, blockSize=128, lse; "decode_bf16_batched") in GB/s; the same line
carries, under ``workloads``, the ALiBi prefix prefill (fp16, B=8, 512 new tokens over
2560, H=Hkv=32; "prefill_alibi_f16") in TFLOP/s and the long INT8-KV decode (B=32,
kvSeqLen=16384, H=64, Hkv=8; "decode_int8_long") in GB/s in both cache layouts, each
with its own roofline and CPU baseline.  --workload NAME measures one named workload.

Throughput: prefill workloads report algorithmic TFLOP/s (4*D flops per visible
(query, key) pair, exact causal count); decode workloads report algorithmic GB/s
(K/V bytes of the valid tokens + Q + out + lse + used block-table entries +
antiquant scales).  ``roofline`` covers the op's kernels (decode: the decode kernel and
the split-KV combine; prefill: the prefill kernel), timed with HIP events attached to
the first kernel's dispatch and the last one's, over K executes made right after the
warmup (mean, and p10 / median / p90), back to back (warm caches) and, under
``roofline.cold``, after a 1 GiB read before each execute (cold caches); prefill is
also given against the HBM roof under ``roofline.hbm_view``, and with the MFMA work
the kernel executed (from rocprofv3 counters) under ``roofline.executed``.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, GB/s
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}   # dense MFMA, published
# default warmup length: MFMA-heavy kernels run several percent slower during the first
# tens of milliseconds on an idle GPU (measured: ALiBi prefix prefill 218 us per step
# after 10 warmup steps, 193 us after 300)
WARMUP_SECONDS = 0.5
FLUSH_MIB = 1024                 # cache flush before each cold launch (256 MB MALL + L2s)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=-1,
                    help="untimed warmup steps; default: as many as fill %.1f s (at least 10), "
                         "so that the GPU clock has ramped up before timing" % WARMUP_SECONDS)
    ap.add_argument("--workload", default=None,
                    help="measure one named workload (default: the batched decode as the "
                         "headline, with the ALiBi prefix prefill and the long INT8-KV decode "
                         "in both cache layouts in the same line)")
    ap.add_argument("--kv-layout", choices=["bnbsh", "bnnbsd"], default="bnbsh",
                    help="K/V pool memory layout: (block, slot, kv head, d) as the workload "
                         "defines it, or (block, kv head, slot, d) passed as a strided view")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU budget of the oracle baseline sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MiB",
                    help="only run a plain device copy of this size (counter calibration)")
    return ap.parse_args()


# ------------------------------------------------------------------ counts

def algorithmic_counts(inp):
    """(bytes, flops) of one step, from the definition of the operation."""
    import numpy as np
    q, k = inp["query"], inp["key"]
    T, H, D = q.shape
    Hkv = inp["kv_head_num"]
    bs = k.shape[1]
    ql = inp["seq_len"].numpy().astype(np.int64)
    kl = inp["kv_seq_len"].numpy().astype(np.int64)
    kv_elt = k.element_size()
    q_elt = q.element_size()
    causal = inp["mask_type"] in (3, 9)
    pairs = 0
    for a, b in zip(ql, kl):
        if causal:
            p = b - a + np.arange(a)            # absolute positions
            pairs += int(np.sum(np.clip(np.minimum(p, b - 1) + 1, 0, None)))
        else:
            pairs += int(a * b)
    flops = 4 * D * H * pairs
    kv_bytes = int(np.sum(kl)) * Hkv * D * kv_elt * 2
    qo_bytes = 2 * T * H * D * q_elt
    lse_bytes = T * H * 4 if inp["want_lse"] else 0
    table_bytes = int(np.sum((kl + bs - 1) // bs)) * 4
    # antiquant parameters: the whole per-channel tensors, or the per-token entries of
    # the valid tokens
    scale_bytes = 0
    for name, mode in (("key_scale", "key_mode"), ("value_scale", "value_mode"),
                       ("key_offset", "key_mode"), ("value_offset", "value_mode")):
        if inp.get(name) is None:
            continue
        per_token = inp.get(mode, 0) == 1
        scale_bytes += (int(np.sum(kl)) if per_token else Hkv * D) * 4
    nbytes = kv_bytes + qo_bytes + lse_bytes + table_bytes + scale_bytes
    return nbytes, flops


def counters_from_profiles(workload, kernel):
    """The rocprofv3 counter summary of ``kernel`` on ``workload`` under profiles/, if
    one exists and was taken on the current kernel sources; else None."""
    from paged_kv_cache_314_amd.counter_summary import kernel_source_hash
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    return d


def traffic_from_profiles(workload, kernels):
    """HBM bytes per execute measured with rocprofv3 counters (FETCH_SIZE, WRITE_SIZE),
    summed over ``kernels``, if every summary exists and was taken on the current
    kernel sources; else None."""
    total = 0.0
    for k in kernels:
        d = counters_from_profiles(workload, k)
        if d is None or d.get("hbm_bytes_per_launch") is None:
            return None
        total += d["hbm_bytes_per_launch"]
    return total


# ------------------------------------------------------------ cpu baseline

def cpu_baseline(inp, nbytes, flops, decode, budget_s):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload:
    whole sequences, one after another (starting again at the first after the last),
    until the time budget is spent."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle
    q = inp["query"].double().numpy()
    np64 = lambda name: inp[name].double().numpy() if inp.get(name) is not None else None
    fp8 = inp["key"].dtype == torch.float8_e4m3fn
    if fp8:
        k = inp["key"].view(torch.uint8).numpy()
        v = inp["value"].view(torch.uint8).numpy()
    elif inp["key"].dtype.is_floating_point:
        k = inp["key"].double().numpy()
        v = inp["value"].double().numpy()
    else:
        k = inp["key"].numpy()
        v = inp["value"].numpy()
    ks, vs, ko, vo = np64("key_scale"), np64("value_scale"), np64("key_offset"), np64("value_offset")
    kmode, vmode = inp.get("key_mode", 0), inp.get("value_mode", 0)

    def dequant(x, b, scale, offset, mode):
        if scale is None:
            return x
        if mode == 0:
            return oracle.dequantize_per_channel(x, scale, offset)
        return oracle.dequantize_per_token(x, scale[b], None if offset is None else offset[b])
    sl = inp["slopes"].double().numpy() if inp["slopes"] is not None else None
    table = inp["block_tables"].numpy()
    ql = inp["seq_len"].numpy().astype(np.int64)
    kl = inp["kv_seq_len"].numpy().astype(np.int64)
    q0 = np.concatenate([[0], np.cumsum(ql)])
    H, Hkv = inp["head_num"], inp["kv_head_num"]
    bs = k.shape[1]
    done_units = 0.0
    total_units = 0.0
    for b in range(len(ql)):
        total_units += ql[b] * kl[b] if not decode else kl[b]
    t0 = time.perf_counter()
    nseq = 0
    # whole sequences in order, wrapping round to the first one, until the budget is spent
    for i in range(1 << 30):
        b = i % len(ql)
        kb = oracle.gather_sequence(k, table[b], kl[b], bs)
        vb = oracle.gather_sequence(v, table[b], kl[b], bs)
        if fp8:
            kb, vb = oracle.decode_e4m3fn(kb), oracle.decode_e4m3fn(vb)
        kb = dequant(kb, b, ks, ko, kmode)
        vb = dequant(vb, b, vs, vo, vmode)
        oracle.attention_contiguous(q[q0[b]:q0[b + 1]], kb, vb,
                                    oracle.query_positions(ql[b], kl[b]), inp["mask_type"],
                                    inp["qk_scale"], H, Hkv, sl)
        nseq += 1
        done_units += ql[b] * kl[b] if not decode else kl[b]
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    frac = done_units / total_units if total_units else 1.0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    cores = len(os.sched_getaffinity(0))
    if decode:
        value, unit = nbytes * frac / dt / 1e9, "GB/s"
    else:
        value, unit = flops * frac / dt / 1e12, "TFLOP/s"
    return {"value": value, "unit": unit, "cores": int(min(threads, cores)), "kind": "oracle",
            "host_cores": cores, "blas_threads": int(threads),
            "sample": f"{nseq} sequences (all heads) taken in order from the step's "
                      f"{len(ql)}, {frac:.3f} times the step's work, {dt:.1f} s, fp64 NumPy "
                      f"(BLAS threads {threads} on {cores} host cores)"}


def warmup(args, step):
    """Run the untimed warmup steps: exactly --warmup W if given, else at least 10 and
    until WARMUP_SECONDS have passed.  Returns the number run."""
    import torch
    if args.warmup >= 0:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        return args.warmup
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= WARMUP_SECONDS:
            return n


# ------------------------------------------------------------ kernel timing

def time_kernels(op, run, stream, n, combine, before=None):
    """Durations (ms) of the op's kernels over ``n`` executes, from HIP events attached to
    each kernel's own dispatch: (main kernel list, split-KV combine list or None).
    ``before`` (optional) runs ahead of every execute, outside the timed kernels."""
    import torch

    import paged_kv_cache_314_amd as pa
    kinds = [pa.PA_TIMED_MAIN] + ([pa.PA_TIMED_COMBINE] if combine else [])
    ev = {k: ([torch.cuda.Event(enable_timing=True) for _ in range(n)],
              [torch.cuda.Event(enable_timing=True) for _ in range(n)]) for k in kinds}
    for starts, stops in ev.values():
        for e in starts + stops:
            e.record(stream)       # torch creates its events on first use
    torch.cuda.synchronize()
    for i in range(n):
        if before is not None:
            before()
        for k in kinds:
            pa.pa_op_set_timing_events(op, ev[k][0][i], ev[k][1][i], kernel=k)
        run(stream)
    for k in kinds:
        pa.pa_op_set_timing_events(op, None, None, kernel=k)
    torch.cuda.synchronize()
    out = [[s.elapsed_time(e) for s, e in zip(*ev[k])] for k in kinds]
    return out[0], (out[1] if combine else None)


# ------------------------------------------------------------ KV-cache append

def bench_append(args, w, dev):
    """Time the KV-cache append of workload ``w`` (HBM-bound copy: the new rows are read
    and written once; bytes = 2 x (K + V) x nTokens x kvHeadNum x headSize x element)."""
    import numpy as np
    import torch

    import paged_kv_cache_314_amd as pa
    from paged_kv_cache_314_amd import workloads as wl

    inp = wl.make_inputs(w, poison=False)
    kn, vn = inp["key_new"].to(dev), inp["value_new"].to(dev)
    kc, vc = inp["key"].to(dev), inp["value"].to(dev)
    if args.kv_layout == "bnnbsd":
        kc = kc.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        vc = vc.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    table = inp["block_tables"].to(dev)
    nbytes = 2 * 2 * kn.numel() * kn.element_size()
    pa.load()
    first = pa.pa_kv_cache_append_plan(kn, vn, kc, vc, table, inp["seq_len"], inp["kv_seq_len"])
    first.destroy()
    t_plan = time.perf_counter()
    op = pa.pa_kv_cache_append_plan(kn, vn, kc, vc, table, inp["seq_len"], inp["kv_seq_len"])
    plan_us = (time.perf_counter() - t_plan) * 1e6
    info = pa.pa_op_describe(op)
    stream = torch.cuda.current_stream()
    run = lambda st: pa.pa_kv_cache_append(op, st)
    args.warmup = warmup(args, lambda: run(stream))
    # kernel events first after the warmup, then the graph-timed steps, then eager (as
    # for the attention workloads)
    kms, _ = time_kernels(op, run, stream, args.steps, False)
    kernel_ms = sum(kms) / len(kms)
    ref_k, ref_v = kc.clone(), vc.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for _ in range(args.steps):
            run(cap)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    if not (torch.equal(kc, ref_k) and torch.equal(vc, ref_v)):
        raise RuntimeError("graph replay of the append differs from the eager result")
    del graph, ref_k, ref_v
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run(stream)
    torch.cuda.synchronize()
    ms_per_step_eager = (time.perf_counter() - t0) * 1e3 / args.steps
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic_from_profiles(args.workload, ["append_kernel"]),
            "kernel": "append_kernel", "kernel_us": kernel_ms * 1e3, "algorithmic_bytes": nbytes,
            "algorithmic_flops": 0}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_info
        raw = lambda t: t.contiguous().view(torch.uint8).numpy()
        table_np = inp["block_tables"].numpy()
        ql, kl = inp["seq_len"].tolist(), inp["kv_seq_len"].tolist()
        kraw, vraw = raw(inp["key"]), raw(inp["value"])
        knew, vnew = raw(inp["key_new"]), raw(inp["value_new"])
        # the whole append (K and V), repeated until the time budget is spent
        reps = 0
        tc = time.perf_counter()
        while reps == 0 or time.perf_counter() - tc < args.cpu_seconds:
            oracle.append_kv_rows(kraw, knew, table_np, ql, kl)
            oracle.append_kv_rows(vraw, vnew, table_np, ql, kl)
            reps += 1
        dt = time.perf_counter() - tc
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        cpu = {"value": reps * nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
               "host_cores": len(os.sched_getaffinity(0)), "blas_threads": int(threads),
               "sample": f"the whole append (K and V, {len(ql)} sequences) {reps} times, "
                         f"{dt:.1f} s, NumPy row copies (one thread; BLAS threads {threads} "
                         f"unused)"}
    result = {
        "metric": "decode HBM GB/s (% peak) + prefill TFLOP/s (% MFMA peak), paged attention",
        "value": nbytes / (ms_per_step * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "launch": "one HIP graph of the K steps", "ms_per_step_eager": ms_per_step_eager,
        "dtype": w.kv_dtype, "data": "synthetic",
        "config": {"workload": args.workload, "mode": "append", "batch": w.batch,
                   "kv_head_num": w.kv_head_num, "head_size": w.head_size,
                   "block_size": w.block_size, "kv_dtype": w.kv_dtype, "new_tokens": int(kn.shape[0]),
                   "kv_layout": args.kv_layout, "parallelism": "single GPU",
                   "work_items": len(info["append_items"])},
        "plan_us": plan_us, "roofline": roof, "cpu_baseline": cpu,
    }
    op.destroy()
    print(json.dumps(result), flush=True)


# -------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the hot path is a "
              "single-GPU kernel and no multi-GPU figure is produced.", file=sys.stderr)
        sys.exit(2)
    import torch

    import paged_kv_cache_314_amd as pa
    from paged_kv_cache_314_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.copy_probe:
        n = args.copy_probe * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": max(args.steps, 1)}))
        return

    if args.workload is not None and wl.WORKLOADS[args.workload].op == "append":
        return bench_append(args, wl.WORKLOADS[args.workload], dev)
    if args.workload is not None:
        r = measure(args, args.workload, args.kv_layout, dev,
                    None if args.no_cpu_baseline else args.cpu_seconds)
        print(json.dumps(headline(args, r)), flush=True)
        return
    # default: the batched decode is the headline; the ALiBi prefix prefill and the long
    # INT8-KV decode (both cache layouts) ride along in the same line
    cpu = lambda t: None if args.no_cpu_baseline else t
    head = measure(args, HEADLINE, "bnbsh", dev, cpu(args.cpu_seconds))
    line = headline(args, head)
    line["workloads"] = {}
    for name, layout in ALSO:
        r = measure(args, name, layout, dev, cpu(SECONDARY_CPU_SECONDS))
        key = name if layout == "bnbsh" else f"{name}@{layout}"
        line["workloads"][key] = {k: r[k] for k in (
            "value", "unit", "ms_per_step", "ms_per_step_eager", "dtype", "config", "plan_us",
            "plan_us_first", "roofline", "cpu_baseline")}
    print(json.dumps(line), flush=True)


HEADLINE = "decode_bf16_batched"
ALSO = [("prefill_alibi_f16", "bnbsh"), ("decode_int8_long", "bnbsh"),
        ("decode_int8_long", "bnnbsd")]
SECONDARY_CPU_SECONDS = 5.0


def headline(args, r):
    """The driver's JSON line for one measured workload ``r``."""
    return {
        "metric": "decode HBM GB/s (% peak) + prefill TFLOP/s (% MFMA peak), paged attention",
        "value": r["value"],
        "unit": r["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": r["warmup"],
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "launch": "one HIP graph of the K steps",
        "ms_per_step_eager": r["ms_per_step_eager"],
        "dtype": r["dtype"],
        "data": "synthetic",
        "config": r["config"],
        "plan_us": r["plan_us"],
        "plan_us_first": r["plan_us_first"],
        "roofline": r["roofline"],
        "cpu_baseline": r["cpu_baseline"],
    }


def measure(args, name, layout, dev, cpu_seconds):
    """Plan, warm up and time workload ``name`` (K graph-replayed steps, K eager steps,
    K event-timed executes warm and up to 20 cold); returns its figures."""
    import torch

    import paged_kv_cache_314_amd as pa
    from paged_kv_cache_314_amd import workloads as wl

    w = wl.WORKLOADS[name]
    decode = w.seq_len == "decode"
    kind = "decode" if decode else "prefill"
    inp = wl.make_inputs(w, poison=False)
    nbytes, flops = algorithmic_counts(inp)
    g = {key: (val.to(dev) if isinstance(val, torch.Tensor) and key not in ("seq_len", "kv_seq_len")
               else val) for key, val in inp.items()}
    if layout == "bnnbsd":
        for key in ("key", "value"):
            g[key] = g[key].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    out = torch.empty_like(g["query"])
    lse = (torch.empty((out.shape[0], w.head_num), dtype=torch.float32, device=dev)
           if w.lse else None)

    def plan():
        return pa.pa_paged_attention_get_workspace_size_ex(
            g["query"], g["key"], g["value"], g["block_tables"], None, g["seq_len"],
            g["kv_seq_len"], g["slopes"], g["mask_type"], g["head_num"], g["kv_head_num"],
            g["qk_scale"], g["key_scale"], g["value_scale"], g.get("key_offset"),
            g.get("value_offset"), g.get("key_mode", 0), g.get("value_mode", 0), out, lse)

    # phase 1 twice: the first call (library already loaded) may take a fresh pinned
    # buffer for the work lists; the second, warm one is what a serving loop pays per step
    pa.load()
    t_plan = time.perf_counter()
    first = plan()
    plan_us_first = (time.perf_counter() - t_plan) * 1e6
    first.destroy()
    t_plan = time.perf_counter()
    op = plan()
    plan_us = (time.perf_counter() - t_plan) * 1e6
    ws = pa.alloc_workspace(op.workspace_size, dev)
    info = pa.pa_op_describe(op)
    stream = torch.cuda.current_stream()
    run = lambda st: pa.pa_paged_attention(ws, op.workspace_size, op, st)

    n_warm = warmup(args, lambda: run(stream))

    # the warmup's result: every later execute must reproduce it bit for bit
    torch.cuda.synchronize()
    ref_out = out.clone()
    ref_lse = lse.clone() if lse is not None else None

    # kernel durations: HIP events attached to the dispatch of each of the op's kernels,
    # taken first after the warmup (the GPU's clock drifts under long runs of
    # back-to-back launches; rocprofv3's kernel averages of the same command are taken in
    # this state).  The op's kernel time is the sum of its kernels' mean durations.
    has_combine = len(info["combine_items"]) > 0
    kms, cms = time_kernels(op, run, stream, args.steps, has_combine)
    main_ms = sum(kms) / len(kms)
    combine_ms = sum(cms) / len(cms) if cms else 0.0
    kernel_ms = main_ms + combine_ms

    # timed region: K whole steps, captured once into a HIP graph and replayed as one
    # launch (no host work between steps)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for _ in range(args.steps):
            run(cap)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    if not torch.equal(out, ref_out) or (lse is not None and not torch.equal(lse, ref_lse)):
        raise RuntimeError(f"{name}: graph replay of the execute differs from the eager result")
    del graph

    # the same K steps launched one by one from the host (reported beside the graph)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run(stream)
    torch.cuda.synchronize()
    ms_per_step_eager = (time.perf_counter() - t0) * 1e3 / args.steps

    # the same kernels from cold caches: a read of a FLUSH_MIB buffer (larger than the
    # 256 MB Infinity Cache and the L2s together) runs on the stream before each execute
    nc = min(args.steps, 20)
    flush = torch.ones(FLUSH_MIB << 18, dtype=torch.float32, device=dev)
    ck, cc = time_kernels(op, run, stream, nc, has_combine, before=lambda: flush.sum())
    cold_ms = sum(ck) / nc + (sum(cc) / nc if cc else 0.0)
    del flush

    kernels = [f"{kind}_kernel"] + (["combine_kernel"] if has_combine else [])
    if decode:
        value = nbytes / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        achieved = nbytes / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
        dtype = "f16" if w.kv_dtype in ("i8", "f8") else w.dtype   # one-byte caches run in f16
    else:
        value = flops / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        achieved = flops / (kernel_ms * 1e-3) / 1e12
        peak = PEAK_MFMA_TFLOPS[w.dtype]
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak}
        dtype = w.dtype
    roof["traffic"] = traffic_from_profiles(name if layout == "bnbsh" else f"{name}@{layout}",
                                            kernels)
    roof["kernel"] = "+".join(kernels)
    roof["kernel_us"] = kernel_ms * 1e3
    if has_combine:
        roof["kernel_us_each"] = {f"{kind}_kernel": main_ms * 1e3, "combine_kernel": combine_ms * 1e3}
    tot = sorted(a + b for a, b in zip(kms, cms)) if cms else sorted(kms)
    pick = lambda f: tot[int(round(f * (len(tot) - 1)))] * 1e3
    roof["kernel_us_p10_median_p90"] = [pick(0.1), pick(0.5), pick(0.9)]
    work = nbytes / 1e9 if decode else flops / 1e12
    roof["cold"] = {"kernel_us": cold_ms * 1e3, "achieved": work / (cold_ms * 1e-3),
                    "frac": work / (cold_ms * 1e-3) / roof["peak"], "launches": nc,
                    "flush": f"read of {FLUSH_MIB} MiB before each execute"}
    if not decode:
        # the same launch against the HBM roof: a prefill whose flops per algorithmic
        # byte fall below the ridge (2.5 PFLOP/s / 8 TB/s = 312.5) is bound by HBM first
        ai = flops / nbytes
        hbm = nbytes / (kernel_ms * 1e-3) / 1e9
        roof["hbm_view"] = {"achieved": hbm, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": hbm / PEAK_HBM_GBS, "flop_per_byte": ai,
                            "ridge_flop_per_byte": peak * 1e12 / (PEAK_HBM_GBS * 1e9),
                            "roof_tflops": min(peak, ai * PEAK_HBM_GBS / 1e3)}
        # the MFMA work the kernel executed (it skips the P V of tiles whose weights are
        # negligible under ALiBi, and adds the rank-1 bias products), from counters
        sq = counters_from_profiles(name, "prefill_kernel")
        if sq is not None and sq.get("mfma_flops_per_launch"):
            ex = sq["mfma_flops_per_launch"]
            roof["executed"] = {"flops": ex, "algorithmic_flops": flops, "ratio": ex / flops,
                                "achieved": ex / (kernel_ms * 1e-3) / 1e12,
                                "frac": ex / (kernel_ms * 1e-3) / 1e12 / peak,
                                "mfma_busy_frac": sq.get("mfma_busy_frac"),
                                "source": "rocprofv3 SQ counters under profiles/"}
        else:
            roof["executed"] = None
    roof["algorithmic_bytes"] = nbytes
    roof["algorithmic_flops"] = flops

    cpu = None
    if cpu_seconds is not None:
        cpu = cpu_baseline(inp, nbytes, flops, decode, cpu_seconds)
    op.destroy()
    return {
        "value": value, "unit": unit, "warmup": n_warm, "ms_per_step": ms_per_step,
        "ms_per_step_eager": ms_per_step_eager, "dtype": dtype, "plan_us": plan_us,
        "plan_us_first": plan_us_first, "roofline": roof, "cpu_baseline": cpu,
        "config": {
            "workload": name, "mode": kind, "batch": w.batch,
            "head_num": w.head_num, "kv_head_num": w.kv_head_num, "head_size": w.head_size,
            "block_size": w.block_size, "q_dtype": w.dtype, "kv_dtype": w.kv_dtype,
            "mask_type": w.mask_type, "lse": w.lse, "kv_layout": layout,
            "parallelism": "single GPU",
            "work_items": len(info["decode_items"]) + len(info["prefill_items"]),
            "combine_items": len(info["combine_items"]),
        },
    }


if __name__ == "__main__":
    main()
