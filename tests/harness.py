"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI,
run the fp64 oracle on the same seeded inputs, compare at the stated gates."""

import numpy as np
import torch

import oracle
import paged_kv_cache_314_amd as pa

# Gates (max-abs on out; lse relative): fp16 out 5e-3, bf16 out 2e-2 (also the int8-KV
# path, whose output is bf16 here), lse |d| <= 1e-3 * max(1, |lse_ref|).
OUT_TOL = {torch.float16: 5e-3, torch.bfloat16: 2e-2}
LSE_RTOL = 1e-3


def to_device(inp, device="cuda"):
    d = dict(inp)
    for k in ("query", "key", "value", "block_tables", "slopes", "key_scale", "value_scale",
              "key_offset", "value_offset"):
        if d.get(k) is not None:
            d[k] = d[k].to(device)
    return d


def gpu_run(inp, *, want_lse=True, out=None, lse=None, stream=None, keep_op=False):
    """Run the library on the inputs of ``inp`` (CPU tensors are moved to the GPU)."""
    g = to_device(inp)
    q = g["query"]
    if out is None:
        out = torch.full_like(q, float("nan"))
    if want_lse and lse is None:
        lse = torch.full((q.shape[0], g["head_num"]), float("nan"), dtype=torch.float32,
                         device=q.device)
    op = pa.pa_paged_attention_get_workspace_size_ex(
        q, g["key"], g["value"], g["block_tables"], None, g["seq_len"], g["kv_seq_len"],
        g["slopes"], g["mask_type"], g["head_num"], g["kv_head_num"], g["qk_scale"],
        g["key_scale"], g["value_scale"], g.get("key_offset"), g.get("value_offset"),
        g.get("key_mode", 0), g.get("value_mode", 0), out, lse if want_lse else None)
    ws = pa.alloc_workspace(op.workspace_size, q.device)
    pa.pa_paged_attention(ws, op.workspace_size, op, stream)
    torch.cuda.synchronize()
    if keep_op:
        return out, lse, op, ws
    op.destroy()
    return out, lse


def oracle_inputs(inp):
    key, value = inp["key"], inp["value"]
    kv_format = None
    if key.dtype == torch.int8:
        k = key.numpy().astype(np.int64)
        v = value.numpy().astype(np.int64)
    elif key.dtype == torch.float8_e4m3fn:
        # byte codes: the oracle decodes them itself
        k = key.view(torch.uint8).numpy().astype(np.int64)
        v = value.view(torch.uint8).numpy().astype(np.int64)
        kv_format = "e4m3fn"
    else:
        k = key.double().numpy()
        v = value.double().numpy()
    np64 = lambda name: inp[name].double().numpy() if inp.get(name) is not None else None
    aq = dict(ks=np64("key_scale"), vs=np64("value_scale"), ko=np64("key_offset"),
              vo=np64("value_offset"), kmode=inp.get("key_mode", 0),
              vmode=inp.get("value_mode", 0), kv_format=kv_format)
    return k, v, aq, np64("slopes")


def _dequant(x, b, scale, offset, mode):
    if scale is None:
        return x
    if mode == 0:
        return oracle.dequantize_per_channel(x, scale, offset)
    return oracle.dequantize_per_token(x, scale[b], None if offset is None else offset[b])


def oracle_run(inp, batches=None):
    """fp64 oracle result.  With ``batches`` only those sequences are computed; the
    function returns (out, lse, rows) where rows are the packed query rows covered."""
    k, v, aq, sl = oracle_inputs(inp)
    q = inp["query"].double().numpy()
    table = inp["block_tables"].numpy()
    ql = inp["seq_len"].numpy().astype(np.int64)
    kl = inp["kv_seq_len"].numpy().astype(np.int64)
    H, Hkv = inp["head_num"], inp["kv_head_num"]
    if batches is None:
        out, lse = oracle.paged_attention(
            q, k, v, table, ql, kl, inp["mask_type"], H, Hkv, inp["qk_scale"], slopes=sl,
            key_antiquant_scale=aq["ks"], value_antiquant_scale=aq["vs"],
            key_antiquant_offset=aq["ko"], value_antiquant_offset=aq["vo"],
            key_antiquant_mode=aq["kmode"], value_antiquant_mode=aq["vmode"],
            kv_format=aq["kv_format"])
        return out, lse, np.arange(q.shape[0])
    q0 = np.concatenate([[0], np.cumsum(ql)])
    bs = k.shape[1]
    outs, lses, rows = [], [], []
    for b in batches:
        kb = oracle.gather_sequence(k, table[b], kl[b], bs)
        vb = oracle.gather_sequence(v, table[b], kl[b], bs)
        if aq["kv_format"] == "e4m3fn":
            kb = oracle.decode_e4m3fn(kb)
            vb = oracle.decode_e4m3fn(vb)
        kb = _dequant(kb, b, aq["ks"], aq["ko"], aq["kmode"])
        vb = _dequant(vb, b, aq["vs"], aq["vo"], aq["vmode"])
        r = np.arange(q0[b], q0[b + 1])
        o, l = oracle.attention_contiguous(
            q[r], kb, vb, oracle.query_positions(ql[b], kl[b]), inp["mask_type"],
            inp["qk_scale"], H, Hkv, sl)
        outs.append(o)
        lses.append(l)
        rows.append(r)
    return np.concatenate(outs), np.concatenate(lses), np.concatenate(rows)


def compare(out_gpu, lse_gpu, out_ref, lse_ref, rows, out_dtype, label=""):
    """Assert the gates; return a dict of error statistics.  Every row of the GPU output
    (not only ``rows``) must be finite, and every lse must be finite or +inf."""
    full = out_gpu.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(full)), f"{label}: non-finite output"
    if lse_gpu is not None:
        lf = lse_gpu.cpu().numpy()
        assert np.all(np.isfinite(lf) | (lf == np.inf)), f"{label}: lse NaN or -inf"
    og = full[rows]
    tol = OUT_TOL[out_dtype]
    err = np.abs(og - out_ref)
    ref_max = float(np.max(np.abs(out_ref))) if out_ref.size else 0.0
    stats = {
        "max_abs": float(err.max()) if err.size else 0.0,
        "rms": float(np.sqrt(np.mean(err ** 2))) if err.size else 0.0,
        "ref_max": ref_max,
    }
    stats["normalized"] = stats["max_abs"] / ref_max if ref_max > 0 else 0.0
    assert stats["max_abs"] <= tol, f"{label}: out max-abs {stats['max_abs']:.3g} > {tol} ({stats})"
    # rows with no visible key: exactly 0 out and +inf lse
    empty = ~np.isfinite(lse_ref)
    if empty.any():
        assert np.all(og[empty] == 0.0), f"{label}: empty rows not zero"
    if lse_gpu is not None:
        lg = lse_gpu.cpu().numpy().astype(np.float64)[rows]
        assert np.array_equal(np.isinf(lg) & (lg > 0), empty), f"{label}: lse inf pattern"
        fin = ~empty
        if fin.any():
            d = np.abs(lg[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
            stats["lse_rel"] = float(d.max())
            assert stats["lse_rel"] <= LSE_RTOL, f"{label}: lse rel err {stats['lse_rel']:.3g}"
    return stats
