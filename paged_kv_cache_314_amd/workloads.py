"""Seeded synthetic inputs for paged attention.

This module only draws random inputs and lays them out (pool, block tables,
lengths, scales).  It holds none of the attention arithmetic, and it is the
one module that both the HIP path's tests/benchmark and the CPU oracle are
fed from.  Everything is returned as CPU torch tensors; callers move them to
the GPU themselves.

Named workloads (shapes of the five benchmark configurations):

  decode_f16_small   decode, fp16, B=2, H=Hkv=4, D=64, kvSeqLen=[256,200],
                     blockSize=16, 40 blocks, table [2,16], qkScale=1/8, lse
  prefill_causal_bf16  causal prefill, bf16, B=4, seqLen=kvSeqLen=512, H=32,
                     Hkv=8, D=128, blockSize=128, 16 shuffled blocks
  decode_bf16_batched  decode, bf16, B=64, kvSeqLen ~ U[1024, 8192], H=32,
                     Hkv=8, D=128, blockSize=128, pool = needed blocks + 10%, lse
  prefill_alibi_f16  prefix-encoder prefill with ALiBi, fp16, B=8, 512 new
                     tokens over kvSeqLen=2560, H=Hkv=32, D=128, blockSize=128,
                     slopes 2^(-8(h+1)/32)
  decode_int8_long   decode, bf16 Q/out, int8 K/V ~ U[-127,127], B=32,
                     kvSeqLen=16384, H=64, Hkv=8, D=128, blockSize=128,
                     per-channel fp32 scales ~ U[0.005, 0.02], pool +10%

Random draws use numpy.random.default_rng([314, k]) with k the workload's
index, in the order: query, key pool, value pool, block permutation, scales.
Random kv lengths come from the child generator default_rng([314, k, 1]) so
that they can size the pool before it is drawn.  Floats are drawn N(0,1) in
fp32 and rounded to fp16/bf16 (round to nearest even) by torch.
"""

import math
from dataclasses import dataclass, field

import numpy as np
import torch

MASK_NONE = 0
MASK_ALIBI = 3
MASK_CAUSAL = 9

_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8,
           "f8": torch.float8_e4m3fn}


@dataclass
class Workload:
    """Shape sheet of one workload."""
    name: str
    index: int
    dtype: str                  # query / out dtype: "f16" | "bf16"
    kv_dtype: str               # "f16" | "bf16" | "i8" | "f8"
    batch: int
    head_num: int
    kv_head_num: int
    head_size: int
    block_size: int
    seq_len: object             # int (same for every sequence) or "decode"
    kv_seq_len: object          # int, list of ints, or ("uniform", lo, hi)
    mask_type: int = MASK_NONE
    qk_scale: float = 1.0
    lse: bool = False
    alibi: bool = False
    pool: object = "exact"      # "exact", ("plus", 0.10) or an int block count
    table_width: object = None  # None = max blocks needed
    table_padding: str = "minus_one"   # "minus_one" | "ids"
    antiquant: object = None    # int8 only: (key mode, value mode, offsets?); None = (0, 0, False)
    op: str = "attention"       # "attention" | "append" (KV-cache append of the seqLen new tokens)
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "decode_f16_small": Workload(
        "decode_f16_small", 1, "f16", "f16", 2, 4, 4, 64, 16, "decode",
        [256, 200], MASK_NONE, 1.0 / 8.0, lse=True, pool=40, table_width=16,
        table_padding="ids"),
    "prefill_causal_bf16": Workload(
        "prefill_causal_bf16", 2, "bf16", "bf16", 4, 32, 8, 128, 128, 512, 512,
        MASK_CAUSAL, 1.0 / math.sqrt(128.0)),
    "decode_bf16_batched": Workload(
        "decode_bf16_batched", 3, "bf16", "bf16", 64, 32, 8, 128, 128, "decode",
        ("uniform", 1024, 8192), MASK_NONE, 1.0 / math.sqrt(128.0), lse=True,
        pool=("plus", 0.10)),
    "prefill_alibi_f16": Workload(
        "prefill_alibi_f16", 4, "f16", "f16", 8, 32, 32, 128, 128, 512, 2560,
        MASK_ALIBI, 1.0 / math.sqrt(128.0), alibi=True),
    "decode_int8_long": Workload(
        "decode_int8_long", 5, "bf16", "i8", 32, 64, 8, 128, 128, "decode", 16384,
        MASK_NONE, 1.0 / math.sqrt(128.0), pool=("plus", 0.10)),
    # the INT8 long decode with per-token scales and offsets on K and V (same shapes)
    # the INT8 long decode's shapes with a FLOAT8_E4M3FN cache and per-channel scales
    "decode_fp8_long": Workload(
        "decode_fp8_long", 7, "bf16", "f8", 32, 64, 8, 128, 128, "decode", 16384,
        MASK_NONE, 1.0 / math.sqrt(128.0), pool=("plus", 0.10)),
    # KV-cache append of the prefix + ALiBi prefill's new tokens (8 x 512 into 2560-token
    # sequences, 32 kv heads, f16): the step before that prefill
    "append_prefix_f16": Workload(
        "append_prefix_f16", 8, "f16", "f16", 8, 32, 32, 128, 128, 512, 2560,
        MASK_NONE, 1.0 / math.sqrt(128.0), op="append"),
    "decode_int8_pertoken_long": Workload(
        "decode_int8_pertoken_long", 6, "bf16", "i8", 32, 64, 8, 128, 128, "decode", 16384,
        MASK_NONE, 1.0 / math.sqrt(128.0), pool=("plus", 0.10), antiquant=(1, 1, True)),
}


def alibi_slopes(head_num):
    """Per-head ALiBi slopes 2^(-8(h+1)/headNum), the usual geometric series."""
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / head_num) for h in range(head_num)],
                        dtype=torch.float32)


def _normal(rng, shape, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(_DTYPES[dtype])


def _kv_pool(rng, shape, kv_dtype):
    if kv_dtype == "i8":
        return torch.from_numpy(rng.integers(-127, 128, size=shape, dtype=np.int8))
    if kv_dtype == "f8":
        # FLOAT8_E4M3FN codes of N(0, 64^2) values (clamped to the format's +-448), so
        # that the codes span the format's exponent range; RNE by torch
        x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(64.0)
        return torch.from_numpy(np.clip(x, -448.0, 448.0)).to(torch.float8_e4m3fn)
    return _normal(rng, shape, kv_dtype)


def antiquant_params(rng, kmode, vmode, offsets, kv_head_num, head_size, batch, kv_lens,
                     pad_cols=5):
    """Random int8 antiquant scales (and offsets): per-channel (mode 0) [Hkv, D] or
    per-token (mode 1) [batch, max(kv_lens) + pad_cols], fp32; scales U(0.005, 0.02),
    offsets U(-20, 20).  Returns (key_scale, value_scale, key_offset, value_offset)."""
    S = max([int(n) for n in kv_lens] + [0]) + pad_cols

    def draw(mode, lo, hi):
        shape = (kv_head_num, head_size) if mode == 0 else (batch, S)
        return torch.from_numpy(rng.uniform(lo, hi, size=shape).astype(np.float32))
    ks, vs = draw(kmode, 0.005, 0.02), draw(vmode, 0.005, 0.02)
    ko = draw(kmode, -20.0, 20.0) if offsets else None
    vo = draw(vmode, -20.0, 20.0) if offsets else None
    return ks, vs, ko, vo


def build_block_tables(rng, kv_lens, block_size, num_blocks, width, padding):
    """Hand out ceil(kvSeqLen/blockSize) ids of a random permutation per sequence."""
    need = [-(-int(n) // block_size) for n in kv_lens]
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((len(kv_lens), width), -1, dtype=np.int32)
    pos = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[pos:pos + nb]
        pos += nb
    if padding == "ids":
        for b, nb in enumerate(need):
            extra = width - nb
            take = perm[pos:pos + extra]
            if len(take) < extra:       # reuse ids (padding is never read)
                take = np.resize(perm, extra)
            table[b, nb:] = take
            pos += len(take)
    return torch.from_numpy(table)


def used_slots(block_tables, kv_lens, block_size, num_blocks):
    """Boolean [numBlocks, blockSize]: True where a slot holds a live token."""
    used = torch.zeros((num_blocks, block_size), dtype=torch.bool)
    for b, n in enumerate(kv_lens.tolist()):
        nb = -(-n // block_size)
        for i in range(nb):
            blk = int(block_tables[b, i])
            cnt = min(block_size, n - i * block_size)
            used[blk, :cnt] = True
    return used


def poison_unused(pool, used):
    """Fill every slot no sequence owns with NaN (float) or -128 (int8)."""
    mask = ~used
    if pool.dtype == torch.int8:
        pool[mask] = -128
    elif pool.dtype == torch.float8_e4m3fn:
        pool.view(torch.uint8)[mask] = 0x7F         # a NaN code
    else:
        pool[mask] = float("nan")
    return pool


def make_inputs(w, seed=None, poison=False, kv_lens=None, q_scale=1.0):
    """Draw the inputs of workload ``w`` (a Workload).

    Returns a dict with CPU tensors query, key, value, block_tables (int32),
    seq_len, kv_seq_len (int32, host), slopes (or None), key_scale /
    value_scale (fp32 or None) and the scalars mask_type, head_num,
    kv_head_num, qk_scale, want_lse.  ``poison`` fills unused pool slots with
    NaN / -128 so that a read of them shows up in the result.  ``q_scale``
    multiplies the drawn queries before rounding (high-contrast variants).
    """
    k = w.index if seed is None else seed
    rng = np.random.default_rng([314, k])
    B, H, Hkv, D, bs = w.batch, w.head_num, w.kv_head_num, w.head_size, w.block_size

    # query lengths are fixed per workload; they give the token count.
    if w.seq_len == "decode":
        q_lens_fixed = [1] * B
    else:
        q_lens_fixed = [int(w.seq_len)] * B
    n_tokens = sum(q_lens_fixed)

    q32 = rng.standard_normal(size=(n_tokens, H, D), dtype=np.float32) * np.float32(q_scale)
    query = torch.from_numpy(q32).to(_DTYPES[w.dtype])

    # kv lengths (possibly random) decide the pool size: draw them from a
    # child generator so that the pool draws keep their place in the order.
    len_rng = np.random.default_rng([314, k, 1])
    if kv_lens is not None:
        kvl = [int(x) for x in kv_lens]
    elif isinstance(w.kv_seq_len, tuple) and w.kv_seq_len[0] == "uniform":
        kvl = len_rng.integers(w.kv_seq_len[1], w.kv_seq_len[2] + 1, size=B).tolist()
    elif isinstance(w.kv_seq_len, list):
        kvl = list(w.kv_seq_len)
    else:
        kvl = [int(w.kv_seq_len)] * B
    need = sum(-(-n // bs) for n in kvl)
    if isinstance(w.pool, int):
        num_blocks = w.pool
    elif isinstance(w.pool, tuple):
        num_blocks = int(math.ceil(need * (1.0 + w.pool[1]) - 1e-9))
    else:
        num_blocks = need
    width = w.table_width or max(1, max(-(-n // bs) for n in kvl))

    key = _kv_pool(rng, (num_blocks, bs, Hkv, D), w.kv_dtype)
    value = _kv_pool(rng, (num_blocks, bs, Hkv, D), w.kv_dtype)
    tables = build_block_tables(rng, kvl, bs, num_blocks, width, w.table_padding)
    key_scale = value_scale = key_offset = value_offset = None
    kmode, vmode, offs = w.antiquant or (0, 0, False)
    if w.kv_dtype in ("i8", "f8") and w.antiquant is None:
        key_scale = torch.from_numpy(rng.uniform(0.005, 0.02, size=(Hkv, D)).astype(np.float32))
        value_scale = torch.from_numpy(rng.uniform(0.005, 0.02, size=(Hkv, D)).astype(np.float32))
    elif w.kv_dtype == "i8":
        key_scale, value_scale, key_offset, value_offset = antiquant_params(
            rng, kmode, vmode, offs, Hkv, D, B, kvl)
    seq_len = torch.tensor(q_lens_fixed, dtype=torch.int32)
    kv_seq_len = torch.tensor(kvl, dtype=torch.int32)
    extra = {}
    if w.op == "append":
        # the new tokens' K/V rows [nTokens, kvHeadNum, headSize]
        extra["key_new"] = _kv_pool(rng, (n_tokens, Hkv, D), w.kv_dtype)
        extra["value_new"] = _kv_pool(rng, (n_tokens, Hkv, D), w.kv_dtype)
    if poison:
        used = used_slots(tables, kv_seq_len, bs, num_blocks)
        poison_unused(key, used)
        poison_unused(value, used)
    return dict(
        query=query, key=key, value=value, block_tables=tables,
        seq_len=seq_len, kv_seq_len=kv_seq_len,
        slopes=alibi_slopes(H) if w.alibi else None,
        key_scale=key_scale, value_scale=value_scale,
        key_offset=key_offset, value_offset=value_offset, key_mode=kmode, value_mode=vmode,
        mask_type=w.mask_type, head_num=H, kv_head_num=Hkv,
        qk_scale=float(w.qk_scale), want_lse=bool(w.lse), **extra,
    )


def make_random_case(seed, *, batch, head_num, kv_head_num, head_size, block_size,
                     q_lens, kv_lens, dtype="bf16", kv_dtype=None, mask_type=MASK_NONE,
                     qk_scale=None, extra_blocks=3, poison=True, q_scale=1.0,
                     table_extra_cols=1, antiquant=None):
    """Small random case with explicit per-sequence lengths (parity tests).

    The pool has the needed blocks plus ``extra_blocks`` spare ones, handed
    out in a random permutation; unused table entries are -1 and unused slots
    are poisoned when ``poison``.
    """
    kv_dtype = kv_dtype or dtype
    rng = np.random.default_rng([314, 1000 + seed])
    H, Hkv, D, bs = head_num, kv_head_num, head_size, block_size
    n_tokens = int(sum(q_lens))
    q32 = rng.standard_normal(size=(n_tokens, H, D), dtype=np.float32) * np.float32(q_scale)
    query = torch.from_numpy(q32).to(_DTYPES[dtype])
    need = sum(-(-int(n) // bs) for n in kv_lens)
    num_blocks = need + extra_blocks
    width = max(1, max(-(-int(n) // bs) for n in kv_lens)) + table_extra_cols
    key = _kv_pool(rng, (num_blocks, bs, Hkv, D), kv_dtype)
    value = _kv_pool(rng, (num_blocks, bs, Hkv, D), kv_dtype)
    tables = build_block_tables(rng, kv_lens, bs, num_blocks, width, "minus_one")
    key_scale = value_scale = key_offset = value_offset = None
    kmode, vmode, offs = antiquant or (0, 0, False)
    if kv_dtype in ("i8", "f8") and antiquant is None:
        key_scale = torch.from_numpy(rng.uniform(0.005, 0.02, size=(Hkv, D)).astype(np.float32))
        value_scale = torch.from_numpy(rng.uniform(0.005, 0.02, size=(Hkv, D)).astype(np.float32))
    elif kv_dtype == "i8":
        key_scale, value_scale, key_offset, value_offset = antiquant_params(
            rng, kmode, vmode, offs, Hkv, D, len(kv_lens), kv_lens)
    seq_len = torch.tensor([int(x) for x in q_lens], dtype=torch.int32)
    kv_seq_len = torch.tensor([int(x) for x in kv_lens], dtype=torch.int32)
    if poison and num_blocks > 0:
        used = used_slots(tables, kv_seq_len, bs, num_blocks)
        poison_unused(key, used)
        poison_unused(value, used)
    slopes = None
    if mask_type == MASK_ALIBI:
        slopes = torch.from_numpy(rng.uniform(0.0, 1.0, size=H).astype(np.float32))
    if qk_scale is None:
        qk_scale = 1.0 / math.sqrt(D)
    return dict(
        query=query, key=key, value=value, block_tables=tables,
        seq_len=seq_len, kv_seq_len=kv_seq_len, slopes=slopes,
        key_scale=key_scale, value_scale=value_scale,
        key_offset=key_offset, value_offset=value_offset, key_mode=kmode, value_mode=vmode,
        mask_type=mask_type, head_num=H, kv_head_num=Hkv,
        qk_scale=float(qk_scale), want_lse=True,
    )
