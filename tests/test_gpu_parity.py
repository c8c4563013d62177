"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Inputs come from paged_kv_cache_314_amd.workloads (seeded, synthetic).  Unused
pool slots are NaN (-128 for int8) and unused table entries -1 unless stated,
so a read of memory the method must not touch shows up as a failure.
"""

import os
import sys

import numpy as np
import pytest

import oracle
import torch

import paged_kv_cache_314_amd as pa
from paged_kv_cache_314_amd import workloads as wl
from tests.harness import compare, gpu_run, oracle_run

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.load()
    yield


# ----------------------------------------------------------- named workloads

@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_named_workload_parity(name):
    """Every sequence, head and row of each full-size workload against the oracle."""
    w = wl.WORKLOADS[name]
    _say(f"[parity] {name}")
    if w.op == "append":
        # the whole cache after the append, byte for byte against the oracle
        inp = wl.make_inputs(w, poison=True)
        kc, vc = inp["key"].cuda(), inp["value"].cuda()
        pa.kv_cache_append(inp["key_new"].cuda(), inp["value_new"].cuda(), kc, vc,
                           inp["block_tables"].cuda(), inp["seq_len"], inp["kv_seq_len"])
        raw = lambda t: t.cpu().contiguous().view(torch.uint8).numpy()
        ql, kl = inp["seq_len"].tolist(), inp["kv_seq_len"].tolist()
        for cache, pool, new in ((kc, inp["key"], inp["key_new"]),
                                 (vc, inp["value"], inp["value_new"])):
            want = oracle.append_kv_rows(raw(pool), raw(new), inp["block_tables"].numpy(), ql, kl)
            assert np.array_equal(raw(cache), want)
        return
    inp = wl.make_inputs(w, poison=True)
    out, lse = gpu_run(inp, want_lse=True)
    ro, rl, rows = oracle_run(inp)
    assert len(rows) == out.shape[0]
    st = compare(out, lse, ro, rl, rows, inp["query"].dtype, name)
    _say(f"[parity] {name} {st}")


@pytest.mark.parametrize("name", ["decode_bf16_batched", "decode_int8_long",
                                  "decode_int8_pertoken_long", "decode_fp8_long"])
def test_high_contrast_decode(name):
    """Queries x4 sharpen the softmax so the 2e-2 bf16 gate bites harder (every
    sequence of the workload)."""
    w = wl.WORKLOADS[name]
    _say(f"[parity] {name} high-contrast")
    inp = wl.make_inputs(w, poison=True, q_scale=4.0)
    out, lse = gpu_run(inp)
    ro, rl, rows = oracle_run(inp)
    st = compare(out, lse, ro, rl, rows, inp["query"].dtype, name + "-x4")
    _say(f"[parity] {name} x4 {st}")


def test_decode_is_deterministic():
    w = wl.WORKLOADS["decode_bf16_batched"]
    inp = wl.make_inputs(w)
    a_out, a_lse = gpu_run(inp)
    b_out, b_lse = gpu_run(inp)
    assert torch.equal(a_out.view(torch.int16), b_out.view(torch.int16))
    assert torch.equal(a_lse, b_lse)


def test_prefill_is_deterministic():
    w = wl.WORKLOADS["prefill_causal_bf16"]
    inp = wl.make_inputs(w)
    a_out, a_lse = gpu_run(inp)
    b_out, b_lse = gpu_run(inp)
    assert torch.equal(a_out.view(torch.int16), b_out.view(torch.int16))
    assert torch.equal(a_lse, b_lse)


def test_alibi_far_tiles_are_deterministic():
    """The far-tile bound takes data-dependent branches (which tiles are computed); two
    runs on the same inputs, one of them with a dominant key in a far tile, still give
    bitwise equal results."""
    inp = wl.make_random_case(977, batch=2, head_num=4, kv_head_num=2, head_size=128,
                              block_size=64, q_lens=[200, 70], kv_lens=[3200, 3070],
                              dtype="f16", mask_type=pa.PA_MASK_ALIBI)
    inp["slopes"] = torch.full((4,), 0.5, dtype=torch.float32)
    u = torch.full((128,), 1.0 / 128 ** 0.5)
    blk = int(inp["block_tables"][1, 300 // 64])
    inp["key"][blk, 300 % 64] = (400.0 * u).to(inp["key"].dtype)
    a_out, a_lse = gpu_run(inp, want_lse=True)
    b_out, b_lse = gpu_run(inp, want_lse=True)
    assert torch.equal(a_out.view(torch.int16), b_out.view(torch.int16))
    assert torch.equal(a_lse, b_lse)


# ----------------------------------------------------------- random decode

DECODE_CASES = [
    # (dtype, kv_dtype, D, H, Hkv, bs, kv_lens, mask)
    ("f16", None, 64, 4, 4, 16, [1, 31, 32, 33, 200], pa.PA_MASK_NONE),
    ("bf16", None, 128, 8, 2, 16, [5, 64, 65, 1000], pa.PA_MASK_NONE),
    ("bf16", None, 128, 32, 1, 32, [17, 300], pa.PA_MASK_CAUSAL),       # g = 32: two head groups
    ("f16", None, 128, 24, 1, 128, [129, 7, 2048], pa.PA_MASK_ALIBI),   # g = 24: partial group
    ("f16", None, 64, 6, 3, 48, [0, 95, 96, 97], pa.PA_MASK_NONE),      # blockSize 48, kvlen 0
    ("bf16", "i8", 128, 16, 2, 32, [1, 33, 500, 4097], pa.PA_MASK_NONE),
    ("f16", "i8", 64, 8, 8, 64, [63, 64, 65], pa.PA_MASK_ALIBI),
    ("bf16", "i8", 128, 64, 8, 128, [3000, 16], pa.PA_MASK_NONE),
]


@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
def test_decode_random(case):
    dt, kvdt, D, H, Hkv, bs, kv_lens, mask = DECODE_CASES[case]
    _say(f"[decode] case {case}: {DECODE_CASES[case]}")
    inp = wl.make_random_case(case, batch=len(kv_lens), head_num=H, kv_head_num=Hkv,
                              head_size=D, block_size=bs, q_lens=[1] * len(kv_lens),
                              kv_lens=kv_lens, dtype=dt, kv_dtype=kvdt, mask_type=mask)
    out, lse = gpu_run(inp)
    ro, rl, rows = oracle_run(inp)
    compare(out, lse, ro, rl, rows, inp["query"].dtype, f"decode case {case}")


@pytest.mark.parametrize("chunk", ["8", "12", "64"])
def test_decode_forced_splits(chunk):
    """Many split-KV partials merged by the combine kernel equal the oracle."""
    inp = wl.make_random_case(50, batch=3, head_num=8, kv_head_num=2, head_size=128,
                              block_size=16, q_lens=[1, 1, 1], kv_lens=[3000, 257, 40],
                              dtype="bf16", mask_type=pa.PA_MASK_ALIBI)
    with pa.plan_options({pa.PA_OPT_DECODE_CHUNK_TILES: int(chunk)}):
        out, lse, op, ws = gpu_run(inp, keep_op=True)
    info = pa.pa_op_describe(op)
    op.destroy()
    assert len(info["combine_items"]) > 0
    ro, rl, rows = oracle_run(inp)
    compare(out, lse, ro, rl, rows, inp["query"].dtype, f"split chunk {chunk}")


WAVE_HEAD_CASES = [
    # (dtype, kv_dtype, D, H, Hkv, bs, kv_lens, mask, chunk)
    ("bf16", None, 128, 16, 4, 32, [1, 33, 700, 4097], pa.PA_MASK_NONE, None),
    ("f16", None, 64, 8, 8, 16, [0, 95, 96, 300], pa.PA_MASK_ALIBI, "8"),
    ("bf16", "i8", 128, 32, 8, 64, [63, 2000, 129], pa.PA_MASK_NONE, "12"),
    ("f16", "i8", 64, 16, 4, 32, [500, 31], pa.PA_MASK_ALIBI, None),
]


@pytest.mark.parametrize("case", range(len(WAVE_HEAD_CASES)))
def test_decode_wave_per_head(case):
    """Items of four kv heads, one per wave (forced on for small shapes)."""
    dt, kvdt, D, H, Hkv, bs, kv_lens, mask, chunk = WAVE_HEAD_CASES[case]
    _say(f"[decode wave-per-head] case {case}: {WAVE_HEAD_CASES[case]}")
    opts = {pa.PA_OPT_DECODE_WAVE_HEADS: 1}
    if chunk is not None:
        opts[pa.PA_OPT_DECODE_CHUNK_TILES] = int(chunk)
    inp = wl.make_random_case(300 + case, batch=len(kv_lens), head_num=H, kv_head_num=Hkv,
                              head_size=D, block_size=bs, q_lens=[1] * len(kv_lens),
                              kv_lens=kv_lens, dtype=dt, kv_dtype=kvdt, mask_type=mask)
    with pa.plan_options(opts):
        out, lse, op, ws = gpu_run(inp, keep_op=True)
    info = pa.pa_op_describe(op)
    op.destroy()
    assert info["decode_wave_heads"] == 1
    ro, rl, rows = oracle_run(inp)
    compare(out, lse, ro, rl, rows, inp["query"].dtype, f"wave-per-head case {case}")


ANTIQUANT_MODES = [(0, 0, True), (1, 1, False), (1, 1, True), (0, 1, False), (0, 1, True)]


@pytest.mark.parametrize("aq", ANTIQUANT_MODES, ids=lambda m: f"k{m[0]}v{m[1]}o{int(m[2])}")
@pytest.mark.parametrize("shape", ["plain", "alibi_d64", "splits", "wave_heads"])
def test_decode_antiquant_modes(aq, shape):
    """int8 decode with per-channel / per-token scales and offsets against the oracle."""
    _say(f"[decode antiquant] modes {aq} shape {shape}")
    kw = dict(batch=3, head_num=8, kv_head_num=2, head_size=128, block_size=32,
              q_lens=[1, 1, 1], kv_lens=[300, 45, 1], dtype="bf16", mask_type=pa.PA_MASK_NONE)
    opts = {}
    if shape == "alibi_d64":
        kw.update(head_size=64, dtype="f16", mask_type=pa.PA_MASK_ALIBI, kv_lens=[97, 160, 33])
    elif shape == "splits":
        opts[pa.PA_OPT_DECODE_CHUNK_TILES] = 8
        kw.update(kv_lens=[1500, 257, 31])
    elif shape == "wave_heads":
        opts[pa.PA_OPT_DECODE_WAVE_HEADS] = 1
        kw.update(head_num=32, kv_head_num=8, kv_lens=[700, 64, 2049], block_size=64)
    inp = wl.make_random_case(400 + len(shape), kv_dtype="i8", antiquant=aq, **kw)
    with pa.plan_options(opts):
        out, lse, op, ws = gpu_run(inp, keep_op=True)
    info = pa.pa_op_describe(op)
    op.destroy()
    assert info["antiquant"] == [aq[0], aq[1], int(aq[2])]
    if shape == "splits":
        assert len(info["combine_items"]) > 0
    if shape == "wave_heads":
        assert info["decode_wave_heads"] == 1
    ro, rl, rows = oracle_run(inp)
    compare(out, lse, ro, rl, rows, inp["query"].dtype, f"decode antiquant {aq} {shape}")


@pytest.mark.parametrize("aq", ANTIQUANT_MODES, ids=lambda m: f"k{m[0]}v{m[1]}o{int(m[2])}")
@pytest.mark.parametrize("mask", [pa.PA_MASK_CAUSAL, pa.PA_MASK_ALIBI])
def test_prefill_antiquant_modes(aq, mask):
    """int8 prefill (prefix encoder) with per-channel / per-token scales and offsets."""
    _say(f"[prefill antiquant] modes {aq} mask {mask}")
    inp = wl.make_random_case(500 + mask, batch=3, head_num=8, kv_head_num=2, head_size=128,
                              block_size=32, q_lens=[70, 1, 130], kv_lens=[200, 33, 130],
                              dtype="f16", kv_dtype="i8", mask_type=mask, antiquant=aq)
    out, lse = gpu_run(inp)
    ro, rl, rows = oracle_run(inp)
    compare(out, lse, ro, rl, rows, inp["query"].dtype, f"prefill antiquant {aq} {mask}")


FP8_CASES = [
    # (kind, dtype, D, H, Hkv, bs, q_lens, kv_lens, mask, env)
    ("decode", "bf16", 128, 8, 2, 32, [1, 1, 1], [300, 45, 1], pa.PA_MASK_NONE, {}),
    ("decode", "f16", 64, 8, 2, 64, [1, 1, 1], [97, 160, 33], pa.PA_MASK_ALIBI, {}),
    ("decode", "bf16", 128, 8, 2, 32, [1, 1, 1], [1500, 257, 31], pa.PA_MASK_NONE,
     {pa.PA_OPT_DECODE_CHUNK_TILES: 8}),
    ("decode", "bf16", 128, 32, 8, 64, [1, 1, 1], [700, 64, 2049], pa.PA_MASK_NONE,
     {pa.PA_OPT_DECODE_WAVE_HEADS: 1}),
    ("prefill", "f16", 128, 8, 2, 32, [70, 1, 130], [200, 33, 130], pa.PA_MASK_CAUSAL, {}),
    ("prefill", "bf16", 128, 8, 8, 32, [64, 100], [600, 100], pa.PA_MASK_ALIBI, {}),
    ("prefill", "f16", 64, 4, 2, 64, [33, 90], [33, 200], pa.PA_MASK_NONE, {}),
]


@pytest.mark.parametrize("case", range(len(FP8_CASES)))
def test_fp8_cache(case):
    """FLOAT8_E4M3FN K/V with per-channel scales (unused slots hold NaN codes)."""
    kind, dt, D, H, Hkv, bs, ql, kl, mask, opts = FP8_CASES[case]
    _say(f"[fp8] case {case}: {FP8_CASES[case]}")
    inp = wl.make_random_case(600 + case, batch=len(kl), head_num=H, kv_head_num=Hkv,
                              head_size=D, block_size=bs, q_lens=ql, kv_lens=kl, dtype=dt,
                              kv_dtype="f8", mask_type=mask)
    with pa.plan_options(opts):
        out, lse, op, ws = gpu_run(inp, keep_op=True)
    info = pa.pa_op_describe(op)
    op.destroy()
    assert info["mode"] == kind
    ro, rl, rows = oracle_run(inp)
    compare(out, lse, ro, rl, rows, inp["query"].dtype, f"fp8 case {case}")


def _append_inputs(seed, kv_dtype, *, q_lens, kv_lens, bs, Hkv=2, D=128, layout="bnbsh"):
    inp = wl.make_random_case(seed, batch=len(kv_lens), head_num=4 * Hkv, kv_head_num=Hkv,
                              head_size=D, block_size=bs, q_lens=q_lens, kv_lens=kv_lens,
                              dtype="bf16" if kv_dtype in ("i8", "f8") else kv_dtype,
                              kv_dtype=kv_dtype, poison=False)
    rng = np.random.default_rng([314, 2000 + seed])
    T = int(sum(q_lens))
    if kv_dtype == "i8":
        draw = lambda: torch.from_numpy(rng.integers(-127, 128, size=(T, Hkv, D), dtype=np.int8))
    elif kv_dtype == "f8":
        draw = lambda: torch.from_numpy(np.clip(rng.standard_normal((T, Hkv, D)).astype(np.float32)
                                                * 64, -448, 448)).to(torch.float8_e4m3fn)
    else:
        dt = torch.bfloat16 if kv_dtype == "bf16" else torch.float16
        draw = lambda: torch.from_numpy(rng.standard_normal((T, Hkv, D)).astype(np.float32)).to(dt)
    inp["key_new"], inp["value_new"] = draw(), draw()
    if layout == "bnnbsd":
        for k in ("key", "value"):
            inp[k] = inp[k].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    return inp


@pytest.mark.parametrize("kv_dtype,bs,layout", [("bf16", 16, "bnbsh"), ("f16", 128, "bnnbsd"),
                                                ("i8", 32, "bnbsh"), ("f8", 64, "bnnbsd"),
                                                ("bf16", 128, "bnbsh")])
def test_kv_cache_append_bit_exact(kv_dtype, bs, layout):
    """The cache after the append equals the oracle's, byte for byte."""
    _say(f"[append] {kv_dtype} bs {bs} {layout}")
    q_lens, kv_lens = [40, 0, 1, 300, 17], [100, 5, 1, 300, 17]
    inp = _append_inputs(700 + bs, kv_dtype, q_lens=q_lens, kv_lens=kv_lens, bs=bs, layout=layout)
    kc, vc = inp["key"].cuda(), inp["value"].cuda()
    pa.kv_cache_append(inp["key_new"].cuda(), inp["value_new"].cuda(), kc, vc,
                       inp["block_tables"].cuda(), inp["seq_len"], inp["kv_seq_len"])
    # compare bytes: rows of [.., headSize * element size] uint8 in the logical layout
    raw = lambda t: t.cpu().contiguous().view(torch.uint8).numpy()
    for cache, pool, new in ((kc, inp["key"], inp["key_new"]), (vc, inp["value"], inp["value_new"])):
        want = oracle.append_kv_rows(raw(pool), raw(new), inp["block_tables"].numpy(),
                                     q_lens, kv_lens)
        got = raw(cache)
        assert got.shape == want.shape
        assert np.array_equal(got, want)


def test_append_then_prefill_attention():
    """Append the new tokens, then attend with the same lengths: equals the oracle on the
    oracle-appended cache (queries are the new tokens, the prefix-encoder step)."""
    q_lens, kv_lens = [70, 1, 130], [200, 33, 130]
    inp = _append_inputs(801, "bf16", q_lens=q_lens, kv_lens=kv_lens, bs=32, Hkv=2)
    inp["mask_type"] = pa.PA_MASK_CAUSAL
    kc, vc = inp["key"].cuda(), inp["value"].cuda()
    pa.kv_cache_append(inp["key_new"].cuda(), inp["value_new"].cuda(), kc, vc,
                       inp["block_tables"].cuda(), inp["seq_len"], inp["kv_seq_len"])
    table = inp["block_tables"].numpy()
    ref = dict(inp)
    ref["key"] = torch.from_numpy(oracle.append_kv_rows(inp["key"].float().numpy(),
                                                        inp["key_new"].float().numpy(),
                                                        table, q_lens, kv_lens))
    ref["value"] = torch.from_numpy(oracle.append_kv_rows(inp["value"].float().numpy(),
                                                          inp["value_new"].float().numpy(),
                                                          table, q_lens, kv_lens))
    run = dict(inp, key=kc, value=vc)
    out, lse = gpu_run(run)
    ro, rl, rows = oracle_run(ref)
    compare(out, lse, ro, rl, rows, inp["query"].dtype, "append then prefill")


LARGE_CASES = [
    # (kind, dtype, kv_dtype, D, H, Hkv, bs, q_lens, kv_lens, mask)
    ("decode", "bf16", None, 128, 64, 8, 128, [1, 1], [131072 + 17, 1], pa.PA_MASK_NONE),
    ("decode", "bf16", "i8", 128, 64, 8, 256, [1, 1], [131072 + 100, 3], pa.PA_MASK_NONE),
    ("prefill", "f16", None, 128, 4, 2, 1024, [300], [65536 + 300], pa.PA_MASK_ALIBI),
    ("prefill", "bf16", None, 64, 8, 8, 4096, [257, 1], [9000, 5000], pa.PA_MASK_CAUSAL),
]


@pytest.mark.parametrize("case", range(len(LARGE_CASES)))
def test_large_sizes(case):
    """Long sequences (131 k tokens decode, a 65 k-token prefix) and large blocks (up to
    4096 slots) against the oracle."""
    kind, dt, kvdt, D, H, Hkv, bs, ql, kl, mask = LARGE_CASES[case]
    _say(f"[large] case {case}: {kind} {dt}/{kvdt} D{D} H{H}/{Hkv} bs{bs} q{ql} kv{kl}")
    inp = wl.make_random_case(900 + case, batch=len(kl), head_num=H, kv_head_num=Hkv,
                              head_size=D, block_size=bs, q_lens=ql, kv_lens=kl, dtype=dt,
                              kv_dtype=kvdt, mask_type=mask, poison=False)
    out, lse, op, ws = gpu_run(inp, keep_op=True)
    info = pa.pa_op_describe(op)
    op.destroy()
    assert info["mode"] == kind
    ro, rl, rows = oracle_run(inp)
    st = compare(out, lse, ro, rl, rows, inp["query"].dtype, f"large case {case}")
    _say(f"[large] case {case} {st}")


def test_decode_skips_sequences_without_query():
    inp = wl.make_random_case(51, batch=4, head_num=4, kv_head_num=2, head_size=128,
                              block_size=16, q_lens=[1, 0, 1, 0], kv_lens=[100, 50, 0, 7],
                              dtype="f16")
    out, lse = gpu_run(inp)
    ro, rl, rows = oracle_run(inp)
    compare(out, lse, ro, rl, rows, inp["query"].dtype, "decode q_len 0")


# ----------------------------------------------------------- random prefill

PREFILL_CASES = [
    # (dtype, kv_dtype, D, H, Hkv, bs, q_lens, kv_lens, mask)
    ("bf16", None, 128, 4, 2, 128, [512, 300], [512, 300], pa.PA_MASK_CAUSAL),
    ("f16", None, 128, 2, 2, 128, [130, 64], [1000, 64], pa.PA_MASK_ALIBI),
    ("f16", None, 64, 4, 1, 16, [127, 129, 3], [127, 400, 10], pa.PA_MASK_CAUSAL),
    ("bf16", None, 64, 2, 2, 32, [70, 5], [33, 200], pa.PA_MASK_NONE),
    ("bf16", None, 128, 2, 1, 48, [200, 2], [100, 1], pa.PA_MASK_CAUSAL),   # rows with no key
    ("bf16", "i8", 128, 4, 2, 64, [150, 33], [700, 33], pa.PA_MASK_CAUSAL),
    ("f16", "i8", 64, 2, 2, 32, [65], [2000], pa.PA_MASK_ALIBI),
    ("f16", None, 128, 3, 3, 16, [1, 2, 0, 66], [5, 2, 9, 66], pa.PA_MASK_NONE),
    # block sizes that are not powers of two: the tile loads find the block by division
    ("f16", None, 128, 4, 1, 80, [300, 77], [1000, 400], pa.PA_MASK_ALIBI),
    ("bf16", None, 64, 2, 2, 48, [257, 64], [1500, 64], pa.PA_MASK_CAUSAL),
]


@pytest.mark.parametrize("case", range(len(PREFILL_CASES)))
def test_prefill_random(case):
    dt, kvdt, D, H, Hkv, bs, q_lens, kv_lens, mask = PREFILL_CASES[case]
    _say(f"[prefill] case {case}: {PREFILL_CASES[case]}")
    inp = wl.make_random_case(100 + case, batch=len(q_lens), head_num=H, kv_head_num=Hkv,
                              head_size=D, block_size=bs, q_lens=q_lens, kv_lens=kv_lens,
                              dtype=dt, kv_dtype=kvdt, mask_type=mask)
    out, lse = gpu_run(inp)
    ro, rl, rows = oracle_run(inp)
    compare(out, lse, ro, rl, rows, inp["query"].dtype, f"prefill case {case}")


# ----------------------------------------------- steep ALiBi: negligible tiles skipped

@pytest.mark.parametrize("dt,D,bs", [("f16", 128, 64), ("bf16", 64, 64),
                                     ("f16", 128, 80), ("bf16", 64, 48)])
def test_steep_alibi_long_prefix(dt, D, bs):
    """Slopes of 1 over a 3000-token prefix: nearly every prefix tile lies more than 32
    log2 units below its rows' reference (most of them far tiles, skipped on a bound from
    their K rows' norms), so the kernel skips their P and P V; out and lse must still
    match the full computation of the oracle.  Block sizes of 80 and 48 make the far
    tiles' loads find their blocks by division."""
    _say(f"[steep alibi] {dt} D={D} blockSize={bs}")
    inp = wl.make_random_case(950 + D + bs, batch=2, head_num=4, kv_head_num=2, head_size=D,
                              block_size=bs, q_lens=[200, 70], kv_lens=[3200, 3070],
                              dtype=dt, mask_type=pa.PA_MASK_ALIBI)
    inp["slopes"] = torch.full((4,), 1.0, dtype=torch.float32)
    inp["slopes"][3] = 0.004          # one shallow head: its tiles are all computed
    out, lse = gpu_run(inp)
    ro, rl, rows = oracle_run(inp)
    compare(out, lse, ro, rl, rows, inp["query"].dtype, f"steep alibi {dt} D={D} bs={bs}")


# far prefix keys given a dominant K row: one per sequence, or two per sequence in far
# tiles apart (the farthest tile among them), so that the tiles computed run from the
# first to the last uncovered one across covered tiles
DOMINANT_KEYS = {
    "one": ((0, 100), (1, 700)),
    "two_apart": ((0, 20), (0, 1500), (1, 10), (1, 2000)),
}


@pytest.mark.parametrize("keys", list(DOMINANT_KEYS))
@pytest.mark.parametrize("D", [64, 128])
def test_alibi_far_tile_holding_a_dominant_key(D, keys):
    """ALiBi prefix tiles far enough from a workgroup's rows are skipped when a bound on
    their scores (the largest |scaled q| times the largest |k| of the tile, plus the
    tile's largest bias) shows them negligible.  Here keys of such tiles get outsized
    scores (their K rows are 400 times a direction every query leans towards), so they
    dominate their rows' softmax despite the bias: the bound fails for their tiles, which
    must be computed, and the result must match the oracle."""
    _say(f"[alibi dominant far key] D={D} keys={keys}")
    inp = wl.make_random_case(970 + D, batch=2, head_num=4, kv_head_num=2, head_size=D,
                              block_size=64, q_lens=[200, 70], kv_lens=[3200, 3070],
                              dtype="f16", mask_type=pa.PA_MASK_ALIBI)
    inp["slopes"] = torch.full((4,), 0.05, dtype=torch.float32)
    u = torch.full((D,), 1.0 / D ** 0.5)
    inp["query"] = (inp["query"].float() + 5.0 * u).to(inp["query"].dtype)
    table = inp["block_tables"]
    bs = inp["key"].shape[1]
    for b, pos in DOMINANT_KEYS[keys]:
        blk, slot = int(table[b, pos // bs]), pos % bs
        inp["key"][blk, slot] = (400.0 * u).to(inp["key"].dtype)
        inp["value"][blk, slot] = 3.0
    out, lse = gpu_run(inp)
    ro, rl, rows = oracle_run(inp)
    assert float(np.abs(np.asarray(ro, dtype=np.float64)).max()) > 2.5   # a dominant key's V shows
    compare(out, lse, ro, rl, rows, inp["query"].dtype, f"alibi dominant far key D={D} {keys}")


# ----------------------------------------------------------- unusual qkScale

SCALE_KINDS = {
    # kind: (dtype, kv_dtype, D, H, Hkv, bs, q_lens, kv_lens)
    "decode": ("bf16", None, 128, 8, 2, 32, [1, 1], [77, 300]),
    "decode_i8": ("f16", "i8", 128, 8, 1, 32, [1, 1], [40, 257]),
    "prefill": ("f16", None, 128, 4, 4, 64, [100, 70], [260, 70]),
    "prefill_i8": ("bf16", "i8", 64, 2, 1, 32, [90], [150]),
}


@pytest.mark.parametrize("qk_scale", [-0.09, 0.0, 1e-3])
@pytest.mark.parametrize("mask", [pa.PA_MASK_ALIBI, pa.PA_MASK_CAUSAL])
@pytest.mark.parametrize("kind", list(SCALE_KINDS))
def test_unusual_qk_scale(kind, mask, qk_scale):
    """Negative, zero and tiny qkScale (the softmax then follows the bias / mask alone)."""
    dt, kvdt, D, H, Hkv, bs, q_lens, kv_lens = SCALE_KINDS[kind]
    _say(f"[scale] {kind} mask {mask} qk_scale {qk_scale}")
    inp = wl.make_random_case(200 + len(kind), batch=len(q_lens), head_num=H,
                              kv_head_num=Hkv, head_size=D, block_size=bs, q_lens=q_lens,
                              kv_lens=kv_lens, dtype=dt, kv_dtype=kvdt, mask_type=mask,
                              qk_scale=qk_scale)
    out, lse = gpu_run(inp)
    ro, rl, rows = oracle_run(inp)
    compare(out, lse, ro, rl, rows, inp["query"].dtype, f"{kind} qk_scale {qk_scale}")


# ----------------------------------------------------------- empty tensors

def test_empty_key_value_gives_zero_and_inf():
    inp = wl.make_random_case(60, batch=2, head_num=4, kv_head_num=4, head_size=64,
                              block_size=16, q_lens=[1, 1], kv_lens=[20, 3], dtype="f16")
    inp["key"] = inp["key"][:0]
    inp["value"] = inp["value"][:0]
    out, lse = gpu_run(inp)
    assert torch.all(out == 0)
    assert torch.all(torch.isinf(lse)) and torch.all(lse > 0)


def test_all_kv_lengths_zero():
    inp = wl.make_random_case(61, batch=2, head_num=4, kv_head_num=2, head_size=128,
                              block_size=16, q_lens=[3, 2], kv_lens=[0, 0], dtype="bf16",
                              mask_type=pa.PA_MASK_NONE, extra_blocks=2)
    out, lse = gpu_run(inp)
    assert torch.all(out == 0)
    assert torch.all(torch.isinf(lse)) and torch.all(lse > 0)


def test_empty_query_is_noop():
    inp = wl.make_random_case(62, batch=1, head_num=4, kv_head_num=4, head_size=64,
                              block_size=16, q_lens=[0], kv_lens=[20], dtype="f16")
    out, lse = gpu_run(inp)
    assert out.numel() == 0 and lse.numel() == 0


# ----------------------------------------------------------- strided views

def test_strided_query_out_and_head_major_cache():
    """Q sliced out of a fused projection, out with padded heads, K/V given as a
    permuted (numBlocks, kvHeadNum, blockSize, headSize) cache."""
    inp = wl.make_random_case(70, batch=3, head_num=8, kv_head_num=2, head_size=128,
                              block_size=32, q_lens=[1, 1, 1], kv_lens=[90, 513, 32],
                              dtype="bf16", mask_type=pa.PA_MASK_NONE)
    ro, rl, rows = oracle_run(inp)
    T, H, D = inp["query"].shape
    fused = torch.randn(T, H + 4, D).to(torch.bfloat16)
    fused[:, :H] = inp["query"]
    g = dict(inp)
    g["query"] = fused.cuda()[:, :H]
    g["key"] = inp["key"].permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    g["value"] = inp["value"].permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    padded = torch.zeros(T, H, D + 8, dtype=torch.bfloat16, device="cuda")
    out = padded[:, :, :D]
    out2, lse = gpu_run(g, out=out)
    compare(out2, lse, ro, rl, rows, torch.bfloat16, "strided")
    assert torch.all(padded[:, :, D:] == 0), "wrote outside the out view"


def test_two_dimensional_query_form():
    inp = wl.make_random_case(71, batch=2, head_num=4, kv_head_num=4, head_size=64,
                              block_size=16, q_lens=[1, 1], kv_lens=[40, 17], dtype="f16")
    ro, rl, rows = oracle_run(inp)
    g = dict(inp)
    g["query"] = inp["query"].reshape(2, 4 * 64)
    out = torch.empty(2, 4 * 64, dtype=torch.float16, device="cuda")
    out2, lse = gpu_run(g, out=out)
    compare(out2.reshape(2, 4, 64), lse, ro, rl, rows, torch.float16, "2-D query")


def test_reruns_on_other_streams_and_workspaces():
    """An op runs again on other streams, with a fresh workspace filled with garbage,
    and gives bit-identical results (its kernels read the op's pinned work lists)."""
    inp = wl.make_random_case(73, batch=3, head_num=8, kv_head_num=2, head_size=128,
                              block_size=16, q_lens=[1, 1, 1], kv_lens=[5000, 40, 333],
                              dtype="f16")
    s = torch.cuda.Stream()
    out, lse, op, ws = gpu_run(inp, stream=s, keep_op=True)
    try:
        info = pa.pa_op_describe(op)
        assert info["items_bytes"] > 0
        assert info["partial_slots"] > 0          # the split path and its combine ran
        ro, rl, rows = oracle_run(inp)
        compare(out, lse, ro, rl, rows, torch.float16, "first run, side stream")
        ref_o, ref_l = out.clone(), lse.clone()
        for stream, fresh in ((None, False), (torch.cuda.Stream(), True), (s, True)):
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
            w = ws
            if fresh:
                w = torch.full((op.workspace_size,), 0xFF, dtype=torch.uint8, device="cuda")
                torch.cuda.synchronize()
            pa.pa_paged_attention(w, op.workspace_size, op, stream)
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    finally:
        op.destroy()


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_execute_under_graph_capture(kind):
    """An execute captured into a graph (its first run, with no eager run before): every
    replay matches an eager run, with garbage written into the workspace and the
    program's own eager work between the replays."""
    if kind == "decode":
        inp = wl.make_random_case(74, batch=2, head_num=8, kv_head_num=2, head_size=128,
                                  block_size=16, q_lens=[1, 1], kv_lens=[4100, 77], dtype="bf16")
    else:
        inp = wl.make_random_case(75, batch=2, head_num=8, kv_head_num=2, head_size=128,
                                  block_size=64, q_lens=[200, 70], kv_lens=[600, 70],
                                  dtype="f16", mask_type=pa.PA_MASK_CAUSAL)
    ref_o, ref_l = gpu_run(inp)                  # another op, eager
    from tests.harness import to_device
    g = to_device(inp)
    q = g["query"]
    out = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], g["head_num"]), float("nan"), dtype=torch.float32,
                     device=q.device)
    op = pa.pa_paged_attention_get_workspace_size_ex(
        q, g["key"], g["value"], g["block_tables"], None, g["seq_len"], g["kv_seq_len"],
        g["slopes"], g["mask_type"], g["head_num"], g["kv_head_num"], g["qk_scale"],
        g["key_scale"], g["value_scale"], None, None, 0, 0, out, lse)
    ws = pa.alloc_workspace(op.workspace_size, q.device)
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    try:
        with torch.cuda.graph(graph):
            pa.pa_paged_attention(ws, op.workspace_size, op, None)
        for r in range(3):
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
            if ws is not None:
                ws.fill_(0xFF)                  # scratch: its contents on entry do not matter
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {r}"
            # the program's own eager work between replays
            x = torch.randn(4096, device=q.device)
            assert torch.isfinite(x.sum()).item()
        out.fill_(float("nan"))
        pa.pa_paged_attention(ws, op.workspace_size, op, None)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o)
    finally:
        graph.reset()
        op.destroy()


def test_runs_on_a_side_stream():
    inp = wl.make_random_case(72, batch=2, head_num=8, kv_head_num=2, head_size=128,
                              block_size=16, q_lens=[1, 1], kv_lens=[700, 33], dtype="bf16")
    s = torch.cuda.Stream()
    out, lse = gpu_run(inp, stream=s)
    ro, rl, rows = oracle_run(inp)
    compare(out, lse, ro, rl, rows, torch.bfloat16, "side stream")


# ------------------------------------------- BnNBsD cache layout (head-major blocks)

def _head_major(inp):
    """The same pool stored as (numBlocks, kvHeadNum, blockSize, headSize) and passed
    as its permuted (numBlocks, blockSize, kvHeadNum, headSize) view: each (block, kv
    head) is one contiguous blockSize x headSize run (aclnnFusedInferAttentionScoreV3,
    Constraints, paged attention scenario: the BnNBsD layout)."""
    g = dict(inp)
    for k in ("key", "value"):
        g[k] = inp[k].permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
    assert g["key"].stride(1) == inp["key"].shape[3]           # slot stride = headSize
    return g


@pytest.mark.parametrize("name", ["prefill_causal_bf16", "prefill_alibi_f16",
                                  "decode_int8_long", "decode_fp8_long",
                                  "decode_bf16_batched"])
def test_named_workload_head_major_cache(name):
    """Full-size workloads over the BnNBsD view: every row against the oracle."""
    _say(f"[bnnbsd] {name}")
    inp = wl.make_inputs(wl.WORKLOADS[name], poison=True)
    out, lse = gpu_run(_head_major(inp))
    ro, rl, rows = oracle_run(inp)
    st = compare(out, lse, ro, rl, rows, inp["query"].dtype, name + " bnnbsd")
    _say(f"[bnnbsd] {name} {st}")


HEAD_MAJOR_CASES = [
    # (kind, dtype, kv_dtype, D, H, Hkv, bs, q_lens, kv_lens, mask, opts)
    ("prefill", "f16", None, 128, 8, 2, 64, [200, 1, 130], [700, 33, 130], pa.PA_MASK_CAUSAL, {}),
    ("prefill", "bf16", None, 64, 4, 4, 32, [100, 65], [1000, 65], pa.PA_MASK_ALIBI, {}),
    ("prefill", "bf16", "i8", 128, 8, 2, 64, [150, 33], [700, 33], pa.PA_MASK_CAUSAL, {}),
    ("prefill", "f16", "i8", 128, 4, 4, 128, [130, 64], [2000, 64], pa.PA_MASK_ALIBI, {}),
    ("prefill", "f16", "f8", 128, 8, 2, 32, [70, 1, 130], [200, 33, 130], pa.PA_MASK_CAUSAL, {}),
    ("prefill", "bf16", "f8", 64, 8, 8, 64, [64, 100], [600, 100], pa.PA_MASK_ALIBI, {}),
    ("decode", "bf16", "i8", 128, 64, 8, 128, [1, 1, 1], [5000, 31, 2049], pa.PA_MASK_NONE, {}),
    ("decode", "bf16", "i8", 128, 32, 8, 64, [1, 1, 1], [700, 64, 2049], pa.PA_MASK_NONE,
     {pa.PA_OPT_DECODE_WAVE_HEADS: 1}),
    ("decode", "f16", "f8", 64, 8, 2, 32, [1, 1, 1], [1500, 257, 31], pa.PA_MASK_ALIBI,
     {pa.PA_OPT_DECODE_CHUNK_TILES: 8}),
    ("decode", "bf16", "f8", 128, 64, 8, 128, [1, 1], [9000, 130], pa.PA_MASK_NONE, {}),
]


@pytest.mark.parametrize("case", range(len(HEAD_MAJOR_CASES)))
def test_head_major_cache_cases(case):
    """16-bit, INT8 and FP8 caches in the BnNBsD layout: prefill (causal, ALiBi) and
    decode (plain, wave-per-head items, forced splits) against the oracle."""
    kind, dt, kvdt, D, H, Hkv, bs, ql, kl, mask, opts = HEAD_MAJOR_CASES[case]
    _say(f"[bnnbsd] case {case}: {HEAD_MAJOR_CASES[case]}")
    inp = wl.make_random_case(1100 + case, batch=len(kl), head_num=H, kv_head_num=Hkv,
                              head_size=D, block_size=bs, q_lens=ql, kv_lens=kl, dtype=dt,
                              kv_dtype=kvdt, mask_type=mask)
    with pa.plan_options(opts):
        out, lse, op, ws = gpu_run(_head_major(inp), keep_op=True)
    info = pa.pa_op_describe(op)
    op.destroy()
    assert info["mode"] == kind
    ro, rl, rows = oracle_run(inp)
    compare(out, lse, ro, rl, rows, inp["query"].dtype, f"bnnbsd case {case}")
