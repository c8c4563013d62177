"""CPU tests of the C ABI: symbols, phase-1 validation and planning.

Phase 1 (pa_paged_attention_get_workspace_size) never dereferences device
pointers (without a GPU its only HIP calls, the device queries, report no
device), so these tests hand it descriptors with fake, aligned device addresses
and real host length arrays.  Phase 2 is only called on paths that return before
any HIP call (NULL op, short workspace, no-op op, wrong op kind).
"""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import paged_kv_cache_314_amd as pa
from paged_kv_cache_314_amd import workloads as wl

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "pagedattn.h")
FAKE = 0x7f0000000000          # 256-aligned fake device address (never dereferenced)
ESZ = {pa.PA_F16: 2, pa.PA_BF16: 2, pa.PA_I8: 1, pa.PA_F32: 4, pa.PA_I32: 4}


def desc(shape, dtype, ptr=FAKE, strides=None):
    d = pa.PaTensor()
    d.data = ptr
    d.dtype = dtype
    d.ndim = len(shape)
    if strides is None:
        strides, acc = [], 1
        for s in reversed(shape):
            strides.insert(0, acc)
            acc *= s
    for i, (s, st) in enumerate(zip(shape, strides)):
        d.shape[i] = s
        d.stride[i] = st
    return d


def host_i32(values):
    arr = np.ascontiguousarray(np.asarray(values, dtype=np.int32))
    d = desc([arr.shape[0]], pa.PA_I32, ptr=arr.ctypes.data)
    return d, arr


class Case:
    """Descriptor set for one phase-1 call; fields can be overridden per test."""

    def __init__(self, *, q_lens, kv_lens, H, Hkv, D, bs, dtype=pa.PA_BF16, kv_dtype=None,
                 mask=pa.PA_MASK_NONE, lse=True, num_blocks=None, width=None):
        kv_dtype = kv_dtype or dtype
        T = int(sum(q_lens))
        need = sum(-(-k // bs) for k in kv_lens)
        nb = need if num_blocks is None else num_blocks
        W = max([-(-k // bs) for k in kv_lens] + [1]) if width is None else width
        self.query = desc([T, H, D], dtype)
        self.key = desc([nb, bs, Hkv, D], kv_dtype)
        self.value = desc([nb, bs, Hkv, D], kv_dtype)
        self.table = desc([len(q_lens), W], pa.PA_I32)
        self.mask = None
        self.seq_len, self._ql = host_i32(q_lens)
        self.kv_seq_len, self._kl = host_i32(kv_lens)
        self.slopes = desc([H], pa.PA_F32) if mask == pa.PA_MASK_ALIBI else None
        self.mask_type = mask
        self.H, self.Hkv, self.scale = H, Hkv, 1.0 / math.sqrt(D)
        one_byte = kv_dtype in (pa.PA_I8, pa.PA_F8E4M3)
        self.kscale = desc([Hkv, D], pa.PA_F32) if one_byte else None
        self.vscale = desc([Hkv, D], pa.PA_F32) if one_byte else None
        self.out = desc([T, H, D], dtype)
        self.lse = desc([T, H], pa.PA_F32) if lse else None
        self.koff = self.voff = None
        self.kmode = self.vmode = 0
        self.extended = False
        self.kv_lens = [int(k) for k in kv_lens]

    def call(self):
        lib = pa.load()
        ws = ctypes.c_uint64(123)
        op = ctypes.c_void_p(None)
        r = lambda d: ctypes.byref(d) if d is not None else None
        if self.extended:
            st = lib.pa_paged_attention_get_workspace_size_ex(
                r(self.query), r(self.key), r(self.value), r(self.table), r(self.mask),
                r(self.seq_len), r(self.kv_seq_len), r(self.slopes), self.mask_type, self.H,
                self.Hkv, self.scale, r(self.kscale), r(self.vscale), r(self.koff),
                r(self.voff), self.kmode, self.vmode, r(self.out), r(self.lse),
                ctypes.byref(ws), ctypes.byref(op))
        else:
            st = lib.pa_paged_attention_get_workspace_size(
                r(self.query), r(self.key), r(self.value), r(self.table), r(self.mask),
                r(self.seq_len), r(self.kv_seq_len), r(self.slopes), self.mask_type, self.H,
                self.Hkv, self.scale, r(self.kscale), r(self.vscale), r(self.out), r(self.lse),
                ctypes.byref(ws), ctypes.byref(op))
        return st, int(ws.value), op.value

    def plan(self):
        st, ws, op = self.call()
        assert st == pa.PA_OK, pa.pa_last_error()
        info = pa.pa_op_describe(op)
        assert info["workspace_bytes"] == ws
        pa.pa_op_destroy(op)
        return info


# --------------------------------------------------------------- symbols

def test_library_exports_every_header_symbol():
    with open(HEADER) as f:
        text = f.read()
    declared = set(re.findall(r"^\S.*?\b(pa_\w+)\s*\(", text, flags=re.M))
    assert declared == set(pa.EXPORTED)
    lib = pa.load()
    for name in declared:
        assert getattr(lib, name) is not None
    assert pa.pa_version() >= 100
    for st in range(7):
        assert pa.pa_status_string(st)


# ---------------------------------------------------------------- planning

def _named_case(name):
    """A Case with a named workload's shape and its seeded kv lengths."""
    w = wl.WORKLOADS[name]
    rng = np.random.default_rng([314, w.index, 1])
    if isinstance(w.kv_seq_len, tuple):
        kv = rng.integers(w.kv_seq_len[1], w.kv_seq_len[2] + 1, size=w.batch).tolist()
    elif isinstance(w.kv_seq_len, list):
        kv = w.kv_seq_len
    else:
        kv = [w.kv_seq_len] * w.batch
    ql = [1] * w.batch if w.seq_len == "decode" else [w.seq_len] * w.batch
    dt = {"f16": pa.PA_F16, "bf16": pa.PA_BF16, "i8": pa.PA_I8, "f8": pa.PA_F8E4M3}
    c = Case(q_lens=ql, kv_lens=kv, H=w.head_num, Hkv=w.kv_head_num, D=w.head_size,
             bs=w.block_size, dtype=dt[w.dtype], kv_dtype=dt[w.kv_dtype], mask=w.mask_type,
             width=w.table_width)
    return w, c, ql, kv


def _plan_named(name):
    return _named_case(name)[1].plan()


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_plan_for_named_workloads(name):
    w, c, ql, kv = _named_case(name)
    info = c.plan()
    assert info["mode"] == ("decode" if w.seq_len == "decode" else "prefill")
    if info["mode"] == "decode":
        _check_decode_plan(info, ql, kv, w.kv_head_num, w.head_num // w.kv_head_num)
    else:
        _check_prefill_plan(info, ql, kv, w.head_num, w.mask_type, w.head_num // w.kv_head_num)


def _alibi_item_cost(it, head_num):
    """Estimated cost of an ALiBi prefill item: 20 per computed key tile, 3 per far
    prefix tile (bias alone over 64 log2 units below the nearest key's at the item's
    smallest slope, geometric slopes 2^(-8(h+1)/H) assumed)."""
    b, h, qbeg, qlen, kvlen, qrow0, ktiles, heads = it[:8]
    shift, T = kvlen - qlen, ktiles - 1
    P = min(shift // 64 if shift > 0 else 0, T)
    s2 = 2.0 ** (-8.0 * (h + heads) / head_num) * 1.4426950408889634
    # tile t < P is far iff s2 * (shift + qbeg - (64 t + 63)) > 64, i.e. 64 t < y
    y = (shift + qbeg - 63) - 64.0 / s2
    far = min(P, math.ceil(y / 64)) if y > 0 else 0
    # the same count by enumeration
    assert far == sum(1 for t in range(P) if s2 * (shift + qbeg - (64 * t + 63)) > 64.0)
    return 20 * (ktiles - far) + 3 * far


def test_alibi_prefill_items_heaviest_first_by_estimated_cost():
    """ALiBi prefill items run heaviest first by an estimated cost that counts far prefix
    tiles (only bounded, not computed) at 3/20 of a computed tile; the XCD placement keeps
    every item and leaves each XCD's list (longer than two rounds here) heaviest first."""
    w = wl.WORKLOADS["prefill_alibi_f16"]
    with pa.plan_options({pa.PA_OPT_PREFILL_XCD_ORDER: 0}):
        items = _plan_named("prefill_alibi_f16")["prefill_items"]
    costs = [_alibi_item_cost(it, w.head_num) for it in items]
    assert costs == sorted(costs, reverse=True)
    assert costs[0] > costs[-1]                 # the steep heads' items do come out lighter
    placed = _plan_named("prefill_alibi_f16")["prefill_items"]
    real = [it for it in placed if it[7] != 0]
    assert sorted(map(tuple, real)) == sorted(map(tuple, items))
    for x in range(8):
        lst = [it for it in placed[x::8] if it[7] != 0]
        assert len(lst) > 64
        c = [_alibi_item_cost(it, w.head_num) for it in lst]
        assert c == sorted(c, reverse=True)


def test_single_round_prefill_pairs_heavy_with_light():
    """When an XCD's list fits one round (33..64 workgroups for its 32 CUs), positions k
    and k + 32 share a CU: the first 32 are the heaviest, heaviest first, and the rest
    come lightest first, so each CU gets one heavy and one light item."""
    info = _plan_named("prefill_causal_bf16")
    items = info["prefill_items"]
    assert len(items) == 512
    for x in range(8):
        lst = [it for it in items[x::8] if it[7] != 0]
        assert 32 < len(lst) <= 64
        w = [it[6] for it in lst]
        first, second = w[:32], w[32:]
        assert first == sorted(first, reverse=True)
        assert second == sorted(second)
        assert min(first) >= max(second)
        # the causal 16-tile clusters: pairs (8, 1), (7, 2), (6, 3), (5, 4) key tiles
        assert sorted(w[k] + w[k + 32] for k in range(len(lst) - 32)) == [9] * (len(lst) - 32)


def _check_decode_plan(info, q_lens, kv_lens, Hkv, group):
    """Every (sequence, kv head, head group) is covered by tile ranges that partition
    [0, ceil(kvlen/32)) exactly once; split items own consecutive slots merged by one
    combine item; single-split items write directly (slot -1)."""
    n_hg = -(-group // 16)
    items = info["decode_items"]
    wph = info["decode_wave_heads"] == 1
    assert not wph or (Hkv % 4 == 0 and group <= 16)
    by_key = {}
    combs = info["combine_items"]
    written = set()
    for b, kvh, hg, t0, t1, slot, qrow, kvlen, heads, stride, comb, nsplit in items:
        # the first split of each split group hands the combine kernel its item
        if comb >= 0 and t0 == 0:
            for w in range(heads):
                assert combs[comb + w] == [kvh + w, hg, slot + w * stride, nsplit, qrow]
                assert comb + w not in written
                written.add(comb + w)
        assert (comb >= 0) == (slot >= 0) and (nsplit > 1) == (slot >= 0)
        # an item of 4 kv heads stands for one range of each of kvh .. kvh+3
        assert heads == (4 if wph else 1)
        if heads == 4:
            assert kvh % 4 == 0 and hg == 0
        for w in range(heads):
            s = -1 if slot < 0 else slot + w * stride
            by_key.setdefault((b, kvh + w, hg), []).append((t0, t1, s, qrow, kvlen))
    q0 = np.concatenate([[0], np.cumsum(q_lens)])
    combines = {(c[0], c[1], c[4]): c for c in info["combine_items"]}
    slots_seen = set()
    for b, (ql, kl) in enumerate(zip(q_lens, kv_lens)):
        for kvh in range(Hkv):
            for hg in range(n_hg):
                parts = by_key.pop((b, kvh, hg), None) if ql == 1 else None
                if ql != 1:
                    assert (b, kvh, hg) not in by_key
                    continue
                assert parts, (b, kvh, hg)
                parts.sort()                    # launch order is a schedule, not tile order
                tiles = -(-kl // 32)
                cur = 0
                for t0, t1, slot, qrow, kvlen in parts:
                    assert t0 == cur and t1 >= t0 and qrow == q0[b] and kvlen == kl
                    cur = t1
                assert cur == tiles
                if len(parts) == 1:
                    assert parts[0][2] == -1
                else:
                    slots = [p[2] for p in parts]
                    assert slots == list(range(slots[0], slots[0] + len(parts)))
                    assert not (set(slots) & slots_seen)
                    slots_seen |= set(slots)
                    c = combines.pop((kvh, hg, int(q0[b])))
                    assert c[2] == slots[0] and c[3] == len(parts)
    assert not by_key and not combines
    assert info["partial_slots"] == len(slots_seen)
    assert written == set(range(len(combs)))


def _check_xcd_order(items, xcds=8):
    """Items sharing (sequence, head block) sit on one XCD (position % 8) unless the
    cluster exceeds 1/8 of the items; no-op padding (heads == 0) only ends a list."""
    assert len(items) % xcds == 0
    real = sum(1 for it in items if it[7] != 0)
    cap = max(1, -(-real // xcds))
    where = {}
    for pos, it in enumerate(items):
        if it[7] == 0:
            assert all(v == 0 for v in it)
            assert all(items[q][7] == 0 for q in range(pos, len(items), xcds)), "padding ends a list"
            continue
        where.setdefault((it[0], it[1]), []).append(pos % xcds)
    for key, xs in where.items():
        assert len(set(xs)) <= -(-len(xs) // cap), (key, xs)


def _check_prefill_plan(info, q_lens, kv_lens, H, mask, group=None):
    """Every (sequence, query head, query row) is covered exactly once; a workgroup's
    heads share one kv head; ktiles counts the key tiles its rows can see."""
    items = info["prefill_items"]
    cus = info["compute_units"]
    _check_xcd_order(items, min(8, cus // 32) if cus % 32 == 0 else 1)
    items = [it for it in items if it[7] != 0]
    covered = {}
    q0 = np.concatenate([[0], np.cumsum(q_lens)])
    for b, h, qbeg, qlen, kvlen, qrow0, ktiles, heads in items:
        assert heads in (1, 2, 4) and 128 % heads == 0
        if group is not None:
            assert group % heads == 0 and h // group == (h + heads - 1) // group
        nrows = 128 // heads
        assert qlen == q_lens[b] and kvlen == kv_lens[b] and qrow0 == q0[b]
        rows = range(qbeg, min(qbeg + nrows, qlen))
        for hh in range(h, h + heads):
            for i in rows:
                key = (b, hh, i)
                assert key not in covered
                covered[key] = True
        # keys that the tile's rows can see, counted independently
        if mask in (pa.PA_MASK_CAUSAL, pa.PA_MASK_ALIBI):
            last = max(kvlen - qlen + i for i in rows)
        else:
            last = kvlen - 1
        want = 0 if last < 0 else last // 64 + 1
        assert ktiles == want
    expect = {(b, h, i) for b, ql in enumerate(q_lens) for h in range(H) for i in range(ql)}
    assert set(covered) == expect


@pytest.mark.parametrize("seed", range(6))
def test_random_decode_plans(seed):
    rng = np.random.default_rng([314, 500, seed])
    B = int(rng.integers(1, 40))
    kv = rng.integers(0, 20000, size=B).tolist()
    ql = rng.integers(0, 2, size=B).tolist()
    if sum(ql) == 0:
        ql[0] = 1
    Hkv = int(rng.choice([1, 2, 8]))
    g = int(rng.choice([1, 4, 8, 24]))
    c = Case(q_lens=ql, kv_lens=kv, H=Hkv * g, Hkv=Hkv, D=128, bs=int(rng.choice([16, 32, 128])))
    info = c.plan()
    assert info["mode"] == "decode"
    _check_decode_plan(info, ql, kv, Hkv, g)


@pytest.mark.parametrize("mask", [pa.PA_MASK_NONE, pa.PA_MASK_CAUSAL, pa.PA_MASK_ALIBI])
def test_random_prefill_plans(mask):
    rng = np.random.default_rng([314, 501, mask])
    B = 5
    ql = [0, 1, 130, 700, 64]
    kv = [10, 0, 100, 3000, 64]
    c = Case(q_lens=ql, kv_lens=kv, H=4, Hkv=2, D=64, bs=16, dtype=pa.PA_F16, mask=mask)
    info = c.plan()
    assert info["mode"] == "prefill"
    _check_prefill_plan(info, ql, kv, 4, mask, 2)
    assert B == len(ql) and rng is not None


# -------------------------------------------------------- empty tensors

def test_empty_query_is_noop_and_skips_checks():
    c = Case(q_lens=[0, 0], kv_lens=[5, 9], H=4, Hkv=4, D=64, bs=16)
    c.H = 4
    c.Hkv = 3             # would be invalid, but empty tensors skip verification
    c.mask_type = 77
    info = c.plan()
    assert info["mode"] == "noop" and info["workspace_bytes"] == 0


def test_empty_key_value_plans_a_fill():
    c = Case(q_lens=[1, 1], kv_lens=[5, 9], H=4, Hkv=4, D=64, bs=16)
    c.key = desc([0, 16, 4, 64], pa.PA_F16)
    c.value = desc([0, 16, 4, 64], pa.PA_F16)
    info = c.plan()
    assert info["mode"] == "fill" and info["workspace_bytes"] == 0


# ---------------------------------------------------------- validation

def _expect(c, status, text=None):
    st, _, op = c.call()
    assert st == status, (st, pa.pa_last_error())
    assert op is None
    if text:
        assert text in pa.pa_last_error()


def base(**kw):
    args = dict(q_lens=[1, 1], kv_lens=[100, 37], H=8, Hkv=2, D=128, bs=16)
    args.update(kw)
    return Case(**args)


def test_null_arguments():
    c = base()
    c.query = None
    _expect(c, pa.PA_ERR_NULLPTR, "query")
    c = base()
    c.kv_seq_len = None
    _expect(c, pa.PA_ERR_NULLPTR, "kvSeqLen")
    lib = pa.load()
    assert lib.pa_paged_attention_get_workspace_size(
        *([None] * 8), 0, 1, 1, 1.0, None, None, None, None, None, None) == pa.PA_ERR_NULLPTR


def test_head_checks():
    c = base()
    c.H = 0
    _expect(c, pa.PA_ERR_PARAM_INVALID, "headNum")
    c = base(H=6, Hkv=4)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "multiple")
    c = base(D=96)
    _expect(c, pa.PA_ERR_UNSUPPORTED, "headSize")


def test_decode_wave_per_head_switch(monkeypatch):
    """Items of four kv heads only where kvHeadNum % 4 == 0 and a group has <= 16 heads;
    on by default for large batches, forced on / off by PA_OPT_DECODE_WAVE_HEADS."""
    for flag, H, Hkv, want in ((1, 16, 4, 1), (0, 16, 4, 0), (1, 12, 3, 0), (1, 68, 4, 0)):
        with pa.plan_options({pa.PA_OPT_DECODE_WAVE_HEADS: flag}):
            c = base(H=H, Hkv=Hkv)
            info = c.plan()
        assert info["decode_wave_heads"] == want, (flag, H, Hkv)
        _check_decode_plan(info, [1, 1], [100, 37], Hkv, H // Hkv)
    info = _plan_named("decode_int8_long")
    assert info["decode_wave_heads"] == 1
    info = _plan_named("decode_f16_small")
    assert info["decode_wave_heads"] == 0


def _i8_case(kmode, vmode, offsets, S=None):
    c = base(dtype=pa.PA_BF16, kv_dtype=pa.PA_I8, bs=32)
    c.extended = True
    c.kmode, c.vmode = kmode, vmode
    S = max(c.kv_lens) if S is None else S
    mk = lambda mode: desc([2, 128], pa.PA_F32) if mode == 0 else desc([2, S], pa.PA_F32)
    c.kscale, c.vscale = mk(kmode), mk(vmode)
    if offsets:
        c.koff, c.voff = mk(kmode), mk(vmode)
    return c


def test_antiquant_modes_and_offsets_plan():
    """Per-channel / per-token antiquant pairs the pages allow, with and without offsets."""
    for kmode, vmode in ((0, 0), (1, 1), (0, 1)):
        for offsets in (False, True):
            c = _i8_case(kmode, vmode, offsets)
            info = c.plan()
            assert info["antiquant"] == [kmode, vmode, int(offsets)]
            _check_decode_plan(info, [1, 1], [100, 37], 2, 4)
    # (1, batch, S) form and a larger S are accepted
    c = _i8_case(1, 1, True, S=160)
    c.kscale = desc([1, 2, 160], pa.PA_F32)
    c.koff = desc([1, 2, 160], pa.PA_F32)
    c.vscale = desc([1, 2, 160], pa.PA_F32)
    c.voff = desc([1, 2, 160], pa.PA_F32)
    assert c.plan()["antiquant"] == [1, 1, 1]


def test_antiquant_checks():
    # key per-token with value per-channel is not one of the pages' pairs
    _expect(_i8_case(1, 0, False), pa.PA_ERR_PARAM_INVALID, "modes")
    c = _i8_case(0, 0, False)
    c.kmode = 2
    _expect(c, pa.PA_ERR_PARAM_INVALID, "modes")
    # offsets come in pairs
    c = _i8_case(1, 1, True)
    c.voff = None
    _expect(c, pa.PA_ERR_PARAM_INVALID, "both")
    # per-token: f32 only, batch rows, S >= max kvSeqLen
    c = _i8_case(1, 1, False)
    c.kscale = desc([2, 100], pa.PA_BF16)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "f32")
    c = _i8_case(1, 1, False)
    c.kscale = desc([3, 100], pa.PA_F32)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "rows")
    c = _i8_case(1, 1, False, S=99)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "columns")
    # an offset's shape must match its scale's
    c = _i8_case(1, 1, True)
    c.koff = desc([2, 120], pa.PA_F32)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "shape")
    c = _i8_case(0, 0, True)
    c.koff = desc([2, 128], pa.PA_BF16)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "dtype")
    # antiquant parameters on a 16-bit cache
    c = base()
    c.extended = True
    c.kmode = c.vmode = 1
    _expect(c, pa.PA_ERR_PARAM_INVALID, "int8")
    c = base()
    c.extended = True
    c.koff = c.voff = desc([2, 128], pa.PA_F32)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "offsets")


def test_fp8_cache_plans_and_checks():
    """FLOAT8_E4M3FN K/V: per-channel scales required, no offsets, no per-token mode,
    blockSize a multiple of 32."""
    c = base(kv_dtype=pa.PA_F8E4M3, bs=32)
    c.kscale = desc([2, 128], pa.PA_F32)
    c.vscale = desc([2, 128], pa.PA_F32)
    info = c.plan()
    assert info["mode"] == "decode"
    _check_decode_plan(info, [1, 1], [100, 37], 2, 4)
    c = base(kv_dtype=pa.PA_F8E4M3, bs=32)
    c.kscale = c.vscale = None
    _expect(c, pa.PA_ERR_NULLPTR, "Scale")
    c = base(kv_dtype=pa.PA_F8E4M3, bs=16)
    c.kscale = desc([2, 128], pa.PA_F32)
    c.vscale = desc([2, 128], pa.PA_F32)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "multiple of 32")
    for kmode, vmode, offsets in ((1, 1, False), (0, 1, False), (0, 0, True)):
        c = _i8_case(kmode, vmode, offsets)
        c.key = desc(list(c.key.shape[:c.key.ndim]), pa.PA_F8E4M3)
        c.value = desc(list(c.value.shape[:c.value.ndim]), pa.PA_F8E4M3)
        _expect(c, pa.PA_ERR_PARAM_INVALID, "f8e4m3")


class AppendCase:
    """Descriptors for pa_kv_cache_append_plan (fake device pointers)."""

    def __init__(self, *, q_lens, kv_lens, Hkv=2, D=128, bs=16, dtype=pa.PA_BF16, width=None):
        T = int(sum(q_lens))
        need = sum(-(-k // bs) for k in kv_lens)
        W = max([-(-k // bs) for k in kv_lens] + [1]) if width is None else width
        self.knew = desc([T, Hkv, D], dtype)
        self.vnew = desc([T, Hkv, D], dtype)
        self.kc = desc([need + 1, bs, Hkv, D], dtype)
        self.vc = desc([need + 1, bs, Hkv, D], dtype)
        self.table = desc([len(q_lens), W], pa.PA_I32)
        self.seq_len, self._ql = host_i32(q_lens)
        self.kv_seq_len, self._kl = host_i32(kv_lens)

    def call(self):
        lib = pa.load()
        op = ctypes.c_void_p(None)
        r = lambda d: ctypes.byref(d) if d is not None else None
        st = lib.pa_kv_cache_append_plan(r(self.knew), r(self.vnew), r(self.kc), r(self.vc),
                                         r(self.table), r(self.seq_len), r(self.kv_seq_len),
                                         ctypes.byref(op))
        return st, op.value


def test_append_plan_covers_every_new_row_once():
    q_lens, kv_lens = [40, 0, 1, 17], [100, 5, 1, 17]
    c = AppendCase(q_lens=q_lens, kv_lens=kv_lens, bs=32)
    st, op = c.call()
    assert st == pa.PA_OK, pa.pa_last_error()
    info = pa.pa_op_describe(op)
    pa.pa_op_destroy(op)
    assert info["mode"] == "append"
    seen = {}
    for b, row0, pos0, count in info["append_items"]:
        assert 1 <= count <= 16
        for i in range(count):
            assert (row0 + i) not in seen
            seen[row0 + i] = (b, pos0 + i)
    row = 0
    for b, (q, k) in enumerate(zip(q_lens, kv_lens)):
        for i in range(q):
            assert seen[row] == (b, k - q + i)
            row += 1
    assert len(seen) == sum(q_lens)


def test_append_checks_and_op_kinds():
    def expect(c, status, text):
        st, op = c.call()
        assert st == status and op is None, (st, pa.pa_last_error())
        assert text in pa.pa_last_error()
    expect(AppendCase(q_lens=[5, 1], kv_lens=[4, 3]), pa.PA_ERR_PARAM_INVALID, "seqLen")
    c = AppendCase(q_lens=[2, 1], kv_lens=[40, 3])
    c.vc = desc([20, 16, 2, 128], pa.PA_F16)
    expect(c, pa.PA_ERR_PARAM_INVALID, "dtype")
    expect(AppendCase(q_lens=[2, 1], kv_lens=[40, 3], width=2), pa.PA_ERR_PARAM_INVALID, "columns")
    c = AppendCase(q_lens=[2, 1], kv_lens=[40, 3])
    c.knew = desc([4, 2, 128], pa.PA_BF16)
    expect(c, pa.PA_ERR_PARAM_INVALID, "shapes differ")
    c = AppendCase(q_lens=[2, 1], kv_lens=[40, 3])
    c.knew = c.vnew = desc([3, 256], pa.PA_BF16)
    expect(c, pa.PA_ERR_PARAM_INVALID, "nTokens, kvHeadNum, headSize")
    # an append op cannot run as attention, nor an attention op as an append
    st, op = AppendCase(q_lens=[2], kv_lens=[9]).call()
    assert st == pa.PA_OK
    lib = pa.load()
    assert lib.pa_paged_attention(None, 0, op, None) == pa.PA_ERR_PARAM_INVALID
    assert "append" in pa.pa_last_error()
    pa.pa_op_destroy(op)
    st, _, aop = base().call()
    assert st == pa.PA_OK
    assert lib.pa_kv_cache_append(aop, None) == pa.PA_ERR_PARAM_INVALID
    pa.pa_op_destroy(aop)
    # no new tokens: a no-op plan
    st, op = AppendCase(q_lens=[0, 0], kv_lens=[3, 0]).call()
    assert st == pa.PA_OK and pa.pa_op_describe(op)["mode"] == "noop"
    pa.pa_op_destroy(op)


def test_kv_head_num_zero_means_head_num():
    c = base(H=4, Hkv=4)
    c.Hkv = 0
    info = c.plan()
    assert info["mode"] == "decode"
    # every kv head 0..3 is covered (by 4-head items or one item per head)
    assert {it[1] + w for it in info["decode_items"] for w in range(it[8])} == {0, 1, 2, 3}


def test_mask_checks():
    for m in (4, 5):
        c = base()
        c.mask_type = m
        _expect(c, pa.PA_ERR_UNSUPPORTED, "maskType")
    c = base()
    c.mask_type = 7
    _expect(c, pa.PA_ERR_PARAM_INVALID, "maskType")
    c = base()
    c.mask_type = pa.PA_MASK_ALIBI
    _expect(c, pa.PA_ERR_NULLPTR, "slopes")
    c = base()
    c.slopes = desc([8], pa.PA_F32)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "slopes")
    c = base(mask=pa.PA_MASK_ALIBI)
    c.slopes = desc([7], pa.PA_F32)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "slopes")
    c = base()
    c.mask = desc([256, 256], pa.PA_F16)
    _expect(c, pa.PA_ERR_UNSUPPORTED, "mask")


def test_length_and_table_checks():
    c = base()
    c.seq_len, c._ql = host_i32([1, 2])
    _expect(c, pa.PA_ERR_PARAM_INVALID, "sum(seqLen)")
    c = base()
    c.kv_seq_len, c._kl = host_i32([100, -1])
    _expect(c, pa.PA_ERR_PARAM_INVALID, "kvSeqLen[1]")
    c = base(width=6)                       # 100 tokens need 7 blocks of 16
    _expect(c, pa.PA_ERR_PARAM_INVALID, "columns")
    c = base(num_blocks=9)                  # need 7 + 3 = 10 blocks
    _expect(c, pa.PA_ERR_PARAM_INVALID, "numBlocks")
    c = base(bs=24)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "blockSize")
    c = base(kv_dtype=pa.PA_I8, bs=16)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "blockSize")   # int8 needs a multiple of 32
    c = base()
    c.table = desc([2, 7], pa.PA_F32)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "int32")


def test_dtype_and_layout_checks():
    c = base()
    c.out = desc([2, 8, 128], pa.PA_F16)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "attnOut dtype")
    c = base()
    c.key = desc([10, 16, 2, 128], pa.PA_F16)
    c.value = desc([10, 16, 2, 128], pa.PA_F16)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "key dtype")
    c = base(kv_dtype=pa.PA_I8, bs=32)
    c.kscale = None
    _expect(c, pa.PA_ERR_NULLPTR, "AntiquantScale")
    c = base(kv_dtype=pa.PA_I8, bs=32)
    c.vscale = desc([2, 64], pa.PA_F32)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "elements")
    c = base()
    c.kscale = desc([2, 128], pa.PA_F32)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "non-int8")
    c = base()
    c.lse = desc([2, 7], pa.PA_F32)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "lse")
    c = base()
    c.query = desc([2, 8, 128], pa.PA_BF16, ptr=FAKE + 8)
    _expect(c, pa.PA_ERR_PARAM_INVALID, "aligned")
    c = base()
    c.scale = float("nan")
    _expect(c, pa.PA_ERR_PARAM_INVALID, "qkScale")


def test_strided_views_are_accepted():
    # query as a slice of a fused [T, H + 2*Hkv, D] projection; out heads padded;
    # key/value as a permuted (numBlocks, kvHeadNum, blockSize, headSize) cache
    c = base()
    c.query = desc([2, 8, 128], pa.PA_BF16, strides=[12 * 128, 128, 1])
    c.out = desc([2, 8, 128], pa.PA_BF16, strides=[8 * 136, 136, 1])
    c.key = desc([10, 16, 2, 128], pa.PA_BF16, strides=[2 * 16 * 128, 128, 16 * 128, 1])
    c.value = desc([10, 16, 2, 128], pa.PA_BF16, strides=[2 * 16 * 128, 128, 16 * 128, 1])
    assert c.plan()["mode"] == "decode"
    c2 = base()
    c2.out = desc([2, 8, 128], pa.PA_BF16, strides=[64, 128, 1])
    _expect(c2, pa.PA_ERR_PARAM_INVALID, "overlap")


def test_two_dimensional_forms():
    c = base()
    c.query = desc([2, 8 * 128], pa.PA_BF16)
    c.out = desc([2, 8 * 128], pa.PA_BF16)
    c.key = desc([10, 16, 2 * 128], pa.PA_BF16)
    c.value = desc([10, 16, 2 * 128], pa.PA_BF16)
    assert c.plan()["mode"] == "decode"


# ----------------------------------------------- phase 2 without a GPU call

def test_execute_argument_errors():
    lib = pa.load()
    assert lib.pa_paged_attention(None, 0, None, None) == pa.PA_ERR_NULLPTR
    c = base(kv_lens=[20000, 37])           # long enough to be split: needs partials
    st, ws, op = c.call()
    assert st == pa.PA_OK and ws > 0
    assert lib.pa_paged_attention(FAKE, ws - 1, op, None) == pa.PA_ERR_WORKSPACE_TOO_SMALL
    assert lib.pa_paged_attention(None, ws, op, None) == pa.PA_ERR_NULLPTR
    assert lib.pa_paged_attention(FAKE + 16, ws, op, None) == pa.PA_ERR_PARAM_INVALID
    lib.pa_op_destroy(op)
    lib.pa_op_destroy(None)
    c = Case(q_lens=[0], kv_lens=[3], H=2, Hkv=2, D=64, bs=16)
    st, ws, op = c.call()
    assert st == pa.PA_OK and ws == 0
    assert lib.pa_paged_attention(None, 0, op, None) == pa.PA_OK     # no-op, no HIP call
    lib.pa_op_destroy(op)


# ----------------------------------------------------------- plan options

def test_plan_options_are_declared_and_validated():
    """The planner's tuning overrides are an explicit, declared call (not read from the
    environment); out-of-range values and unknown options are refused."""
    for opt in range(pa.PA_OPT_DECODE_CHUNK_TILES, pa.PA_OPT_COMPUTE_UNITS + 1):
        assert pa.pa_get_plan_option(opt) == -1
    lib = pa.load()
    assert lib.pa_set_plan_option(0, 1) == pa.PA_ERR_PARAM_INVALID
    assert lib.pa_set_plan_option(7, 1) == pa.PA_ERR_PARAM_INVALID
    assert lib.pa_set_plan_option(pa.PA_OPT_DECODE_WAVE_HEADS, 2) == pa.PA_ERR_PARAM_INVALID
    assert lib.pa_set_plan_option(pa.PA_OPT_DECODE_CHUNK_TILES, 0) == pa.PA_ERR_PARAM_INVALID
    assert lib.pa_set_plan_option(pa.PA_OPT_COMPUTE_UNITS, -2) == pa.PA_ERR_PARAM_INVALID
    with pa.plan_options({pa.PA_OPT_DECODE_CHUNK_TILES: 12}):
        assert pa.pa_get_plan_option(pa.PA_OPT_DECODE_CHUNK_TILES) == 12
        assert base(kv_lens=[3000, 37]).plan()["chunk_tiles"] == 12
    assert pa.pa_get_plan_option(pa.PA_OPT_DECODE_CHUNK_TILES) == -1


def test_default_plan_ignores_environment(monkeypatch):
    """Variables named like the planner's options change nothing: the default plan is a
    function of the call's arguments and the device size only."""
    cases = [lambda: base(kv_lens=[3000, 37, 9000], q_lens=[1, 1, 1]),
             lambda: Case(q_lens=[300, 70], kv_lens=[800, 70], H=8, Hkv=2, D=128, bs=64,
                          mask=pa.PA_MASK_CAUSAL)]
    before = [c().plan() for c in cases]
    for name in ("PA_DECODE_CHUNK_TILES", "PA_DECODE_TARGET_ITEMS", "PA_DECODE_WAVE_HEADS",
                 "PA_PREFILL_PAIR", "PA_PREFILL_XCD_ORDER", "PA_COMPUTE_UNITS"):
        monkeypatch.setenv(name, "1")
    after = [c().plan() for c in cases]
    assert before == after


def test_workspace_holds_only_split_partials():
    """The device workspace holds the split partials (fp32 O [slots, heads, D] and
    (m, l) [slots, heads, 2]) and the 32-byte combine items, each region 256-aligned;
    the work lists (32-byte prefill items, 48-byte decode items) live in the op's
    pinned buffer."""
    info = base(kv_lens=[100, 37]).plan()                     # short: no split
    n = len(info["decode_items"])
    assert info["partial_slots"] == 0 and info["workspace_bytes"] == 0
    assert info["items_bytes"] == -(-48 * n // 256) * 256
    info = base(kv_lens=[30000, 37]).plan()                   # long: split + combine
    assert info["partial_slots"] > 0
    n, m = len(info["decode_items"]), len(info["combine_items"])
    assert info["items_bytes"] == -(-48 * n // 256) * 256
    o = -(-info["partial_slots"] * 4 * 128 * 4 // 256) * 256
    ml = -(-info["partial_slots"] * 4 * 2 * 4 // 256) * 256
    assert info["workspace_bytes"] == o + ml + -(-32 * m // 256) * 256
    info = Case(q_lens=[300], kv_lens=[300], H=4, Hkv=4, D=64, bs=16,
                mask=pa.PA_MASK_CAUSAL).plan()
    assert info["workspace_bytes"] == 0
    assert info["items_bytes"] == -(-len(info["prefill_items"]) * 32 // 256) * 256


@pytest.mark.parametrize("cus", [32, 64, 128, 256, 80])
def test_plans_for_smaller_devices(cus):
    """A partitioned GPU (whole XCDs of 32 CUs) or any other size: the prefill list is
    ordered for that many XCDs and still covers every row once; decode splits aim at
    that many CUs."""
    with pa.plan_options({pa.PA_OPT_COMPUTE_UNITS: cus}):
        c = Case(q_lens=[512, 512, 300], kv_lens=[512, 2560, 300], H=32, Hkv=8, D=128,
                 bs=128, mask=pa.PA_MASK_CAUSAL)
        info = c.plan()
        assert info["compute_units"] == cus
        _check_prefill_plan(info, [512, 512, 300], [512, 2560, 300], 32, pa.PA_MASK_CAUSAL, 4)
        d = base(kv_lens=[8000] * 16, q_lens=[1] * 16)
        dinfo = d.plan()
        _check_decode_plan(dinfo, [1] * 16, [8000] * 16, 2, 4)



@pytest.mark.parametrize("cus", [256, 80])
def test_decode_items_per_cu_and_near_equal(cus):
    """Wave-per-head decode items: one per CU when the sequence lengths are nearly equal,
    three per CU when they are not (at least one split per sequence), shared out by
    largest remainder so that the longest item stays near the mean; a forced chunk
    length or item target still applies."""
    with pa.plan_options({pa.PA_OPT_COMPUTE_UNITS: cus}):
        rng = np.random.default_rng(7)
        uneven = rng.integers(1024, 8193, size=64).tolist()
        for kv, per_cu in (([4608] * 64, 1), (uneven, 3)):
            c = Case(q_lens=[1] * 64, kv_lens=kv, H=32, Hkv=8, D=128, bs=128,
                     dtype=pa.PA_BF16, kv_dtype=pa.PA_BF16)
            info = c.plan()
            _check_decode_plan(info, [1] * 64, kv, 8, 4)
            items = info["decode_items"]
            # an item covers four of the 8 kv heads, and every sequence takes a split
            assert len(items) == 2 * max(64, (per_cu * cus + 1) // 2)
            lens = [it[4] - it[3] for it in items]
            # the longest item (which bounds the launch) is as short as the count allows:
            # taking a split away from any sequence would leave an item at least as long
            nsplit = {it[0]: it[11] for it in items}
            tiles = {b: -(-kv[b] // 32) for b in nsplit}
            longest = max(lens)
            assert longest == max(-(-tiles[b] // nsplit[b]) for b in nsplit)
            for b, m in nsplit.items():
                if m > 1:
                    assert -(-tiles[b] // (m - 1)) >= longest, (b, m, tiles[b], longest)
            if per_cu == 1:
                assert max(lens) == min(lens)
            assert lens == sorted(lens, reverse=True)            # longest first
        with pa.plan_options({pa.PA_OPT_DECODE_CHUNK_TILES: 40}):
            info = c.plan()
            _check_decode_plan(info, [1] * 64, uneven, 8, 4)
            assert max(it[4] - it[3] for it in info["decode_items"]) <= 40
        with pa.plan_options({pa.PA_OPT_DECODE_TARGET_ITEMS: 1000}):
            info = c.plan()
            assert len(info["decode_items"]) == 1000


def test_timing_events_name_a_kernel_of_the_op():
    """Timing events attach to the main kernel or the split-KV combine; other indices and
    a NULL op are refused (host only, no HIP call)."""
    st, _, op = base().call()
    assert st == pa.PA_OK
    lib = pa.load()
    for k in (pa.PA_TIMED_MAIN, pa.PA_TIMED_COMBINE):
        assert lib.pa_op_set_timing_events(op, k, None, None) == pa.PA_OK
    assert lib.pa_op_set_timing_events(op, 2, None, None) == pa.PA_ERR_PARAM_INVALID
    assert lib.pa_op_set_timing_events(None, 0, None, None) == pa.PA_ERR_NULLPTR
    pa.pa_op_destroy(op)


def test_static_execute_refuses_ops_beyond_its_scratch():
    """pa_paged_attention_static holds 64 MiB of scratch: an op planned with a larger
    workspace is refused before any HIP call (split partials of 8 sequences of 200k
    tokens cut into single tiles need about 200 MB)."""
    with pa.plan_options({pa.PA_OPT_DECODE_CHUNK_TILES: 1}):
        c = base(q_lens=[1] * 8, kv_lens=[200000] * 8, H=8, Hkv=2)
        st, ws, op = c.call()
    assert st == pa.PA_OK and ws > 64 << 20
    lib = pa.load()
    assert lib.pa_paged_attention_static(op, None) == pa.PA_ERR_WORKSPACE_TOO_SMALL
    assert "static scratch" in pa.pa_last_error()
    assert lib.pa_paged_attention_static(None, None) == pa.PA_ERR_NULLPTR
    pa.pa_op_destroy(op)
    st, aop = AppendCase(q_lens=[2], kv_lens=[9]).call()
    assert lib.pa_paged_attention_static(aop, None) == pa.PA_ERR_PARAM_INVALID
    pa.pa_op_destroy(aop)


# ------------------------------------------------------------ counter records

def test_counter_records_key_on_code_not_comments(tmp_path, monkeypatch):
    """profiles/*_counters.json are keyed by a hash of the kernels' and the planner's code
    (bench.py reports a record's traffic and executed work only while its key matches):
    a comment or blank-space edit keeps the key, a code edit changes it."""
    import shutil

    from paged_kv_cache_314_amd import counter_summary as cs

    assert cs.code_text("int a; // note\n/* block\n comment */\n\n  int  b;") == "int a; int b;"
    # edits on a copy of the sources
    src = tmp_path / "csrc"
    shutil.copytree(cs.CSRC, src)
    monkeypatch.setattr(cs, "CSRC", str(src))
    base = cs.kernel_source_hash("prefill_kernel")
    p = src / "prefill.hip"
    text = p.read_text()
    p.write_text("// a new comment line\n" + text.replace("\n", "\n\n", 3))
    assert cs.kernel_source_hash("prefill_kernel") == base
    p.write_text(text.replace("constexpr int BN = kPrefillBN;", "constexpr int BN = kPrefillBN + 0;"))
    assert cs.kernel_source_hash("prefill_kernel") != base
