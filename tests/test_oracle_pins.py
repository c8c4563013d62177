"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

None of these re-types the oracle's formula.  Each pins the oracle against
something else: hand-worked examples (tests/golden), a scalar brute-force
twin written separately (tests/brute_force.py), a library routine
(torch's scaled_dot_product_attention on CPU fp64) for the special cases it
covers, closed forms, and invariants the pages state (paged layout equals the
contiguous one, GQA equals repeated KV heads, empty-tensor rules, the lse
decomposition used by ring attention).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import MASK_ALIBI, MASK_CAUSAL, MASK_NONE
from tests.brute_force import brute_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
TIGHT = 1e-12


# ----------------------------------------------------------------- helpers

def _val(x):
    if x is None:
        return math.nan
    if isinstance(x, (int, float)):
        return float(x)
    x = x.strip()
    if x == "inf":
        return math.inf
    if x.startswith("ln "):
        arg = x[3:].strip()
        return math.log(float(Fraction(arg)))
    return float(Fraction(x))


def _arr(nested):
    if isinstance(nested, list):
        return [_arr(v) for v in nested]
    return _val(nested)


def _random_case(rng, *, B, H, Hkv, D, bs, mask, int8=False, max_kv=12, allow_empty=True):
    q_lens, kv_lens = [], []
    for _ in range(B):
        kv = int(rng.integers(0 if allow_empty else 1, max_kv + 1))
        if mask == "decode":
            ql = 1
        else:
            ql = int(rng.integers(0, 4))
        q_lens.append(ql)
        kv_lens.append(kv)
    need = [-(-k // bs) for k in kv_lens]
    nb = sum(need) + 2
    perm = rng.permutation(nb)
    width = max(need + [1]) + 1
    table = np.full((B, width), -1, dtype=np.int64)
    pos = 0
    for b in range(B):
        table[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    T = sum(q_lens)
    q = rng.standard_normal((T, H, D))
    if int8:
        k = rng.integers(-127, 128, size=(nb, bs, Hkv, D)).astype(np.float64)
        v = rng.integers(-127, 128, size=(nb, bs, Hkv, D)).astype(np.float64)
        ks = rng.uniform(0.005, 0.02, size=(Hkv, D))
        vs = rng.uniform(0.005, 0.02, size=(Hkv, D))
    else:
        k = rng.standard_normal((nb, bs, Hkv, D))
        v = rng.standard_normal((nb, bs, Hkv, D))
        ks = vs = None
    slopes = rng.uniform(0.0, 1.0, size=H)
    return dict(q=q, k=k, v=v, table=table, q_lens=q_lens, kv_lens=kv_lens,
                slopes=slopes, ks=ks, vs=vs)


def _oracle(c, mask_type, H, Hkv, scale):
    return oracle.paged_attention(
        c["q"], c["k"], c["v"], c["table"], c["q_lens"], c["kv_lens"], mask_type,
        H, Hkv, scale, slopes=c["slopes"], key_antiquant_scale=c["ks"],
        value_antiquant_scale=c["vs"])


def _same(a, b, tol=TIGHT):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), "inf pattern differs"
    assert np.array_equal(a[~fin], b[~fin])
    if fin.any():
        assert np.max(np.abs(a[fin] - b[fin])) <= tol * max(1.0, np.max(np.abs(b[fin])))


# ------------------------------------------------------- golden examples

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _pool(blocks, kv_heads, head_size):
    """Nested [block][slot][kvHead][d]; a null slot is one never to be read (NaN)."""
    nan_slot = [[math.nan] * head_size for _ in range(kv_heads)]
    return np.array([[nan_slot if slot in (None, [None]) else _arr(slot) for slot in blk]
                     for blk in blocks], dtype=np.float64)


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_worked_examples(case):
    D = len(case["query"][0][0])
    Hkv = case["kv_head_num"]
    key = _pool(case["key"], Hkv, D)
    value = _pool(case["value"], Hkv, D)
    query = np.array(_arr(case["query"]), dtype=np.float64)
    slopes = np.array(_arr(case["slopes"])) if "slopes" in case else None
    ks = np.array(_arr(case["key_scale"])) if "key_scale" in case else None
    vs = np.array(_arr(case["value_scale"])) if "value_scale" in case else None
    out, lse = oracle.paged_attention(
        query, key, value, np.array(case["block_tables"]), case["seq_len"],
        case["kv_seq_len"], case["mask_type"], case["head_num"], case["kv_head_num"],
        _val(case["qk_scale"]), slopes=slopes, key_antiquant_scale=ks,
        value_antiquant_scale=vs)
    _same(out, np.array(_arr(case["out"])), 1e-14)
    _same(lse, np.array(_arr(case["lse"])), 1e-14)


# ------------------------------------------------------------ brute force

@pytest.mark.parametrize("seed", range(12))
def test_brute_force_agrees(seed):
    rng = np.random.default_rng([314, 77, seed])
    H, Hkv = [(1, 1), (2, 1), (4, 2), (4, 4)][seed % 4]
    mask = [MASK_NONE, MASK_CAUSAL, MASK_ALIBI][seed % 3]
    int8 = seed % 5 == 4
    bs = [1, 2, 4][seed % 3]
    D = [1, 3, 8][seed % 3]
    c = _random_case(rng, B=2, H=H, Hkv=Hkv, D=D, bs=bs,
                     mask="decode" if seed % 6 == 0 else mask, int8=int8)
    scale = float(rng.uniform(0.1, 1.5))
    out, lse = _oracle(c, mask, H, Hkv, scale)
    bo, bl = brute_attention(
        c["q"].tolist(), c["k"].tolist(), c["v"].tolist(), c["table"].tolist(),
        c["q_lens"], c["kv_lens"], mask, H, Hkv, scale, slopes=c["slopes"].tolist(),
        key_scale=None if c["ks"] is None else c["ks"].tolist(),
        value_scale=None if c["vs"] is None else c["vs"].tolist())
    _same(out, np.array(bo).reshape(out.shape))
    _same(lse, np.array(bl).reshape(lse.shape))


# ---------------------------------------------------- library special case

def _sdpa_reference(q, k, v, positions, mask, scale, slopes, H, Hkv):
    """torch SDPA in fp64 with an explicit bottom-right additive mask."""
    g = H // Hkv
    kk = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2)   # [H, kv, D]
    vv = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2)
    qq = torch.from_numpy(q).permute(1, 0, 2)                         # [H, nq, D]
    j = torch.arange(k.shape[0], dtype=torch.float64)
    p = torch.from_numpy(positions.astype(np.float64))
    bias = torch.zeros((H, q.shape[0], k.shape[0]), dtype=torch.float64)
    if mask == MASK_ALIBI:
        bias += torch.from_numpy(slopes)[:, None, None] * (j[None, None, :] - p[None, :, None])
    if mask in (MASK_ALIBI, MASK_CAUSAL):
        bias = bias.masked_fill(j[None, None, :] > p[None, :, None], -math.inf)
    out = torch.nn.functional.scaled_dot_product_attention(
        qq, kk, vv, attn_mask=bias, scale=scale)
    return out.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("mask", [MASK_NONE, MASK_CAUSAL, MASK_ALIBI])
@pytest.mark.parametrize("heads", [(4, 4), (8, 2)])
def test_matches_torch_sdpa(mask, heads):
    H, Hkv = heads
    rng = np.random.default_rng([314, 78, mask, H])
    kv, nq, D = 37, 9, 16
    q = rng.standard_normal((nq, H, D))
    k = rng.standard_normal((kv, Hkv, D))
    v = rng.standard_normal((kv, Hkv, D))
    slopes = rng.uniform(0, 1, H)
    positions = oracle.query_positions(nq, kv)
    out, _ = oracle.attention_contiguous(q, k, v, positions, mask, 0.37, H, Hkv, slopes)
    ref = _sdpa_reference(q, k, v, positions, mask, 0.37, slopes, H, Hkv)
    _same(out, ref)


# ----------------------------------------------------------- closed forms

def test_causal_zero_query_closed_form():
    """Q = 0: every visible score is 0, so out_i = mean(V[0..p_i]), lse = ln(p_i+1)."""
    rng = np.random.default_rng([314, 79])
    kv, nq, D = 20, 6, 4
    q = np.zeros((nq, 1, D))
    k = rng.standard_normal((kv, 1, D))
    v = rng.standard_normal((kv, 1, D))
    pos = oracle.query_positions(nq, kv)
    out, lse = oracle.attention_contiguous(q, k, v, pos, MASK_CAUSAL, 0.5, 1, 1)
    for i, p in enumerate(pos):
        np.testing.assert_allclose(out[i, 0], v[:p + 1, 0].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[i, 0] - math.log(p + 1)) < 1e-14


def test_alibi_zero_query_closed_form():
    """Q = 0 with slope s: weights e^{-s k} for distance k = p - j, a geometric series."""
    rng = np.random.default_rng([314, 80])
    kv, nq, D, s = 15, 4, 3, 0.7
    q = np.zeros((nq, 1, D))
    k = rng.standard_normal((kv, 1, D))
    v = rng.standard_normal((kv, 1, D))
    pos = oracle.query_positions(nq, kv)
    out, lse = oracle.attention_contiguous(q, k, v, pos, MASK_ALIBI, 1.3, 1, 1, [s])
    for i, p in enumerate(pos):
        total = (1 - math.exp(-s * (p + 1))) / (1 - math.exp(-s))
        assert abs(lse[i, 0] - math.log(total)) < 1e-13
        want = sum(math.exp(-s * d) * v[p - d, 0] for d in range(p + 1)) / total
        np.testing.assert_allclose(out[i, 0], want, rtol=0, atol=1e-13)


def test_one_hot_values_expose_softmax_row():
    """V[t] = e_t turns out into the probability row: it sums to 1 and
    equals exp(s_j - lse) (lse definition of the softmaxLse restriction)."""
    rng = np.random.default_rng([314, 81])
    kv, D = 11, 16
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((kv, 1, D))
    v = np.zeros((kv, 1, D))
    v[np.arange(kv), 0, np.arange(kv)] = 1.0
    out, lse = oracle.attention_contiguous(q, k, v, [kv - 1], MASK_NONE, 0.9, 1, 1)
    prob = out[0, 0, :kv]
    assert abs(prob.sum() - 1.0) < 1e-12
    assert np.all(out[0, 0, kv:] == 0)
    s = 0.9 * (k[:, 0, :] @ q[0, 0])
    np.testing.assert_allclose(prob, np.exp(s - lse[0, 0]), rtol=1e-12, atol=0)


def test_constant_values_give_constant_output():
    rng = np.random.default_rng([314, 82])
    c = _random_case(rng, B=3, H=4, Hkv=2, D=5, bs=4, mask=MASK_CAUSAL, allow_empty=False)
    c["v"][:] = 2.75
    out, lse = _oracle(c, MASK_CAUSAL, 4, 2, 0.6)
    seen = np.isfinite(lse)
    assert seen.any()
    np.testing.assert_allclose(out[seen], 2.75, rtol=0, atol=1e-13)


def test_single_key_returns_its_value_row():
    rng = np.random.default_rng([314, 83])
    D = 6
    q = rng.standard_normal((1, 2, D))
    k = rng.standard_normal((1, 1, D))
    v = rng.standard_normal((1, 1, D))
    out, lse = oracle.attention_contiguous(q, k, v, [0], MASK_NONE, 0.25, 2, 1)
    for h in range(2):
        np.testing.assert_array_equal(out[0, h], v[0, 0])
        assert abs(lse[0, h] - 0.25 * float(q[0, h] @ k[0, 0])) < 1e-15


# ------------------------------------------------------------- invariants

def test_paged_equals_contiguous_and_ignores_unused_slots():
    """Paged layout = the blocks of blockTables laid end to end; unused
    blocks, tail slots and -1 table padding are never read."""
    rng = np.random.default_rng([314, 84])
    B, H, Hkv, D, bs = 3, 4, 2, 8, 4
    c = _random_case(rng, B=B, H=H, Hkv=Hkv, D=D, bs=bs, mask=MASK_ALIBI, allow_empty=False)
    out, lse = _oracle(c, MASK_ALIBI, H, Hkv, 0.4)
    # poison every slot no sequence owns
    used = np.zeros(c["k"].shape[:2], dtype=bool)
    for b in range(B):
        for t in range(c["kv_lens"][b]):
            used[c["table"][b, t // bs], t % bs] = True
    pk, pv = c["k"].copy(), c["v"].copy()
    pk[~used] = np.nan
    pv[~used] = np.nan
    p_out, p_lse = oracle.paged_attention(
        c["q"], pk, pv, c["table"], c["q_lens"], c["kv_lens"], MASK_ALIBI, H, Hkv, 0.4,
        slopes=c["slopes"])
    assert np.array_equal(p_out, out) and np.array_equal(p_lse, lse)
    # per-sequence contiguous computation
    q0 = 0
    for b in range(B):
        rows = []
        for t in range(c["kv_lens"][b]):
            rows.append(c["k"][c["table"][b, t // bs], t % bs])
        kc = np.array(rows).reshape(-1, Hkv, D)
        vc = np.array([c["v"][c["table"][b, t // bs], t % bs]
                       for t in range(c["kv_lens"][b])]).reshape(-1, Hkv, D)
        ql = c["q_lens"][b]
        o_b, l_b = oracle.attention_contiguous(
            c["q"][q0:q0 + ql], kc, vc, oracle.query_positions(ql, c["kv_lens"][b]),
            MASK_ALIBI, 0.4, H, Hkv, c["slopes"])
        assert np.array_equal(o_b, out[q0:q0 + ql])
        q0 += ql
    # permuting the physical blocks together with the table changes nothing
    perm = rng.permutation(c["k"].shape[0])
    inv = np.argsort(perm)
    tab = np.where(c["table"] >= 0, inv[np.maximum(c["table"], 0)], -1)
    r_out, r_lse = oracle.paged_attention(
        c["q"], c["k"][perm], c["v"][perm], tab, c["q_lens"], c["kv_lens"], MASK_ALIBI,
        H, Hkv, 0.4, slopes=c["slopes"])
    _same(r_out, out)
    _same(r_lse, lse)


def test_alibi_with_zero_slopes_is_causal():
    rng = np.random.default_rng([314, 85])
    c = _random_case(rng, B=3, H=2, Hkv=1, D=4, bs=2, mask=MASK_CAUSAL)
    c["slopes"] = np.zeros(2)
    a = _oracle(c, MASK_ALIBI, 2, 1, 0.8)
    b = _oracle(c, MASK_CAUSAL, 2, 1, 0.8)
    _same(a[0], b[0])
    _same(a[1], b[1])


def test_alibi_row_shift_changes_lse_only():
    """Adding the same constant to a row's bias leaves out unchanged: the
    out of maskType 3 does not depend on where the bias is anchored."""
    rng = np.random.default_rng([314, 86])
    kv, nq, D = 13, 5, 4
    q = rng.standard_normal((nq, 1, D))
    k = rng.standard_normal((kv, 1, D))
    v = rng.standard_normal((kv, 1, D))
    pos = oracle.query_positions(nq, kv)
    o1, l1 = oracle.attention_contiguous(q, k, v, pos, MASK_ALIBI, 0.5, 1, 1, [0.3])
    # the same causal pattern with a bias anchored at key 0 instead of p_i
    out2 = np.zeros_like(o1)
    for i, p in enumerate(pos):
        s = 0.5 * (k[:p + 1, 0] @ q[i, 0]) + 0.3 * np.arange(p + 1)
        e = np.exp(s - s.max())
        out2[i, 0] = e @ v[:p + 1, 0] / e.sum()
    np.testing.assert_allclose(o1, out2, rtol=0, atol=1e-13)


def test_scale_invariance():
    rng = np.random.default_rng([314, 87])
    c = _random_case(rng, B=2, H=4, Hkv=4, D=6, bs=3, mask=MASK_ALIBI)
    a = _oracle(c, MASK_ALIBI, 4, 4, 0.5)
    c2 = dict(c, q=c["q"] * 4.0)
    b = _oracle(c2, MASK_ALIBI, 4, 4, 0.125)
    _same(a[0], b[0], 1e-12)
    _same(a[1], b[1], 1e-12)


def test_gqa_equals_repeated_kv_heads():
    rng = np.random.default_rng([314, 88])
    H, Hkv = 8, 2
    c = _random_case(rng, B=3, H=H, Hkv=Hkv, D=5, bs=2, mask=MASK_CAUSAL)
    a = _oracle(c, MASK_CAUSAL, H, Hkv, 0.7)
    c2 = dict(c, k=np.repeat(c["k"], H // Hkv, axis=2), v=np.repeat(c["v"], H // Hkv, axis=2))
    b = _oracle(c2, MASK_CAUSAL, H, H, 0.7)
    _same(a[0], b[0])
    _same(a[1], b[1])
    # kvHeadNum = 0 means kvHeadNum = headNum
    d0 = _oracle(c2, MASK_CAUSAL, H, 0, 0.7)
    _same(d0[0], b[0])


def test_int8_equals_float_on_dequantised_pool():
    rng = np.random.default_rng([314, 89])
    c = _random_case(rng, B=2, H=4, Hkv=2, D=6, bs=4, mask=MASK_NONE, int8=True)
    a = _oracle(c, MASK_NONE, 4, 2, 0.3)
    kf = c["k"] * c["ks"][None, None]
    vf = c["v"] * c["vs"][None, None]
    b = oracle.paged_attention(c["q"], kf, vf, c["table"], c["q_lens"], c["kv_lens"],
                               MASK_NONE, 4, 2, 0.3)
    _same(a[0], b[0])
    _same(a[1], b[1])
    # dequant multiplies per (kv head, channel), not per token or transposed
    x = np.arange(2 * 3, dtype=np.int64).reshape(1, 2, 3) - 3
    sc = np.array([[1.0, 2.0, 4.0], [8.0, 16.0, 32.0]])
    np.testing.assert_array_equal(oracle.dequantize_per_channel(x, sc),
                                  [[[-3.0, -4.0, -4.0], [0.0, 16.0, 64.0]]])


def _antiquant_case(rng, *, kmode, vmode, offsets, B=2, H=4, Hkv=2, D=5, bs=4, max_kv=11):
    """A random int8 case with scales (and offsets) in the given modes: per-channel
    [Hkv, D] or per-token [B, S] with S = max kv + 3 (entries past kv never used)."""
    c = _random_case(rng, B=B, H=H, Hkv=Hkv, D=D, bs=bs, mask=MASK_NONE, int8=True,
                     max_kv=max_kv)
    S = max(c["kv_lens"]) + 3

    def draw(mode, lo, hi):
        return rng.uniform(lo, hi, size=(Hkv, D) if mode == 0 else (B, S))
    c["ks"], c["vs"] = draw(kmode, 0.005, 0.02), draw(vmode, 0.005, 0.02)
    c["ko"] = draw(kmode, -20.0, 20.0) if offsets else None
    c["vo"] = draw(vmode, -20.0, 20.0) if offsets else None
    c["kmode"], c["vmode"] = kmode, vmode
    return c


def _oracle_aq(c, mask_type, H, Hkv, scale):
    return oracle.paged_attention(
        c["q"], c["k"], c["v"], c["table"], c["q_lens"], c["kv_lens"], mask_type, H, Hkv,
        scale, slopes=c["slopes"], key_antiquant_scale=c["ks"], value_antiquant_scale=c["vs"],
        key_antiquant_offset=c["ko"], value_antiquant_offset=c["vo"],
        key_antiquant_mode=c["kmode"], value_antiquant_mode=c["vmode"])


@pytest.mark.parametrize("seed", range(9))
def test_brute_force_agrees_antiquant_modes(seed):
    """Per-channel / per-token scales with and without offsets, against the scalar twin."""
    rng = np.random.default_rng([314, 91, seed])
    kmode, vmode = [(0, 0), (1, 1), (0, 1)][seed % 3]
    mask = [MASK_NONE, MASK_CAUSAL, MASK_ALIBI][(seed // 3) % 3]
    c = _antiquant_case(rng, kmode=kmode, vmode=vmode, offsets=seed % 2 == 0)
    out, lse = _oracle_aq(c, mask, 4, 2, 0.4)
    lst = lambda x: None if x is None else x.tolist()
    bo, bl = brute_attention(
        c["q"].tolist(), c["k"].tolist(), c["v"].tolist(), c["table"].tolist(),
        c["q_lens"], c["kv_lens"], mask, 4, 2, 0.4, slopes=c["slopes"].tolist(),
        key_scale=lst(c["ks"]), value_scale=lst(c["vs"]), key_offset=lst(c["ko"]),
        value_offset=lst(c["vo"]), key_per_token=kmode == 1, value_per_token=vmode == 1)
    _same(out, np.array(bo).reshape(out.shape))
    _same(lse, np.array(bl).reshape(lse.shape))


def test_per_channel_key_offset_moves_lse_only():
    """A per-channel key offset o adds qkScale * sum_d q_d s_d o_d to every score of a row:
    out is unchanged and lse moves by that constant (which fixes where the offset
    enters: inside the scale, added to the integer)."""
    rng = np.random.default_rng([314, 92])
    c = _antiquant_case(rng, kmode=0, vmode=0, offsets=True, max_kv=9)
    c0 = dict(c, ko=None, vo=c["vo"])
    a = _oracle_aq(c, MASK_CAUSAL, 4, 2, 0.7)
    b = _oracle_aq(c0, MASK_CAUSAL, 4, 2, 0.7)
    _same(a[0], b[0], 1e-10)
    shift = 0.7 * np.einsum("thd,hd->th", c["q"], np.repeat(c["ks"] * c["ko"], 2, axis=0))
    fin = np.isfinite(b[1])
    assert np.max(np.abs(a[1][fin] - (b[1][fin] + shift[fin]))) < 1e-10
    assert np.array_equal(np.isfinite(a[1]), fin)


def test_per_token_value_offset_closed_form():
    """Zero int8 values and zero queries: every visible key has weight 1/n, so each
    output element is the mean of s_t * o_t over the visible tokens t and lse = ln n."""
    rng = np.random.default_rng([314, 93])
    c = _antiquant_case(rng, kmode=1, vmode=1, offsets=True, max_kv=10)
    c["q"][:] = 0.0
    c["v"][:] = 0.0
    out, lse = _oracle_aq(c, MASK_CAUSAL, 4, 2, 0.5)
    row = 0
    for b, (ql, kl) in enumerate(zip(c["q_lens"], c["kv_lens"])):
        for i in range(ql):
            n = kl - ql + i + 1
            if n <= 0:
                assert np.all(out[row] == 0) and np.all(lse[row] == np.inf)
            else:
                want = float(np.mean(c["vs"][b, :n] * c["vo"][b, :n]))
                assert np.max(np.abs(out[row] - want)) < 1e-12
                assert np.max(np.abs(lse[row] - math.log(n))) < 1e-12
            row += 1


def test_per_token_key_scale_closed_form():
    """Constant int8 keys k0 and all-ones queries: the score of token t is
    qkScale * D * s_t * (k0 + o_t), so lse = log sum_t exp(score_t) over visible t."""
    rng = np.random.default_rng([314, 94])
    c = _antiquant_case(rng, kmode=1, vmode=1, offsets=True, D=3, max_kv=8)
    c["q"][:] = 1.0
    c["k"][:] = 7.0
    _, lse = _oracle_aq(c, MASK_NONE, 4, 2, 0.9)
    row = 0
    for b, (ql, kl) in enumerate(zip(c["q_lens"], c["kv_lens"])):
        for i in range(ql):
            if kl == 0:
                assert np.all(lse[row] == np.inf)
            else:
                sc = [0.9 * 3 * c["ks"][b, t] * (7.0 + c["ko"][b, t]) for t in range(kl)]
                m = max(sc)
                want = m + math.log(math.fsum(math.exp(x - m) for x in sc))
                assert np.max(np.abs(lse[row] - want)) < 1e-12
            row += 1


def test_uniform_per_token_equals_uniform_per_channel():
    """The same scale and offset everywhere gives the same result in either mode."""
    rng = np.random.default_rng([314, 95])
    c = _antiquant_case(rng, kmode=1, vmode=1, offsets=True)
    S = c["ks"].shape[1]
    tok = dict(c, ks=np.full((2, S), 0.013), vs=np.full((2, S), 0.007),
               ko=np.full((2, S), -3.0), vo=np.full((2, S), 5.5))
    chan = dict(c, ks=np.full((2, 5), 0.013), vs=np.full((2, 5), 0.007),
                ko=np.full((2, 5), -3.0), vo=np.full((2, 5), 5.5), kmode=0, vmode=0)
    a = _oracle_aq(tok, MASK_ALIBI, 4, 2, 0.8)
    b = _oracle_aq(chan, MASK_ALIBI, 4, 2, 0.8)
    _same(a[0], b[0])
    _same(a[1], b[1])


def test_e4m3fn_decode_matches_library_and_hand_values():
    """Every byte code against torch's float8_e4m3fn conversion (a library routine),
    and the format's landmark values worked by hand."""
    codes = np.arange(256)
    mine = oracle.decode_e4m3fn(codes)
    lib = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(lib))
    fin = ~np.isnan(lib)
    assert np.array_equal(mine[fin], lib[fin])
    hand = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
            0x39: 1.125, 0xB8: -1.0, 0x7E: 448.0, 0xFE: -448.0, 0x40: 2.0, 0x30: 0.5}
    for c, v in hand.items():
        assert oracle.decode_e4m3fn([c])[0] == v, hex(c)
    assert np.isnan(oracle.decode_e4m3fn([0x7F, 0xFF])).all()


def test_fp8_equals_float_on_decoded_pool():
    """FLOAT8_E4M3FN codes with per-channel scales equal the fp cache of the decoded,
    scaled values."""
    rng = np.random.default_rng([314, 96])
    c = _random_case(rng, B=2, H=4, Hkv=2, D=6, bs=4, mask=MASK_ALIBI)
    k = rng.integers(0, 256, size=c["k"].shape)
    v = rng.integers(0, 256, size=c["v"].shape)
    k[(k & 0x7F) == 0x7F] = 0x10                       # no NaN codes
    v[(v & 0x7F) == 0x7F] = 0x22
    ks = rng.uniform(0.005, 0.02, size=(2, 6))
    vs = rng.uniform(0.005, 0.02, size=(2, 6))
    a = oracle.paged_attention(c["q"], k, v, c["table"], c["q_lens"], c["kv_lens"], MASK_ALIBI,
                               4, 2, 0.3, slopes=c["slopes"], key_antiquant_scale=ks,
                               value_antiquant_scale=vs, kv_format="e4m3fn")
    kf = oracle.decode_e4m3fn(k) * ks[None, None]
    vf = oracle.decode_e4m3fn(v) * vs[None, None]
    b = oracle.paged_attention(c["q"], kf, vf, c["table"], c["q_lens"], c["kv_lens"],
                               MASK_ALIBI, 4, 2, 0.3, slopes=c["slopes"])
    _same(a[0], b[0])
    _same(a[1], b[1])


def test_append_worked_example():
    """Two sequences, blockSize 2: sequence 0 has 3 cached + 2 new tokens (positions 3
    and 4) in blocks [4, 1, 0], sequence 1 has 0 cached + 1 new token in block [2].
    Position 3 is block 1 slot 1, position 4 is block 0 slot 0, sequence 1's token is
    block 2 slot 0 (worked by hand); nothing else changes."""
    pool = np.arange(5 * 2 * 1 * 2, dtype=np.int64).reshape(5, 2, 1, 2) * 10
    new = np.array([[[-1, -2]], [[-3, -4]], [[-5, -6]]])
    out = oracle.append_kv_rows(pool, new, [[4, 1, 0], [2, -1, -1]], [2, 1], [5, 1])
    want = pool.copy()
    want[1, 1, 0] = [-1, -2]
    want[0, 0, 0] = [-3, -4]
    want[2, 0, 0] = [-5, -6]
    assert np.array_equal(out, want)
    assert np.array_equal(pool, np.arange(20).reshape(5, 2, 1, 2) * 10)   # input untouched


def test_append_then_gather_returns_new_rows_last():
    """After an append, gathering a sequence gives its old prefix followed by its new
    rows (gather_sequence is pinned separately), and no other slot changes."""
    rng = np.random.default_rng([314, 97])
    bs, Hkv, D = 4, 2, 3
    q_lens, kv_lens = [3, 0, 5, 1], [7, 4, 5, 9]
    need = [-(-k // bs) for k in kv_lens]
    nb = sum(need) + 3
    perm = rng.permutation(nb)
    table = np.full((4, max(need)), -1)
    pos = 0
    for b in range(4):
        table[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    pool = rng.standard_normal((nb, bs, Hkv, D))
    new = rng.standard_normal((sum(q_lens), Hkv, D))
    out = oracle.append_kv_rows(pool, new, table, q_lens, kv_lens)
    row = 0
    written = np.zeros((nb, bs), dtype=bool)
    for b in range(4):
        before = oracle.gather_sequence(pool, table[b], kv_lens[b], bs)
        after = oracle.gather_sequence(out, table[b], kv_lens[b], bs)
        keep = kv_lens[b] - q_lens[b]
        assert np.array_equal(after[:keep], before[:keep])
        assert np.array_equal(after[keep:], new[row:row + q_lens[b]])
        for t in range(keep, kv_lens[b]):
            written[table[b][t // bs], t % bs] = True
        row += q_lens[b]
    assert np.array_equal(out[~written], pool[~written])


def test_empty_tensor_rules():
    """aclnnFusedInferAttentionScoreV4, Constraints, empty input: empty
    query/out returns empty; empty key/value gives out 0 and lse inf."""
    q = np.zeros((0, 2, 4))
    k = np.ones((3, 2, 1, 4))
    out, lse = oracle.paged_attention(q, k, k, np.zeros((1, 2), int), [0], [3], 0, 2, 1, 1.0)
    assert out.shape == (0, 2, 4) and lse.shape == (0, 2)
    q = np.ones((2, 2, 4))
    ek = np.zeros((0, 2, 1, 4))
    out, lse = oracle.paged_attention(q, ek, ek, np.zeros((2, 1), int), [1, 1], [5, 5],
                                      0, 2, 1, 1.0)
    assert np.all(out == 0) and np.all(np.isinf(lse)) and np.all(lse > 0)
    out, lse = oracle.paged_attention(q, k, k, np.zeros((2, 1), int), [1, 1], [0, 0],
                                      0, 2, 1, 1.0)
    assert np.all(out == 0) and np.all(lse == np.inf)


def test_merge_partials_equals_unsplit():
    """The max/sum/log decomposition of the softmaxLse restriction merges
    results over disjoint key ranges into the full result."""
    rng = np.random.default_rng([314, 90])
    kv, nq, H, D = 29, 4, 2, 5
    q = rng.standard_normal((nq, H, D))
    k = rng.standard_normal((kv, H, D))
    v = rng.standard_normal((kv, H, D))
    pos = oracle.query_positions(nq, kv)
    full = oracle.attention_contiguous(q, k, v, pos, MASK_CAUSAL, 0.6, H, H)
    cuts = [0, 7, 8, 20, kv]
    outs, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        # the chunk's keys keep their absolute index: shift the positions
        o, l = oracle.attention_contiguous(q, k[a:b], v[a:b], pos - a, MASK_CAUSAL,
                                           0.6, H, H)
        outs.append(o)
        lses.append(l)
    out, lse = oracle.merge_partials(outs, lses)
    _same(out, full[0])
    _same(lse, full[1])


def test_merge_partials_skips_chunks_a_row_cannot_see():
    """Causal split where some chunks lie wholly past a row's position: those
    partials are empty (out 0, lse +inf, the empty-row convention) and must drop
    out of the merge; rows that see no key at all stay out 0 / lse +inf.  The
    merge must still reproduce the unsplit result (softmaxLse decomposition,
    aclnnFusedInferAttentionScoreV3, Constraints)."""
    rng = np.random.default_rng([314, 91])
    kv, nq, H, D = 29, 31, 2, 5          # positions -2 .. 28: rows 0 and 1 see no key
    q = rng.standard_normal((nq, H, D))
    k = rng.standard_normal((kv, H, D))
    v = rng.standard_normal((kv, H, D))
    pos = oracle.query_positions(nq, kv)
    full = oracle.attention_contiguous(q, k, v, pos, MASK_CAUSAL, 0.6, H, H)
    cuts = [0, 10, 26, 27, 29]
    outs, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = oracle.attention_contiguous(q, k[a:b], v[a:b], pos - a, MASK_CAUSAL, 0.6, H, H)
        outs.append(o)
        lses.append(l)
    # the chunks past a row's position really are empty partials for that row
    assert np.all(np.isinf(lses[3][: nq - 2]) & (lses[3][: nq - 2] > 0))   # p <= 26
    assert np.all(outs[3][: nq - 2] == 0.0)
    assert np.all(np.isinf(lses[2][: nq - 3]))                             # p <= 25
    assert np.all(np.isfinite(lses[2][nq - 3:]))
    out, lse = oracle.merge_partials(outs, lses)
    assert np.all(np.isfinite(out))
    assert np.all(out[:2] == 0.0) and np.all(lse[:2] == np.inf)
    _same(out, full[0])
    _same(lse, full[1])
    # a single live partial merged with empty ones is returned unchanged
    live = np.isfinite(lses[0])
    o1, l1 = oracle.merge_partials([outs[0], np.zeros_like(outs[0])],
                                   [lses[0], np.full_like(lses[0], np.inf)])
    assert np.array_equal(o1[live], outs[0][live]) and np.array_equal(l1[live], lses[0][live])
