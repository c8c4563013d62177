"""fp64 NumPy oracle for paged-KV fused attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this module.  It shares no code with the HIP library.

Notation follows the pages:
  query  [nTokens, headNum, headSize]       (PrefixEncoder, Members: query)
  key / value  [numBlocks, blockSize, kvHeadNum, headSize]
                                            (PrefixEncoder, Members: key, value)
  blockTables  [batch, maxBlockNum]         (PrefixEncoder, Members: blockTables)
  seqLen / kvSeqLen  [batch], host side     (PrefixEncoder, Members: seqLen, kvSeqLen)
  slopes [headNum]                          (PrefixEncoder, Members: slopes)
  lse    [nTokens, headNum], natural log    (aclnnFusedInferAttentionScoreV3,
                                             Constraints: softmaxLse)

Readings where the pages are silent:
  * query head h uses kv head h // (headNum / kvHeadNum);
  * the seqLen new queries of a sequence are its LAST seqLen positions, so
    query i sits at absolute position p_i = kvSeqLen - seqLen + i
    (bottom-right alignment of the causal mask);
  * the ALiBi bias of maskType 3 is slope_h * (j - p_i), added after the
    qkScale multiplication, and keys j > p_i are masked (causal);
  * a row that sees no key gives out = 0 and lse = +inf;
  * antiquant K_hat = scale * (K + offset): the pages name a scale and an
    optional offset (absent = symmetric) but print no formula; the offset is
    taken as added to the stored integer before scaling (a zero point z is
    passed as offset = -z);
  * antiquant modes 0 = per-channel (scale[kvh, d]) and 1 = per-token
    (scale[b, t], t the token's position in its sequence, shared by every kv
    head and channel): the pages allow key mode 0 with value mode 1 as the one
    pair of different modes, which fixes 0 as per-channel and 1 as per-token.
"""

import numpy as np

MASK_NONE = 0     # no mask: every key 0 <= j < kvSeqLen is visible
MASK_ALIBI = 3    # PrefixEncoder maskType 3, MASK_TYPE_ALIBI_COMPRESS
MASK_CAUSAL = 9   # PrefixEncoder maskType 9, MASK_TYPE_CAUSAL_MASK

ANTIQUANT_PER_CHANNEL = 0
ANTIQUANT_PER_TOKEN = 1


def decode_e4m3fn(codes):
    """Real values of FLOAT8_E4M3FN codes (aclnnFusedInferAttentionScoreV3, Constraints:
    key/value may be FLOAT8_E4M3FN in the fake-quantization scenario).

    The format (OCP 8-bit floating point, E4M3 "FN"): bit 7 sign, bits 6..3 a biased
    exponent e (bias 7), bits 2..0 a mantissa m.  e > 0 gives (1 + m/8) * 2^(e-7);
    e == 0 gives the subnormal (m/8) * 2^-6; e == 15 with m == 7 is NaN; there is no
    infinity (e == 15, m < 7 are ordinary values up to 448).
    codes: integer array of byte values 0..255.  Returns float64.
    """
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def gather_sequence(pool, table_row, kv_len, block_size):
    """Contiguous rows [kv_len, kvHeadNum, headSize] of one sequence.

    aclnnFusedInferAttentionScoreV3, Constraints, paged attention scenario:
    the cache is stored block by block, and the sequence is the blocks named
    by its row of blockTables laid end to end.  Token t therefore lives in
    physical block table_row[t // blockSize] at slot t % blockSize.  Only the
    first ceil(kv_len / blockSize) entries of the row are read; the slots of
    the last block beyond kv_len are dropped.
    """
    kv_len = int(kv_len)
    n_blocks = -(-kv_len // block_size)
    ids = np.asarray(table_row[:n_blocks], dtype=np.int64)
    blocks = np.asarray(pool)[ids]                      # [n_blocks, bs, Hkv, D]
    rows = blocks.reshape((n_blocks * block_size,) + blocks.shape[2:])
    return rows[:kv_len].astype(np.float64)


def dequantize_per_channel(x, scale, offset=None):
    """Per-channel antiquant of int8 K or V rows.

    aclnnFusedInferAttentionScoreV3, Constraints on antiquantScale /
    antiquantOffset (per-channel mode; symmetric when the offset is null,
    asymmetric otherwise): the real value is (stored integer + offset) times
    the scale of its (kv head, channel).  x: [..., kvHeadNum, headSize]
    integers; scale, offset: [kvHeadNum, headSize].
    """
    x = np.asarray(x, dtype=np.float64)
    if offset is not None:
        x = x + np.asarray(offset, dtype=np.float64)
    return x * np.asarray(scale, dtype=np.float64)


def dequantize_per_token(x, scale_row, offset_row=None):
    """Per-token antiquant of one sequence's int8 K or V rows.

    aclnnFusedInferAttentionScoreV3, Constraints on the KV antiquant
    parameters, per-token mode (scale shape (B, S), float32): token t of the
    sequence has one scale (and offset) for all its kv heads and channels.
    x: [kv_len, kvHeadNum, headSize] integers; scale_row, offset_row: the
    sequence's row of the (B, S) tensors, S >= kv_len.
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    if offset_row is not None:
        x = x + np.asarray(offset_row, dtype=np.float64)[:n, None, None]
    return x * np.asarray(scale_row, dtype=np.float64)[:n, None, None]


def query_positions(q_len, kv_len):
    """Absolute positions p_i = kv_len - q_len + i of a sequence's queries.

    PrefixEncoder, Members: query holds only the new tokens (nTokens rows),
    while kvSeqLen counts the cached prefix plus the new tokens, so the new
    queries are the last q_len positions of the kv sequence.  For decode
    (q_len = 1) this is p_0 = kv_len - 1.
    """
    return np.arange(q_len, dtype=np.int64) + (int(kv_len) - int(q_len))


def attention_contiguous(q, k, v, positions, mask_type, qk_scale,
                         head_num, kv_head_num, slopes=None):
    """Attention of one sequence's queries over its contiguous K/V.

    aclnnFusedInferAttentionScoreV4, Function, formula
    Attention = Softmax(QK^T / sqrt(d) + mask) V, softmax per row; the
    PrefixEncoder generalises 1/sqrt(d) to qkScale ("post-multiplied by
    Q*K^T") and adds the mask / ALiBi term after that scaling.
    The lse is max + log(sum(exp(s - max))) (aclnnFusedInferAttentionScoreV3,
    Constraints: softmaxLse, ring-attention decomposition).

    q: [nq, headNum, D]; k, v: [kv, kvHeadNum, D]; positions: [nq].
    Returns out [nq, headNum, D] and lse [nq, headNum], both float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, H, D = q.shape
    kv = k.shape[0]
    group = head_num // kv_head_num
    positions = np.asarray(positions, dtype=np.int64)
    out = np.zeros((nq, H, D), dtype=np.float64)
    lse = np.full((nq, H), np.inf, dtype=np.float64)
    if nq == 0 or kv == 0:
        return out, lse
    j = np.arange(kv, dtype=np.int64)
    hidden = j[None, :] > positions[:, None]            # keys after the query
    for h in range(H):
        kvh = h // group
        s = qk_scale * (q[:, h, :] @ k[:, kvh, :].T)     # [nq, kv]
        if mask_type == MASK_ALIBI:
            s = s + float(slopes[h]) * (j[None, :] - positions[:, None])
        if mask_type in (MASK_ALIBI, MASK_CAUSAL):
            s = np.where(hidden, -np.inf, s)
        m = s.max(axis=1)
        for i in range(nq):
            if not np.isfinite(m[i]):
                continue                                  # no visible key
            e = np.exp(s[i] - m[i])                       # exp(-inf) = 0
            l = e.sum()
            out[i, h, :] = (e @ v[:, kvh, :]) / l
            lse[i, h] = m[i] + np.log(l)
    return out, lse


def paged_attention(query, key, value, block_tables, seq_len, kv_seq_len,
                    mask_type, head_num, kv_head_num, qk_scale, slopes=None,
                    key_antiquant_scale=None, value_antiquant_scale=None,
                    key_antiquant_offset=None, value_antiquant_offset=None,
                    key_antiquant_mode=ANTIQUANT_PER_CHANNEL,
                    value_antiquant_mode=ANTIQUANT_PER_CHANNEL, kv_format=None):
    """Reference result of the paged fused-attention call.

    PrefixEncoder, Definition and Members: query [nTokens, headNum, headSize]
    packs the new tokens of every sequence back to back (sequence b owns rows
    q0[b] .. q0[b] + seqLen[b] - 1 with q0[b] = sum of the earlier seqLen);
    key/value are the paged pool [numBlocks, blockSize, kvHeadNum, headSize]
    read through blockTables; kvHeadNum = 0 means kvHeadNum = headNum.

    Empty-tensor rules (aclnnFusedInferAttentionScoreV4, Constraints,
    processing when the input parameter is empty): an empty query/out returns
    empty tensors; an empty key/value returns out all 0 and lse all inf.

    int8 key/value are dequantised before anything else: per channel
    (mode 0) with scales / offsets [kvHeadNum, headSize], or per token
    (mode 1) with scales / offsets [batch, S] (a leading 1 is dropped).
    kv_format="e4m3fn": key/value hold FLOAT8_E4M3FN byte codes, decoded
    (decode_e4m3fn) before the per-channel scales are applied.
    Returns out [nTokens, headNum, headSize] and lse [nTokens, headNum].
    """
    if kv_head_num == 0:
        kv_head_num = head_num
    query = np.asarray(query)
    n_tokens = query.shape[0]
    D = query.shape[2]
    out = np.zeros((n_tokens, head_num, D), dtype=np.float64)
    lse = np.full((n_tokens, head_num), np.inf, dtype=np.float64)
    key = np.asarray(key)
    value = np.asarray(value)
    if query.size == 0 or key.size == 0 or value.size == 0:
        return out, lse
    block_size = key.shape[1]
    seq_len = np.asarray(seq_len, dtype=np.int64)
    kv_seq_len = np.asarray(kv_seq_len, dtype=np.int64)
    q0 = 0
    for b in range(seq_len.shape[0]):
        ql, kl = int(seq_len[b]), int(kv_seq_len[b])
        k_b = gather_sequence(key, block_tables[b], kl, block_size)
        v_b = gather_sequence(value, block_tables[b], kl, block_size)
        if kv_format == "e4m3fn":
            k_b = decode_e4m3fn(k_b)
            v_b = decode_e4m3fn(v_b)
        k_b = _dequantize(k_b, b, key_antiquant_scale, key_antiquant_offset,
                          key_antiquant_mode)
        v_b = _dequantize(v_b, b, value_antiquant_scale, value_antiquant_offset,
                          value_antiquant_mode)
        o_b, l_b = attention_contiguous(
            query[q0:q0 + ql], k_b, v_b, query_positions(ql, kl), mask_type,
            qk_scale, head_num, kv_head_num, slopes)
        out[q0:q0 + ql] = o_b
        lse[q0:q0 + ql] = l_b
        q0 += ql
    return out, lse


def _dequantize(x_b, b, scale, offset, mode):
    """Antiquant of sequence b's gathered rows in the given mode (no-op without a scale)."""
    if scale is None:
        return x_b
    if mode == ANTIQUANT_PER_CHANNEL:
        return dequantize_per_channel(x_b, scale, offset)
    scale = np.asarray(scale, dtype=np.float64)
    scale = scale.reshape(scale.shape[-2:])
    off_row = None
    if offset is not None:
        offset = np.asarray(offset, dtype=np.float64)
        off_row = offset.reshape(offset.shape[-2:])[b]
    return dequantize_per_token(x_b, scale[b], off_row)


def append_kv_rows(pool, new_rows, block_tables, seq_len, kv_seq_len):
    """The cache after writing the new tokens' rows (KV-cache append).

    aclnnFusedInferAttentionScoreV3, Constraints, paged attention scenario: token t
    of sequence b lives in block table_row[t // blockSize], slot t % blockSize.
    PrefixEncoder, Members: kvSeqLen counts the cached prefix plus the seqLen new
    tokens, which are the sequence's last positions; the new tokens' rows are packed
    sequence after sequence like the query.  Reading (no API on the pages): new token
    i of sequence b goes to position kvSeqLen[b] - seqLen[b] + i.
    pool: [numBlocks, blockSize, kvHeadNum, headSize]; new_rows: [nTokens, kvHeadNum,
    headSize], same dtype.  Returns a new array; the input pool is not modified.
    """
    out = np.array(pool, copy=True)
    new_rows = np.asarray(new_rows)
    block_size = out.shape[1]
    row = 0
    for b in range(len(seq_len)):
        ql, kl = int(seq_len[b]), int(kv_seq_len[b])
        for i in range(ql):
            t = kl - ql + i
            out[int(block_tables[b][t // block_size]), t % block_size] = new_rows[row]
            row += 1
    return out


def merge_partials(outs, lses):
    """Combine attention results computed over disjoint key ranges.

    aclnnFusedInferAttentionScoreV3, Constraints: softmaxLse.  The lse is
    softmax_max + log(softmax_sum); results over key subsets are merged by
    weighting each partial output with exp(lse_s - lse) where
    lse = log(sum_s exp(lse_s)).  A partial with lse = +inf (the empty-row
    convention) saw no key and is skipped.  outs: list of [..., D];
    lses: list of [...].  Returns (out, lse).
    """
    outs = [np.asarray(o, dtype=np.float64) for o in outs]
    lses = [np.asarray(x, dtype=np.float64) for x in lses]
    live = [np.where(np.isfinite(x), x, -np.inf) for x in lses]
    m = np.max(np.stack(live), axis=0)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    weights = [np.exp(x - safe_m) for x in live]
    total = np.sum(np.stack(weights), axis=0)
    out = np.zeros_like(outs[0])
    for o, w in zip(outs, weights):
        out += o * w[..., None]
    seen = total > 0
    out = np.where(seen[..., None], out / np.where(seen, total, 1.0)[..., None], 0.0)
    lse = np.where(seen, safe_m + np.log(np.where(seen, total, 1.0)), np.inf)
    return out, lse
