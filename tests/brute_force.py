"""Scalar pure-Python twin of the attention definition, for tiny inputs only.

Written independently of ``oracle/`` (no shared helpers): every score,
every exponential and every sum is an explicit Python loop, with math.fsum
for the sums.  It follows aclnnFusedInferAttentionScoreV4, Function (formula
Softmax(scale * QK^T + mask) V, softmax per row) with the PrefixEncoder
argument conventions (paged pool, host lengths, maskType 3 / 9, slopes,
qkScale) and the ring-attention lse definition of
aclnnFusedInferAttentionScoreV3, Constraints: softmaxLse.
"""

import math


def _deq(x, b, j, c, d, scale, offset, per_token):
    """One antiquantised element: (x + offset) * scale, the scale / offset picked by
    (kv head, channel) in per-channel mode or by (sequence, token) in per-token mode."""
    if scale is None:
        return x
    if per_token:
        o = offset[b][j] if offset is not None else 0.0
        return (x + o) * scale[b][j]
    o = offset[c][d] if offset is not None else 0.0
    return (x + o) * scale[c][d]


def brute_attention(query, key, value, tables, seq_len, kv_seq_len, mask_type,
                    head_num, kv_head_num, qk_scale, slopes=None,
                    key_scale=None, value_scale=None, key_offset=None, value_offset=None,
                    key_per_token=False, value_per_token=False):
    """query [T][H][D], key/value [NB][bs][Hkv][D] as nested lists; per-channel scales /
    offsets [Hkv][D], per-token ones [B][S]."""
    n_tokens = len(query)
    D = len(query[0][0]) if n_tokens else 0
    bs = len(key[0]) if len(key) else 1
    per_group = head_num // kv_head_num
    out = [[[0.0] * D for _ in range(head_num)] for _ in range(n_tokens)]
    lse = [[math.inf] * head_num for _ in range(n_tokens)]
    row = 0
    for b in range(len(seq_len)):
        for i in range(seq_len[b]):
            pos = kv_seq_len[b] - seq_len[b] + i
            for h in range(head_num):
                c = h // per_group
                visible = []
                for j in range(kv_seq_len[b]):
                    if mask_type in (3, 9) and j > pos:
                        continue
                    blk = tables[b][j // bs]
                    krow = key[blk][j % bs][c]
                    terms = []
                    for d in range(D):
                        kd = _deq(krow[d], b, j, c, d, key_scale, key_offset, key_per_token)
                        terms.append(query[row][h][d] * kd)
                    s = qk_scale * math.fsum(terms)
                    if mask_type == 3:
                        s += slopes[h] * (j - pos)
                    visible.append((j, s))
                if not visible:
                    continue
                m = max(s for _, s in visible)
                weights = [(j, math.exp(s - m)) for j, s in visible]
                total = math.fsum(w for _, w in weights)
                for d in range(D):
                    acc = []
                    for j, w in weights:
                        blk = tables[b][j // bs]
                        vd = _deq(value[blk][j % bs][c][d], b, j, c, d, value_scale,
                                  value_offset, value_per_token)
                        acc.append(w * vd)
                    out[row][h][d] = math.fsum(acc) / total
                lse[row][h] = m + math.log(total)
            row += 1
    return out, lse
