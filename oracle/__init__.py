"""Plain, slow, obviously correct CPU oracle for paged-KV fused attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this package; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it.  It shares no code with the HIP path
(``paged_kv_cache_314_amd``), and the HIP path never falls back to it.

Everything is computed in float64 with NumPy: the paged K/V cache is first
gathered into contiguous per-sequence arrays, then the attention of every
query row is written out as explicit scores, an explicit mask/bias, an
explicit softmax and a weighted sum of V rows.

Sources (the pages this follows):
  * aclnnFusedInferAttentionScoreV4 / V3, "Function" (formula
    Softmax(QK^T/sqrt(d) + mask) V), "Constraints" (empty-tensor rules,
    deterministic computation, paged-attention layout, GQA divisibility,
    per-channel and per-token KV antiquant with optional offsets, FLOAT8_E4M3FN
    key/value codes, and the
    softmax-LSE decomposition used by
    ring attention).
  * The same pages' cache layout and length conventions for the KV-cache
    append (append_kv_rows), whose API the pages do not print.
  * PrefixEncoder (Ascend Transformer Boost SelfAttention, calcType
    PREFIX_ENCODER), "Definition" and "Members" table (argument list,
    qkScale, maskType 3 = ALiBi compressed, 9 = causal, slopes per head,
    host-side seqLen / kvSeqLen).

Every function is pinned by ``tests/test_oracle_pins.py`` (closed forms,
brute force, a library special case and page invariants); none is
"parity unpinned".
"""

from .attention import (
    MASK_NONE,
    MASK_ALIBI,
    MASK_CAUSAL,
    ANTIQUANT_PER_CHANNEL,
    ANTIQUANT_PER_TOKEN,
    decode_e4m3fn,
    gather_sequence,
    dequantize_per_channel,
    dequantize_per_token,
    query_positions,
    attention_contiguous,
    paged_attention,
    merge_partials,
    append_kv_rows,
)

__all__ = [
    "MASK_NONE",
    "MASK_ALIBI",
    "MASK_CAUSAL",
    "gather_sequence",
    "dequantize_per_channel",
    "query_positions",
    "attention_contiguous",
    "paged_attention",
    "merge_partials",
]
