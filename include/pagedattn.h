/*
 * pagedattn.h -- paged-KV fused inference attention for AMD MI355X (gfx950).
 *
 * Computes, per query row i of sequence b and query head h,
 *
 *     out[i,h,:] = sum_j softmax_j( qkScale * <q[i,h,:], K[j,kvh,:]> + bias(i,j) ) * V[j,kvh,:]
 *     lse[i,h]   = log( sum_j exp( qkScale * <q, K_j> + bias(i,j) ) )        (natural log)
 *
 * with K/V read through a paged cache (blockTables), kvh = h / (headNum / kvHeadNum) (GQA),
 * and bias from maskType.  Formula: aclnnFusedInferAttentionScoreV4, "Function"
 * (Attention = Softmax(QK^T/sqrt(d) + mask) V, softmax per row); qkScale generalises
 * 1/sqrt(d) and the mask/bias is added after the scaling (PrefixEncoder, Members:
 * qkScale, maskType).  lse definition: aclnnFusedInferAttentionScoreV3, Constraints,
 * softmaxLse (max + log of the sum of exponentials, the ring-attention decomposition).
 *
 * Two-phase call, as the pages' operator APIs (PrefixEncoder, Definition; the
 * "GetWorkspaceSize then execute" pattern of aclnnFusedInferAttentionScoreV3/V4):
 *   1. pa_paged_attention_get_workspace_size(...) validates every argument, plans the
 *      work for the current device and returns the device workspace size plus an
 *      operator handle.  It touches no device memory; its HIP calls are device queries
 *      (the current device's compute-unit count) and, on a host with a device, a pinned
 *      host buffer for the op's work lists (taken from a pool that pa_op_destroy
 *      refills, so steady-state planning allocates nothing).
 *   2. pa_paged_attention(workspace, size, op, stream) enqueues the kernels on `stream`;
 *      it allocates nothing and never waits.
 *
 * Conventions shared by every entry point
 *   - Tensors are described by pa_tensor (data pointer, dtype, shape, strides in
 *     elements).  The innermost dimension must be contiguous; see each argument.
 *   - "device" = HIP device memory (e.g. a torch CUDA tensor on ROCm);
 *     "host" = ordinary CPU memory.
 *   - The caller owns every tensor and the workspace; the library never allocates device
 *     memory.  The library owns the pa_op: its plan and its work lists (32 or 48 bytes
 *     per workgroup) in pinned, device-mapped host memory, which the kernels read in
 *     place (each workgroup loads its own item once).
 *   - Tensors and the workspace must stay alive, and must not be written by others,
 *     until the work enqueued by pa_paged_attention has completed on the stream.
 *   - Block ids in blockTables are not validated (aclnnFusedInferAttentionScoreV3,
 *     Constraints, paged attention scenario: the validity of block ids is not
 *     verified).  An id outside [0, numBlocks) for a token t < kvSeqLen[b] is an
 *     out-of-bounds device read: the caller must not pass one.  Entries past
 *     ceil(kvSeqLen[b] / blockSize) are never read (they may hold -1).
 *   - Results are deterministic: the same call on the same inputs gives bitwise equal
 *     outputs (aclnnFusedInferAttentionScoreV3, Constraints: deterministic computation).
 *     No atomics; split-KV partials are merged in a fixed order.
 *   - Errors: every check happens in phase 1, which returns a pa_status and leaves
 *     *op = NULL on failure; pa_last_error() gives a message naming the failed check.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  The pages' own error-code table is not recoverable, so these are
 * this library's codes for the same classes of failure (null pointer, invalid
 * parameter, unsupported feature) plus the run-time ones. */
typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_NULLPTR = 1,              /* a required pointer argument is NULL */
    PA_ERR_PARAM_INVALID = 2,        /* shape / dtype / value check failed */
    PA_ERR_UNSUPPORTED = 3,          /* valid per the pages, not implemented here */
    PA_ERR_WORKSPACE_TOO_SMALL = 4,  /* phase 2 got less workspace than phase 1 asked */
    PA_ERR_HIP = 5,                  /* a HIP runtime call failed in phase 2 */
    PA_ERR_HOST_ALLOC = 6            /* host memory for the operator could not be had */
} pa_status;

typedef enum pa_dtype {
    PA_F16 = 1,
    PA_BF16 = 2,
    PA_I8 = 3,
    PA_F32 = 4,
    PA_I32 = 5,
    PA_F8E4M3 = 6   /* FLOAT8_E4M3FN byte codes (OCP E4M3: bias 7, no infinity) */
} pa_dtype;

/* Tensor descriptor.  shape[0..ndim-1] and stride[0..ndim-1] (in elements, not bytes)
 * are read; entries past ndim are ignored.  A NULL pa_tensor* means "not passed". */
typedef struct pa_tensor {
    void* data;
    int32_t dtype;        /* pa_dtype */
    int32_t ndim;         /* 1..4 */
    int64_t shape[4];
    int64_t stride[4];
} pa_tensor;

/* maskType values (PrefixEncoder, Members: maskType). */
enum {
    PA_MASK_NONE = 0,               /* every key j < kvSeqLen[b] visible */
    PA_MASK_ALIBI = 3,              /* MASK_TYPE_ALIBI_COMPRESS: bias slopes[h]*(j - p_i), causal */
    PA_MASK_ALIBI_SQRT = 4,         /* MASK_TYPE_ALIBI_COMPRESS_SQRT: PA_ERR_UNSUPPORTED */
    PA_MASK_ALIBI_LEFT_ALIGN = 5,   /* MASK_TYPE_ALIBI_COMPRESS_LEFT_ALIGN: PA_ERR_UNSUPPORTED */
    PA_MASK_CAUSAL = 9              /* MASK_TYPE_CAUSAL_MASK: keys j > p_i hidden */
};

typedef struct pa_op pa_op;

/*
 * Phase 1: validate, plan, size the workspace.  (PrefixEncoder, Definition:
 * AtbSelfAttentionPrefixEncoderGetWorkspaceSize and its Members table; lse and the
 * antiquant scales are added from aclnnFusedInferAttentionScoreV3.)
 *
 * query        device, [nTokens, headNum, headSize] or [nTokens, headNum*headSize],
 *              f16 or bf16.  Rows of all sequences packed back to back: sequence b owns
 *              rows q0[b] .. q0[b]+seqLen[b]-1, q0[b] = seqLen[0] + ... + seqLen[b-1].
 *              The d stride must be 1; token and head strides are free (multiples of
 *              16 bytes; attnOut rows and heads must not overlap).  Data 16-byte aligned.
 * key, value   device, [numBlocks, blockSize, kvHeadNum, headSize] or
 *              [numBlocks, blockSize, kvHeadNum*headSize] (layout BnBsH), dtype = query
 *              dtype, or int8 / FLOAT8_E4M3FN (PA_F8E4M3) with both antiquant scales
 *              given (aclnnFusedInferAttentionScoreV3, Constraints, fake-quantization
 *              scenario; fp8 takes per-channel scales without offsets, and its NaN codes
 *              must not occur in a valid token).  Same shape and dtype.
 *              d stride 1; block, slot and head strides are free (multiples of 16
 *              bytes), so a (numBlocks, kvHeadNum, blockSize, headSize) cache can be
 *              passed as its permuted view.  Data 16-byte aligned.
 *              Token t of sequence b is at block blockTables[b][t / blockSize],
 *              slot t % blockSize.
 * blockTables  device, [batch, maxBlockNum] int32, row stride free, column stride 1.
 *              maxBlockNum >= ceil(max_b kvSeqLen[b] / blockSize).
 * mask         must be NULL (compressed mask tensors are not supported; maskType 3
 *              generates the ALiBi bias from slopes).
 * seqLen       HOST, [batch] int32: new query tokens per sequence, >= 0, summing to
 *              nTokens.  If every seqLen is <= 1 the decode kernels run (one query per
 *              sequence), otherwise the prefill kernels.
 * kvSeqLen     HOST, [batch] int32: tokens in the cache per sequence (cached prefix plus
 *              the new tokens), >= 0.  Query i of sequence b sits at absolute position
 *              p_i = kvSeqLen[b] - seqLen[b] + i (the new tokens are the last ones).
 * slopes       device, [headNum] f32; required iff maskType == PA_MASK_ALIBI, else NULL.
 * maskType     PA_MASK_NONE, PA_MASK_CAUSAL (key j visible iff j <= p_i) or
 *              PA_MASK_ALIBI (causal plus bias slopes[h] * (j - p_i), added after the
 *              qkScale product).  4 and 5 return PA_ERR_UNSUPPORTED.
 * headNum      > 0.   kvHeadNum: 0 means headNum; headNum % kvHeadNum == 0
 *              (aclnnFusedInferAttentionScoreV3, Constraints: numHeads divisible by
 *              numKeyValueHeads).  Query head h reads kv head h / (headNum/kvHeadNum).
 * qkScale      finite float multiplying Q*K^T (default on the pages: 1).
 * keyAntiquantScale, valueAntiquantScale
 *              device, kvHeadNum*headSize elements (shapes [kvHeadNum, headSize],
 *              [1, kvHeadNum, headSize], [kvHeadNum*headSize] ... all accepted),
 *              contiguous, f32 or the query dtype.  Required iff key/value are int8 or
 *              fp8: per-channel symmetric dequant K_hat[t,c,d] = scale[c,d] * K[t,c,d]
 *              (aclnnFusedInferAttentionScoreV3, Constraints on antiquantScale,
 *              per-channel mode; no offset).
 * attnOut      device, same shape form and dtype as query; written in full.
 * lse          device, [nTokens, headNum] f32, or NULL when not wanted.
 * workspaceSize  out: bytes of device workspace phase 2 needs (may be 0).
 * op           out: operator handle; NULL on failure.
 *
 * Empty tensors (aclnnFusedInferAttentionScoreV4, Constraints, processing when the
 * input parameter is empty): nTokens*headNum*headSize == 0 -> nothing is computed and
 * the remaining checks are skipped; key or value with 0 elements -> out is all 0 and
 * lse all +inf.  A query row that sees no key (kvSeqLen[b] == 0, or causal rows with
 * p_i < 0) also gets out 0 and lse +inf.
 */
pa_status pa_paged_attention_get_workspace_size(
    const pa_tensor* query, const pa_tensor* key, const pa_tensor* value,
    const pa_tensor* blockTables, const pa_tensor* mask,
    const pa_tensor* seqLen, const pa_tensor* kvSeqLen, const pa_tensor* slopes,
    int maskType, int32_t headNum, int32_t kvHeadNum, float qkScale,
    const pa_tensor* keyAntiquantScale, const pa_tensor* valueAntiquantScale,
    const pa_tensor* attnOut, const pa_tensor* lse,
    uint64_t* workspaceSize, pa_op** op);

/* Antiquant modes (aclnnFusedInferAttentionScoreV3, Constraints on the KV antiquant
 * parameters).  The pages number the modes without printing the table; they allow
 * key mode 0 with value mode 1 as the only pair of different modes, described as
 * per-channel keys with per-token values, which fixes the numbering. */
enum {
    PA_ANTIQUANT_PER_CHANNEL = 0,   /* scale[kvh, d]: kvHeadNum*headSize elements */
    PA_ANTIQUANT_PER_TOKEN = 1      /* scale[b, t]: shape (batch, S) or (1, batch, S), f32 */
};

/*
 * Phase 1 with the full set of KV antiquant parameters (aclnnFusedInferAttentionScoreV3,
 * Constraints on the KV antiquant parameters: per-channel and per-token modes, optional
 * offsets).  Every argument not listed here means exactly what it means for
 * pa_paged_attention_get_workspace_size, which is this call with NULL offsets and both
 * modes PA_ANTIQUANT_PER_CHANNEL.
 *
 * Dequantisation of int8 K (V likewise): K_hat = scale * (K + offset).  The pages give
 * no formula for the offset; it is taken as added to the stored integer before scaling
 * (pass offset = -z for a zero point z).  Without offsets the dequant is symmetric.
 *
 * keyAntiquantMode, valueAntiquantMode
 *              PA_ANTIQUANT_PER_CHANNEL or PA_ANTIQUANT_PER_TOKEN.  The two must be
 *              equal, except key per-channel with value per-token; other values or pairs
 *              give PA_ERR_PARAM_INVALID.  Modes other than per-channel need int8 K/V.
 * keyAntiquantScale, valueAntiquantScale
 *              per-channel: as for pa_paged_attention_get_workspace_size (f32 or the
 *              query dtype, kvHeadNum*headSize contiguous elements; the two scales of a
 *              per-channel pair share one dtype).  per-token: device f32, shape
 *              (batch, S) or (1, batch, S) with S >= max_b kvSeqLen[b], last stride 1,
 *              row stride free; token t of sequence b (its position in the sequence,
 *              not its cache slot) uses element [b, t] for every kv head and channel.
 * keyAntiquantOffset, valueAntiquantOffset
 *              device, NULL for symmetric dequant.  Both NULL or both given.  Each has
 *              the shape, strides and dtype of its scale.
 */
pa_status pa_paged_attention_get_workspace_size_ex(
    const pa_tensor* query, const pa_tensor* key, const pa_tensor* value,
    const pa_tensor* blockTables, const pa_tensor* mask,
    const pa_tensor* seqLen, const pa_tensor* kvSeqLen, const pa_tensor* slopes,
    int maskType, int32_t headNum, int32_t kvHeadNum, float qkScale,
    const pa_tensor* keyAntiquantScale, const pa_tensor* valueAntiquantScale,
    const pa_tensor* keyAntiquantOffset, const pa_tensor* valueAntiquantOffset,
    int keyAntiquantMode, int valueAntiquantMode,
    const pa_tensor* attnOut, const pa_tensor* lse,
    uint64_t* workspaceSize, pa_op** op);

/*
 * Phase 2: enqueue the computation on `stream` (a hipStream_t; NULL = the null
 * stream).  (PrefixEncoder, Definition: AtbSelfAttentionPrefixEncoder; the pages'
 * context argument becomes a HIP stream.)  workspace: device memory of at least the
 * phase-1 size, 256-byte aligned, or NULL if that size is 0; its contents on entry do
 * not matter and are scratch afterwards.  It holds the split-KV partial results; the
 * size is 0 when no sequence is split.  The call only enqueues kernels: no allocation,
 * no copy, no wait, so it may be captured into a graph (whose kernels read the op's
 * pinned work lists on every replay: such a graph must not be replayed after
 * pa_op_destroy).
 * An op may be executed any number of times, on any stream of any device; two
 * executions must not share a workspace while both are in flight.
 * Returns PA_ERR_NULLPTR (op, or a needed workspace, is NULL), PA_ERR_WORKSPACE_TOO_SMALL,
 * PA_ERR_PARAM_INVALID (workspace not 256-byte aligned) or PA_ERR_HIP on failure (also
 * for an op planned on a host without a HIP device, which holds no pinned lists).
 */
pa_status pa_paged_attention(void* workspace, uint64_t workspaceSize, pa_op* op,
                             void* stream);

/*
 * Phase 2 without a caller workspace, for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels as pa_paged_attention, with the workspace taken from a static scratch
 * array of the library (64 MiB, one per device, held until the process ends).  Allocates
 * nothing; enqueues the kernels on `stream` and never waits.  Every call on one device uses that device's one scratch array: calls whose
 * work overlaps on a device (other streams, or other threads) race and must be ordered
 * by the caller.  An op whose phase-1 workspaceSize exceeds 64 MiB is refused with
 * PA_ERR_WORKSPACE_TOO_SMALL (run it with pa_paged_attention).  Other errors as for
 * pa_paged_attention.
 */
pa_status pa_paged_attention_static(pa_op* op, void* stream);

/*
 * KV-cache append: write the new tokens' key/value rows into their cache blocks, the
 * step before a prefill / prefix-encoder call.  The pages print no API for it; this one
 * follows their cache layout and length conventions (aclnnFusedInferAttentionScoreV3,
 * Constraints, paged attention scenario: token t of sequence b is in block
 * blockTables[b][t / blockSize], slot t % blockSize; PrefixEncoder, Members: kvSeqLen
 * counts the cached prefix plus the seqLen new tokens, which are the last positions).
 * Reading: new token i of sequence b (row q0[b] + i of keyNew/valueNew, packed like the
 * query) is written at position p = kvSeqLen[b] - seqLen[b] + i, so that an append
 * followed by pa_paged_attention_get_workspace_size/pa_paged_attention with the same
 * seqLen / kvSeqLen attends over the updated cache.  A byte copy: a one-byte cache
 * receives the new tokens' codes as given (quantising them is the caller's step).
 *
 * keyNew, valueNew   device, [nTokens, kvHeadNum, headSize], the caches' dtype (f16,
 *                    bf16, i8 or f8e4m3); last stride 1, other strides free (multiples
 *                    of 16 bytes); headSize * element size a multiple of 16 bytes.
 * keyCache, valueCache  device, [numBlocks, blockSize, kvHeadNum, headSize] (or its
 *                    permuted BnNBsD view, or [numBlocks, blockSize, kvHeadNum*headSize]);
 *                    written at the new tokens' slots only.
 * blockTables        device, [batch, maxBlockNum] int32, maxBlockNum * blockSize >=
 *                    max kvSeqLen.  Block ids are not validated (as for the attention
 *                    call); the slots written must not be shared by two sequences.
 * seqLen, kvSeqLen   HOST, [batch] int32, 0 <= seqLen[b] <= kvSeqLen[b],
 *                    sum(seqLen) = nTokens.
 * op                 out: handle (pa_op_destroy releases it); nTokens == 0 gives a no-op.
 * Planning is done as for pa_paged_attention_get_workspace_size (same HIP calls; the
 * work list, 16 new tokens per 32-byte item, is pinned host memory the kernel reads).
 * pa_kv_cache_append enqueues the copy kernel on `stream` (NULL = the null stream); it
 * allocates nothing and never waits, and may be run again, e.g. after the new rows were
 * refilled in place.
 * pa_paged_attention rejects an append op and pa_kv_cache_append an attention op
 * (PA_ERR_PARAM_INVALID).  pa_op_set_timing_events applies to the copy kernel.
 */
pa_status pa_kv_cache_append_plan(const pa_tensor* keyNew, const pa_tensor* valueNew,
                                  const pa_tensor* keyCache, const pa_tensor* valueCache,
                                  const pa_tensor* blockTables, const pa_tensor* seqLen,
                                  const pa_tensor* kvSeqLen, pa_op** op);
pa_status pa_kv_cache_append(pa_op* op, void* stream);

/* Release an operator handle (NULL is ignored).  Work already enqueued is unaffected and
 * the call does not wait for it: the op's pinned work-list buffer goes back to the
 * library's pool and is handed to a new op only after the kernels that read it have
 * run. */
void pa_op_destroy(pa_op* op);

/* Plan options: overrides of the planner's automatic choices, for tuning and tests.
 * Process-wide; they apply to ops planned after the call.  value -1 restores the
 * automatic choice (the default for every option).
 *   PA_OPT_DECODE_CHUNK_TILES   32-token tiles per decode work item (1 .. 2^20)
 *   PA_OPT_DECODE_TARGET_ITEMS  decode workgroups the split aims for (1 .. 2^20)
 *   PA_OPT_DECODE_WAVE_HEADS    0 / 1: decode items of four kv heads, one per wave
 *   PA_OPT_PREFILL_PAIR         0 / 1: heavy + light prefill items sharing a CU
 *   PA_OPT_PREFILL_XCD_ORDER    0 / 1: prefill items grouped per XCD
 *   PA_OPT_COMPUTE_UNITS        compute units to plan for (1 .. 2^20; default: the
 *                               current device's, 256 when no device can be queried)
 * The decode options change how sequences are split, and with it the order of the
 * floating-point sums: results stay within the stated tolerances but their bits
 * change.  The determinism promise (same call, same inputs -> same bits) holds for
 * ops planned with the same options on the same device.  Returns PA_ERR_PARAM_INVALID
 * for an unknown option or a value out of range. */
enum {
    PA_OPT_DECODE_CHUNK_TILES = 1,
    PA_OPT_DECODE_TARGET_ITEMS = 2,
    PA_OPT_DECODE_WAVE_HEADS = 3,
    PA_OPT_PREFILL_PAIR = 4,
    PA_OPT_PREFILL_XCD_ORDER = 5,
    PA_OPT_COMPUTE_UNITS = 6
};
pa_status pa_set_plan_option(int option, int32_t value);
/* The option's current value (-1: automatic, or an unknown option). */
int32_t pa_get_plan_option(int option);

/* Instrumentation: start and stop are hipEvent_t handles (or NULL to clear), created with
 * timing enabled.  While set, each execute of this op attaches them to the dispatch of
 * one of its kernels -- kernel PA_TIMED_MAIN: the decode, prefill or append kernel;
 * PA_TIMED_COMBINE: the split-KV combine, run by decode ops that split a sequence -- so
 * that hipEventElapsedTime(start, stop) is that kernel's own duration.  The events stay
 * owned by the caller.  Host only; returns PA_ERR_NULLPTR if op is NULL and
 * PA_ERR_PARAM_INVALID for another kernel index. */
enum { PA_TIMED_MAIN = 0, PA_TIMED_COMBINE = 1 };
pa_status pa_op_set_timing_events(pa_op* op, int kernel, void* start, void* stop);

/* Write a JSON description of the operator's plan into buf (NUL-terminated, cut at
 * cap - 1 bytes; buf may be NULL when cap is 0) and return the full length without the
 * NUL.  Keys: "mode" ("noop", "fill", "decode", "prefill", "append"), "workspace_bytes",
 * "items_bytes" (the pinned work lists), "compute_units" (planned for), "chunk_tiles",
 * "partial_slots", and the work lists "decode_items" [b, kvh, hg, t0, t1, slot, qrow,
 * kvlen, heads, slot_stride, comb, nsplit], "combine_items" [kvh, hg, slot0, nsplit, qrow],
 * "prefill_items" [b, h, qbeg, qlen, kvlen, qrow0, ktiles, heads] (heads query heads from
 * h, 128/heads query rows from qbeg), "append_items" [b, row0, pos0, count], "antiquant"
 * [key mode, value mode, offsets given].  Host only, no HIP call.
 * For inspection and tests: not a stable interface.  op == NULL returns 0. */
uint64_t pa_op_describe(const pa_op* op, char* buf, uint64_t cap);

/* Static text for a status code. */
const char* pa_status_string(int status);

/* Message describing the last failure on the calling thread ("" if none). */
const char* pa_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
