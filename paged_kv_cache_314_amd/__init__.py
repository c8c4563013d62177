"""Paged-KV fused inference attention for AMD MI355X (gfx950).

The compute lives in libpagedattn.so (HIP kernels behind the C ABI declared in
include/pagedattn.h).  This package is its thin Python binding plus the
seeded synthetic-input generators (``workloads``) used by tests and benchmarks.
"""

from ._lib import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    Op,
    PA_ANTIQUANT_PER_CHANNEL,
    PA_ANTIQUANT_PER_TOKEN,
    PA_BF16,
    PA_ERR_HIP,
    PA_ERR_HOST_ALLOC,
    PA_ERR_NULLPTR,
    PA_ERR_PARAM_INVALID,
    PA_ERR_UNSUPPORTED,
    PA_ERR_WORKSPACE_TOO_SMALL,
    PA_F16,
    PA_F32,
    PA_F8E4M3,
    PA_I8,
    PA_I32,
    PA_MASK_ALIBI,
    PA_MASK_CAUSAL,
    PA_MASK_NONE,
    PA_OK,
    PagedAttentionError,
    PaTensor,
    alloc_workspace,
    describe,
    kv_cache_append,
    load,
    pa_kv_cache_append,
    pa_kv_cache_append_plan,
    pa_last_error,
    pa_op_describe,
    pa_op_destroy,
    pa_op_set_timing_events,
    pa_paged_attention,
    pa_paged_attention_get_workspace_size,
    pa_paged_attention_get_workspace_size_ex,
    pa_status_string,
    pa_version,
    paged_attention,
)
