// Kernel argument blocks and launchers (host side of the HIP kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <cstdint>

#include "pa_internal.h"

namespace pa {

// KV antiquant beyond symmetric per-channel scales (int8 K/V): K_hat = scale * (K + offset)
// with per-channel [kvHeadNum, headSize] or per-token [batch, S] scales / offsets.
struct AntiquantArgs {
    const void* koff;       // offsets, layout and dtype of their scale; NULL: symmetric
    const void* voff;
    int64_t ktok_stride;    // per-token mode: row stride (elements) of the [batch, S] tensors
    int64_t vtok_stride;
    int32_t kmode, vmode;   // 0 per-channel, 1 per-token
    int32_t vscale_is_f32;  // value scale dtype (the key scale's is scale_is_f32)
    int32_t extended;       // anything but per-channel symmetric scales on both
};

struct DecodeArgs {
    const DecodeItem* items;
    const void* q;
    const void* k;
    const void* v;
    const int32_t* table;
    void* out;
    float* lse;
    const float* slopes;
    const void* kscale;
    const void* vscale;
    float* part_o;          // [slots][min(group,16)][D] un-normalised partial outputs
    float* part_ml;         // [slots][min(group,16)][2] partial (max, sum), log2 units
    CombineItem* comb;      // the combine items, written by the first split of each group
    int64_t q_tok_stride, q_head_stride, out_tok_stride, out_head_stride, lse_tok_stride;
    int64_t k_blk_stride, k_slot_stride, k_head_stride;
    int64_t v_blk_stride, v_slot_stride, v_head_stride, table_stride;
    int32_t group;          // headNum / kvHeadNum
    int32_t block_size;
    int32_t mask_type;
    int32_t scale_is_f32;   // antiquant scales are f32 (else the query dtype)
    float scale_log2;       // qkScale * log2(e)
    int32_t wave_heads;     // items of 4 kv heads, one per wave (DecodeItem.heads == 4)
    AntiquantArgs aq;
};

struct CombineArgs {
    const CombineItem* items;
    const float* part_o;
    const float* part_ml;
    void* out;
    float* lse;
    int64_t out_tok_stride, out_head_stride, lse_tok_stride;
    int32_t group;
    int32_t blocks_per_item;   // workgroups per combine item (set at launch)
};

struct PrefillArgs {
    const PrefillItem* items;
    const void* q;
    const void* k;
    const void* v;
    const int32_t* table;
    void* out;
    float* lse;
    const float* slopes;
    const void* kscale;
    const void* vscale;
    int64_t q_tok_stride, q_head_stride, out_tok_stride, out_head_stride, lse_tok_stride;
    int64_t k_blk_stride, k_slot_stride, k_head_stride;
    int64_t v_blk_stride, v_slot_stride, v_head_stride, table_stride;
    int32_t group;
    int32_t block_size;
    int32_t block_shift;    // log2(block_size) when it is a power of two, else -1
    int32_t mask_type;
    int32_t scale_is_f32;
    float scale_log2;
    AntiquantArgs aq;
};

struct AppendArgs {
    const AppendItem* items;
    const void* knew;
    const void* vnew;
    void* kcache;
    void* vcache;
    const int32_t* table;
    int64_t knew_tok_stride, knew_head_stride, vnew_tok_stride, vnew_head_stride;
    int64_t k_blk_stride, k_slot_stride, k_head_stride;
    int64_t v_blk_stride, v_slot_stride, v_head_stride, table_stride;
    int32_t kv_heads;
    int32_t row_chunks;     // headSize * element bytes / 16
    int32_t block_size;
    int32_t elem_bytes;
};

struct FillArgs {
    void* out;
    float* lse;
    int64_t n_tokens, head_num, head_size;
    int64_t out_tok_stride, out_head_stride, lse_tok_stride;
};

// t0 / t1 (optional): events attached to the kernel's own dispatch, so that their
// timestamps bracket the kernel alone (hipExtLaunchKernelGGL)
// i8: one-byte K/V (int8, or FLOAT8_E4M3FN codes when f8)
hipError_t launch_decode(const DecodeArgs& a, int n_items, int head_size, bool bf16, bool i8,
                         bool f8, hipStream_t stream, hipEvent_t t0 = nullptr,
                         hipEvent_t t1 = nullptr);
hipError_t launch_combine(const CombineArgs& a, int n_items, int head_size, bool bf16,
                          hipStream_t stream, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
hipError_t launch_prefill(const PrefillArgs& a, int n_items, int head_size, bool bf16, bool i8,
                          bool f8, hipStream_t stream, hipEvent_t t0 = nullptr,
                          hipEvent_t t1 = nullptr);

hipError_t launch_append(const AppendArgs& a, int n_items, hipStream_t stream,
                         hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);

// 256-thread launch of `kernel` over n workgroups, with timing events if given
template <typename K, typename A>
inline void launch_256(K kernel, int n, hipStream_t s, hipEvent_t t0, hipEvent_t t1, const A& a) {
    if (t0 != nullptr || t1 != nullptr)
        hipExtLaunchKernelGGL(kernel, dim3(n), dim3(256), 0, s, t0, t1, 0, a);
    else
        hipLaunchKernelGGL(kernel, dim3(n), dim3(256), 0, s, a);
}
hipError_t launch_fill(const FillArgs& a, hipStream_t stream);

}  // namespace pa
