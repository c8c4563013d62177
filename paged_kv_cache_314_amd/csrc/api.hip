// C ABI of libpagedattn: two-phase get-workspace-size / execute (PrefixEncoder,
// Definition: GetWorkspaceSize then execute with workspace, size, op and context).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>

#include "pa_internal.h"
#include "pa_kernels.h"
#include "pagedattn.h"

struct pa_op {
    pa::Plan plan;
    void* staging = nullptr;        // pinned, device-mapped work lists (made on first run)
    unsigned char* staging_dev = nullptr;   // the same memory as seen by the GPU
    unsigned char* lists_dev = nullptr;     // device copy of the work lists (first run)
    int lists_device = -1;                  // the device holding lists_dev
    const unsigned char* lists = nullptr;   // what the kernels read: lists_dev or staging_dev
    hipEvent_t done = nullptr;      // recorded after the last kernel of each run
    hipEvent_t t_start = nullptr;   // caller's timing events around the main kernel
    hipEvent_t t_stop = nullptr;
};

namespace {

thread_local std::string g_last_error;

pa_status fail(pa_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

pa_status hip_fail(hipError_t e, const char* what) {
    std::string msg = std::string(what) + ": " + hipGetErrorString(e);
    return fail(PA_ERR_HIP, msg);
}

// The work lists: each workgroup reads its own 32-byte item at start-up, a dependent load
// ahead of everything else it does, so they are read from device memory: the first run
// copies them from a pinned host buffer into a small device buffer of the op, on the
// caller's stream, and waits for that stream once.  A first run made under stream
// capture cannot wait; that op then reads the pinned buffer in place over the bus
// (about 1 us more per launch).  Kernels of later runs on another device are refused.
pa_status make_host_lists(pa_op* op);

pa_status ensure_staging(pa_op* op, hipStream_t stream) {
    const pa::Plan& p = op->plan;
    if (p.items_bytes == 0) return PA_OK;
    if (op->lists != nullptr) {
        if (op->lists_dev == nullptr) return PA_OK;
        int dev = -1;
        hipError_t e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
        if (dev != op->lists_device)
            return fail(PA_ERR_PARAM_INVALID, "op was first run on device " +
                                                  std::to_string(op->lists_device) +
                                                  ", not on device " + std::to_string(dev));
        return PA_OK;
    }
    pa_status st = make_host_lists(op);
    if (st != PA_OK) return st;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cap != hipStreamCaptureStatusNone) {
        op->lists = op->staging_dev;
        return PA_OK;
    }
    int dev = -1;
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    void* d = nullptr;
    e = hipMalloc(&d, p.items_bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(work lists)");
    e = hipMemcpyAsync(d, op->staging, p.items_bytes, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
        (void)hipFree(d);
        return hip_fail(e, "copy of the work lists");
    }
    op->lists_dev = static_cast<unsigned char*>(d);
    op->lists_device = dev;
    op->lists = op->lists_dev;
    return PA_OK;
}

// Copy the host work lists into one pinned, device-mapped buffer.
pa_status make_host_lists(pa_op* op) {
    const pa::Plan& p = op->plan;
    if (op->staging != nullptr) return PA_OK;
    hipError_t e = hipHostMalloc(&op->staging, p.items_bytes, hipHostMallocMapped);
    if (e != hipSuccess) {
        op->staging = nullptr;
        return hip_fail(e, "hipHostMalloc(work lists)");
    }
    void* dev = nullptr;
    e = hipHostGetDevicePointer(&dev, op->staging, 0);
    if (e != hipSuccess) {
        (void)hipHostFree(op->staging);
        op->staging = nullptr;
        return hip_fail(e, "hipHostGetDevicePointer(work lists)");
    }
    op->staging_dev = static_cast<unsigned char*>(dev);
    auto* base = static_cast<unsigned char*>(op->staging);
    std::memset(base, 0, p.items_bytes);
    if (p.mode == pa::Mode::kDecode) {
        std::memcpy(base + p.off_items, p.decode_items.data(),
                    p.decode_items.size() * sizeof(pa::DecodeItem));
        std::memcpy(base + p.off_combine, p.combine_items.data(),
                    p.combine_items.size() * sizeof(pa::CombineItem));
    } else if (p.mode == pa::Mode::kPrefill) {
        std::memcpy(base + p.off_items, p.prefill_items.data(),
                    p.prefill_items.size() * sizeof(pa::PrefillItem));
    } else if (p.mode == pa::Mode::kAppend) {
        std::memcpy(base + p.off_items, p.append_items.data(),
                    p.append_items.size() * sizeof(pa::AppendItem));
    }
    return PA_OK;
}

pa::AntiquantArgs antiquant_args(const pa::Plan& p) {
    pa::AntiquantArgs q{};
    q.koff = p.koff;
    q.voff = p.voff;
    q.ktok_stride = p.ktok_stride;
    q.vtok_stride = p.vtok_stride;
    q.kmode = p.kmode;
    q.vmode = p.vmode;
    q.vscale_is_f32 = p.vscale_type == PA_F32;
    q.extended = (p.kmode != PA_ANTIQUANT_PER_CHANNEL || p.vmode != PA_ANTIQUANT_PER_CHANNEL ||
                  p.koff != nullptr) ? 1 : 0;
    return q;
}

}  // namespace

extern "C" {

pa_status pa_paged_attention_get_workspace_size(
    const pa_tensor* query, const pa_tensor* key, const pa_tensor* value,
    const pa_tensor* blockTables, const pa_tensor* mask, const pa_tensor* seqLen,
    const pa_tensor* kvSeqLen, const pa_tensor* slopes, int maskType, int32_t headNum,
    int32_t kvHeadNum, float qkScale, const pa_tensor* keyAntiquantScale,
    const pa_tensor* valueAntiquantScale, const pa_tensor* attnOut, const pa_tensor* lse,
    uint64_t* workspaceSize, pa_op** op) {
    return pa_paged_attention_get_workspace_size_ex(
        query, key, value, blockTables, mask, seqLen, kvSeqLen, slopes, maskType, headNum,
        kvHeadNum, qkScale, keyAntiquantScale, valueAntiquantScale, nullptr, nullptr,
        PA_ANTIQUANT_PER_CHANNEL, PA_ANTIQUANT_PER_CHANNEL, attnOut, lse, workspaceSize, op);
}

pa_status pa_paged_attention_get_workspace_size_ex(
    const pa_tensor* query, const pa_tensor* key, const pa_tensor* value,
    const pa_tensor* blockTables, const pa_tensor* mask, const pa_tensor* seqLen,
    const pa_tensor* kvSeqLen, const pa_tensor* slopes, int maskType, int32_t headNum,
    int32_t kvHeadNum, float qkScale, const pa_tensor* keyAntiquantScale,
    const pa_tensor* valueAntiquantScale, const pa_tensor* keyAntiquantOffset,
    const pa_tensor* valueAntiquantOffset, int keyAntiquantMode, int valueAntiquantMode,
    const pa_tensor* attnOut, const pa_tensor* lse, uint64_t* workspaceSize, pa_op** op) {
    if (op != nullptr) *op = nullptr;
    if (workspaceSize == nullptr || op == nullptr)
        return fail(PA_ERR_NULLPTR, "workspaceSize and op must not be NULL");
    *workspaceSize = 0;
    pa_op* h = new (std::nothrow) pa_op();
    if (h == nullptr) return fail(PA_ERR_HOST_ALLOC, "cannot allocate the operator");
    std::string err;
    const pa_status st = pa::plan(query, key, value, blockTables, mask, seqLen, kvSeqLen, slopes,
                                  maskType, headNum, kvHeadNum, qkScale, keyAntiquantScale,
                                  valueAntiquantScale, keyAntiquantOffset, valueAntiquantOffset,
                                  keyAntiquantMode, valueAntiquantMode, attnOut, lse, h->plan, err);
    if (st != PA_OK) {
        delete h;
        return fail(st, err);
    }
    *workspaceSize = h->plan.workspace_bytes;
    *op = h;
    g_last_error.clear();
    return PA_OK;
}

pa_status pa_paged_attention(void* workspace, uint64_t workspaceSize, pa_op* op, void* stream) {
    if (op == nullptr) return fail(PA_ERR_NULLPTR, "op is NULL");
    const pa::Plan& p = op->plan;
    if (p.mode == pa::Mode::kAppend)
        return fail(PA_ERR_PARAM_INVALID, "op is a KV-cache append plan: run it with pa_kv_cache_append");
    if (p.mode == pa::Mode::kNoop) return PA_OK;
    if (workspaceSize < p.workspace_bytes)
        return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                    "workspace of " + std::to_string(workspaceSize) + " bytes, need " +
                        std::to_string(p.workspace_bytes));
    if (p.workspace_bytes > 0 && workspace == nullptr)
        return fail(PA_ERR_NULLPTR, "workspace is NULL");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(PA_ERR_PARAM_INVALID, "workspace must be 256-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf16 = p.qtype == PA_BF16;
    const bool f8 = p.kvtype == PA_F8E4M3;
    const bool i8 = p.kvtype == PA_I8 || f8;      // one-byte K/V
    hipError_t e;

    if (p.mode == pa::Mode::kFill) {
        pa::FillArgs f{};
        f.out = p.out;
        f.lse = p.lse;
        f.n_tokens = p.n_tokens;
        f.head_num = p.head_num;
        f.head_size = p.head_size;
        f.out_tok_stride = p.out_tok_stride;
        f.out_head_stride = p.out_head_stride;
        f.lse_tok_stride = p.lse_tok_stride;
        e = pa::launch_fill(f, s);
        return e == hipSuccess ? PA_OK : hip_fail(e, "fill kernel launch");
    }

    pa_status st = ensure_staging(op, s);
    if (st != PA_OK) return st;
    if (op->done == nullptr) {
        e = hipEventCreateWithFlags(&op->done, hipEventDisableTiming);
        if (e != hipSuccess) {
            op->done = nullptr;
            return hip_fail(e, "hipEventCreateWithFlags");
        }
    }
    auto* ws = static_cast<unsigned char*>(workspace);
    const unsigned char* lists = op->lists;
    const float scale_log2 = p.qk_scale * 1.4426950408889634f;

    if (p.mode == pa::Mode::kDecode) {
        pa::DecodeArgs a{};
        a.items = reinterpret_cast<const pa::DecodeItem*>(lists + p.off_items);
        a.q = p.q;
        a.k = p.k;
        a.v = p.v;
        a.table = p.table;
        a.out = p.out;
        a.lse = p.lse;
        a.slopes = p.slopes;
        a.kscale = p.kscale;
        a.vscale = p.vscale;
        a.part_o = p.workspace_bytes ? reinterpret_cast<float*>(ws + p.off_part_o) : nullptr;
        a.part_ml = p.workspace_bytes ? reinterpret_cast<float*>(ws + p.off_part_ml) : nullptr;
        a.q_tok_stride = p.q_tok_stride;
        a.q_head_stride = p.q_head_stride;
        a.out_tok_stride = p.out_tok_stride;
        a.out_head_stride = p.out_head_stride;
        a.lse_tok_stride = p.lse_tok_stride;
        a.k_blk_stride = p.k_blk_stride;
        a.k_slot_stride = p.k_slot_stride;
        a.k_head_stride = p.k_head_stride;
        a.v_blk_stride = p.v_blk_stride;
        a.v_slot_stride = p.v_slot_stride;
        a.v_head_stride = p.v_head_stride;
        a.table_stride = p.table_stride;
        a.group = p.group;
        a.block_size = p.block_size;
        a.mask_type = p.mask_type;
        a.scale_is_f32 = p.scale_type == PA_F32;
        a.scale_log2 = scale_log2;
        a.wave_heads = p.decode_wave_heads;
        a.aq = antiquant_args(p);
        e = pa::launch_decode(a, static_cast<int>(p.decode_items.size()), p.head_size, bf16, i8, f8,
                              s, op->t_start, op->t_stop);
        if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
        if (!p.combine_items.empty()) {
            pa::CombineArgs c{};
            c.items = reinterpret_cast<const pa::CombineItem*>(lists + p.off_combine);
            c.part_o = a.part_o;
            c.part_ml = a.part_ml;
            c.out = p.out;
            c.lse = p.lse;
            c.out_tok_stride = p.out_tok_stride;
            c.out_head_stride = p.out_head_stride;
            c.lse_tok_stride = p.lse_tok_stride;
            c.group = p.group;
            e = pa::launch_combine(c, static_cast<int>(p.combine_items.size()), p.head_size, bf16, s);
            if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
        }
    } else {
        pa::PrefillArgs a{};
        a.items = reinterpret_cast<const pa::PrefillItem*>(lists + p.off_items);
        a.q = p.q;
        a.k = p.k;
        a.v = p.v;
        a.table = p.table;
        a.out = p.out;
        a.lse = p.lse;
        a.slopes = p.slopes;
        a.kscale = p.kscale;
        a.vscale = p.vscale;
        a.q_tok_stride = p.q_tok_stride;
        a.q_head_stride = p.q_head_stride;
        a.out_tok_stride = p.out_tok_stride;
        a.out_head_stride = p.out_head_stride;
        a.lse_tok_stride = p.lse_tok_stride;
        a.k_blk_stride = p.k_blk_stride;
        a.k_slot_stride = p.k_slot_stride;
        a.k_head_stride = p.k_head_stride;
        a.v_blk_stride = p.v_blk_stride;
        a.v_slot_stride = p.v_slot_stride;
        a.v_head_stride = p.v_head_stride;
        a.table_stride = p.table_stride;
        a.group = p.group;
        a.block_size = p.block_size;
        a.block_shift = -1;
        for (int sh = 0; sh < 31; ++sh)
            if ((1 << sh) == p.block_size) a.block_shift = sh;
        a.mask_type = p.mask_type;
        a.scale_is_f32 = p.scale_type == PA_F32;
        a.scale_log2 = scale_log2;
        a.aq = antiquant_args(p);
        e = pa::launch_prefill(a, static_cast<int>(p.prefill_items.size()), p.head_size, bf16, i8, f8,
                               s, op->t_start, op->t_stop);
        if (e != hipSuccess) return hip_fail(e, "prefill kernel launch");
    }
    // the kernels read the op's work lists from host memory until they finish
    e = hipEventRecord(op->done, s);
    return e == hipSuccess ? PA_OK : hip_fail(e, "hipEventRecord(done)");
}

pa_status pa_kv_cache_append_plan(const pa_tensor* keyNew, const pa_tensor* valueNew,
                                  const pa_tensor* keyCache, const pa_tensor* valueCache,
                                  const pa_tensor* blockTables, const pa_tensor* seqLen,
                                  const pa_tensor* kvSeqLen, pa_op** op) {
    if (op == nullptr) return fail(PA_ERR_NULLPTR, "op must not be NULL");
    *op = nullptr;
    pa_op* h = new (std::nothrow) pa_op();
    if (h == nullptr) return fail(PA_ERR_HOST_ALLOC, "cannot allocate the operator");
    std::string err;
    const pa_status st =
        pa::plan_append(keyNew, valueNew, keyCache, valueCache, blockTables, seqLen, kvSeqLen, h->plan, err);
    if (st != PA_OK) {
        delete h;
        return fail(st, err);
    }
    *op = h;
    g_last_error.clear();
    return PA_OK;
}

pa_status pa_kv_cache_append(pa_op* op, void* stream) {
    if (op == nullptr) return fail(PA_ERR_NULLPTR, "op is NULL");
    const pa::Plan& p = op->plan;
    if (p.mode == pa::Mode::kNoop) return PA_OK;
    if (p.mode != pa::Mode::kAppend)
        return fail(PA_ERR_PARAM_INVALID, "op is not a KV-cache append plan");
    hipStream_t s = static_cast<hipStream_t>(stream);
    pa_status st = ensure_staging(op, s);
    if (st != PA_OK) return st;
    hipError_t e;
    if (op->done == nullptr) {
        e = hipEventCreateWithFlags(&op->done, hipEventDisableTiming);
        if (e != hipSuccess) {
            op->done = nullptr;
            return hip_fail(e, "hipEventCreateWithFlags");
        }
    }
    pa::AppendArgs a{};
    a.items = reinterpret_cast<const pa::AppendItem*>(op->lists + p.off_items);
    a.knew = p.knew;
    a.vnew = p.vnew;
    a.kcache = const_cast<void*>(p.k);
    a.vcache = const_cast<void*>(p.v);
    a.table = p.table;
    a.knew_tok_stride = p.knew_tok_stride;
    a.knew_head_stride = p.knew_head_stride;
    a.vnew_tok_stride = p.vnew_tok_stride;
    a.vnew_head_stride = p.vnew_head_stride;
    a.k_blk_stride = p.k_blk_stride;
    a.k_slot_stride = p.k_slot_stride;
    a.k_head_stride = p.k_head_stride;
    a.v_blk_stride = p.v_blk_stride;
    a.v_slot_stride = p.v_slot_stride;
    a.v_head_stride = p.v_head_stride;
    a.table_stride = p.table_stride;
    a.kv_heads = p.kv_head_num;
    a.row_chunks = p.head_size * p.elem_bytes / 16;
    a.block_size = p.block_size;
    a.elem_bytes = p.elem_bytes;
    e = pa::launch_append(a, static_cast<int>(p.append_items.size()), s, op->t_start, op->t_stop);
    if (e != hipSuccess) return hip_fail(e, "append kernel launch");
    e = hipEventRecord(op->done, s);
    return e == hipSuccess ? PA_OK : hip_fail(e, "hipEventRecord(done)");
}

void pa_op_destroy(pa_op* op) {
    if (op == nullptr) return;
    // kernels enqueued with this op may still read its work lists: wait for the last run
    if (op->done != nullptr) {
        (void)hipEventSynchronize(op->done);
        (void)hipEventDestroy(op->done);
    }
    if (op->lists_dev != nullptr) (void)hipFree(op->lists_dev);
    if (op->staging != nullptr) (void)hipHostFree(op->staging);
    delete op;
}

pa_status pa_op_set_timing_events(pa_op* op, void* start, void* stop) {
    if (op == nullptr) return fail(PA_ERR_NULLPTR, "op is NULL");
    op->t_start = static_cast<hipEvent_t>(start);
    op->t_stop = static_cast<hipEvent_t>(stop);
    return PA_OK;
}

uint64_t pa_op_describe(const pa_op* op, char* buf, uint64_t cap) {
    if (op == nullptr) return 0;
    const pa::Plan& p = op->plan;
    static const char* modes[] = {"noop", "fill", "decode", "prefill", "append"};
    std::string s = "{\"mode\": \"";
    s += modes[static_cast<int>(p.mode)];
    s += "\", \"workspace_bytes\": " + std::to_string(p.workspace_bytes);
    s += ", \"chunk_tiles\": " + std::to_string(p.decode_chunk_tiles);
    s += ", \"decode_wave_heads\": " + std::to_string(p.decode_wave_heads);
    s += ", \"antiquant\": [" + std::to_string(p.kmode) + ", " + std::to_string(p.vmode) + ", " +
         std::to_string(p.koff != nullptr ? 1 : 0) + "]";
    s += ", \"partial_slots\": " + std::to_string(p.partial_slots);
    s += std::string(", \"work_lists\": \"") +
         (op->lists == nullptr ? "none" : (op->lists_dev != nullptr ? "device" : "host")) + "\"";
    s += ", \"decode_items\": [";
    for (size_t i = 0; i < p.decode_items.size(); ++i) {
        const pa::DecodeItem& d = p.decode_items[i];
        if (i) s += ", ";
        s += "[" + std::to_string(d.b) + ", " + std::to_string(d.kvh) + ", " + std::to_string(d.hg) +
             ", " + std::to_string(d.t0) + ", " + std::to_string(d.t1) + ", " +
             std::to_string(d.slot) + ", " + std::to_string(d.qrow) + ", " +
             std::to_string(d.kvlen) + ", " + std::to_string(d.heads) + ", " +
             std::to_string(d.slot_stride) + "]";
    }
    s += "], \"combine_items\": [";
    for (size_t i = 0; i < p.combine_items.size(); ++i) {
        const pa::CombineItem& c = p.combine_items[i];
        if (i) s += ", ";
        s += "[" + std::to_string(c.kvh) + ", " + std::to_string(c.hg) + ", " +
             std::to_string(c.slot0) + ", " + std::to_string(c.nsplit) + ", " +
             std::to_string(c.qrow) + "]";
    }
    s += "], \"prefill_items\": [";
    for (size_t i = 0; i < p.prefill_items.size(); ++i) {
        const pa::PrefillItem& q = p.prefill_items[i];
        if (i) s += ", ";
        s += "[" + std::to_string(q.b) + ", " + std::to_string(q.h) + ", " + std::to_string(q.qbeg) +
             ", " + std::to_string(q.qlen) + ", " + std::to_string(q.kvlen) + ", " +
             std::to_string(q.qrow0) + ", " + std::to_string(q.ktiles) + ", " +
             std::to_string(q.heads) + "]";
    }
    s += "], \"append_items\": [";
    for (size_t i = 0; i < p.append_items.size(); ++i) {
        const pa::AppendItem& q = p.append_items[i];
        if (i) s += ", ";
        s += "[" + std::to_string(q.b) + ", " + std::to_string(q.row0) + ", " + std::to_string(q.pos0) +
             ", " + std::to_string(q.count) + "]";
    }
    s += "]}";
    if (buf != nullptr && cap > 0) {
        const uint64_t n = std::min<uint64_t>(cap - 1, s.size());
        std::memcpy(buf, s.data(), n);
        buf[n] = 0;
    }
    return s.size();
}

const char* pa_status_string(int status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_NULLPTR: return "PA_ERR_NULLPTR: a required pointer is NULL";
        case PA_ERR_PARAM_INVALID: return "PA_ERR_PARAM_INVALID: invalid argument";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: not implemented";
        case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL: workspace too small or misaligned";
        case PA_ERR_HIP: return "PA_ERR_HIP: HIP runtime error";
        case PA_ERR_HOST_ALLOC: return "PA_ERR_HOST_ALLOC: host allocation failed";
        default: return "unknown pa_status";
    }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int32_t pa_version(void) { return 100; }

}  // extern "C"
