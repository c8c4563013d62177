// C ABI of libpagedattn: two-phase get-workspace-size / execute (PrefixEncoder,
// Definition: GetWorkspaceSize then execute with workspace, size, op and context).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "pa_internal.h"
#include "pa_kernels.h"
#include "pagedattn.h"

// A pinned, device-mapped host buffer holding an op's work lists, which the kernels read
// in place (each workgroup loads its own item once, at start-up), with the event recorded
// after the last kernel that read it.  Buffers are drawn from a pool in phase 1 and given
// back by pa_op_destroy, so steady-state planning allocates nothing.
struct HostLists {
    void* ptr = nullptr;                // host address
    const unsigned char* dev = nullptr; // the same memory as the GPU addresses it
    uint64_t bytes = 0;
    hipEvent_t done = nullptr;
};

struct pa_op {
    pa::Plan plan;
    HostLists lists;                // the plan's work lists, pinned (made in phase 1)
    bool planned_without_device = false;
    // caller's timing events: [0] around the main kernel, [1] around the split-KV combine
    hipEvent_t t_start[2] = {nullptr, nullptr};
    hipEvent_t t_stop[2] = {nullptr, nullptr};
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

// ---------------------------------------------------------------- plan options

constexpr int kNumOptions = PA_OPT_COMPUTE_UNITS + 1;
std::atomic<int32_t> g_options[kNumOptions] = {};   // 0 = automatic (the stored value is v + 1)

int32_t option(int opt) { return g_options[opt].load(std::memory_order_relaxed) - 1; }

// compute units of the current device (cached per device); 256, a full MI355X, when no
// device can be queried (planning on a host without a GPU)
int32_t device_compute_units() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int32_t> cache[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return 256;
    }
    if (dev < kMaxDevices) {
        const int32_t c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    if (dev < kMaxDevices) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

pa::PlanConfig plan_config() {
    pa::PlanConfig c;
    c.compute_units = option(PA_OPT_COMPUTE_UNITS) > 0 ? option(PA_OPT_COMPUTE_UNITS)
                                                       : device_compute_units();
    c.decode_chunk_tiles = option(PA_OPT_DECODE_CHUNK_TILES);
    c.decode_target_items = option(PA_OPT_DECODE_TARGET_ITEMS);
    c.decode_wave_heads = option(PA_OPT_DECODE_WAVE_HEADS);
    c.prefill_pair = option(PA_OPT_PREFILL_PAIR);
    c.prefill_xcd_order = option(PA_OPT_PREFILL_XCD_ORDER);
    return c;
}

// ------------------------------------------------------- pinned work-list buffers

std::mutex g_pool_mu;
std::vector<HostLists> g_pool;      // given back by pa_op_destroy
constexpr size_t kPoolKeep = 64;    // buffers kept for reuse

// A pinned buffer of at least `bytes` whose previous user's kernels have finished.
pa_status acquire_lists(uint64_t bytes, HostLists& out) {
    {
        std::lock_guard<std::mutex> lock(g_pool_mu);
        for (size_t i = 0; i < g_pool.size(); ++i) {
            HostLists& c = g_pool[i];
            if (c.bytes < bytes) continue;
            const hipError_t q = hipEventQuery(c.done);
            if (q == hipErrorNotReady) continue;
            (void)hipGetLastError();
            out = c;
            g_pool.erase(g_pool.begin() + static_cast<std::ptrdiff_t>(i));
            return PA_OK;
        }
    }
    HostLists c;
    c.bytes = std::max<uint64_t>(4096, bytes);
    // coherent: a buffer handed to a new op is never seen stale through a GPU cache
    hipError_t e = hipHostMalloc(&c.ptr, c.bytes, hipHostMallocMapped | hipHostMallocCoherent);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc(work lists)");
    void* dev = nullptr;
    e = hipHostGetDevicePointer(&dev, c.ptr, 0);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c.done, hipEventDisableTiming);
    if (e != hipSuccess) {
        (void)hipHostFree(c.ptr);
        return hip_fail(e, "device mapping of the work lists");
    }
    c.dev = static_cast<const unsigned char*>(dev);
    out = c;
    return PA_OK;
}

void release_lists(HostLists& c) {
    if (c.ptr == nullptr) return;
    HostLists drop;
    {
        std::lock_guard<std::mutex> lock(g_pool_mu);
        g_pool.push_back(c);
        if (g_pool.size() > kPoolKeep) {
            // free the oldest buffer whose last reader has finished
            for (size_t i = 0; i < g_pool.size(); ++i) {
                if (hipEventQuery(g_pool[i].done) == hipErrorNotReady) continue;
                drop = g_pool[i];
                g_pool.erase(g_pool.begin() + static_cast<std::ptrdiff_t>(i));
                break;
            }
            (void)hipGetLastError();
        }
    }
    if (drop.ptr != nullptr) {
        (void)hipEventDestroy(drop.done);
        (void)hipHostFree(drop.ptr);
    }
    c = HostLists{};
}

// Write the plan's work lists into the op's pinned buffer (phase 1).  Without a usable
// HIP device (planning on a host without a GPU) the op is left without one; its execute
// then fails.
pa_status make_host_lists(pa_op* op) {
    const pa::Plan& p = op->plan;
    if (p.items_bytes == 0) return PA_OK;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
        (void)hipGetLastError();
        op->planned_without_device = true;
        return PA_OK;
    }
    pa_status st = acquire_lists(p.items_bytes, op->lists);
    if (st != PA_OK) return st;
    auto* base = static_cast<unsigned char*>(op->lists.ptr);
    std::memset(base, 0, p.items_bytes);
    if (p.mode == pa::Mode::kDecode) {
        std::memcpy(base + p.off_items, p.decode_items.data(),
                    p.decode_items.size() * sizeof(pa::DecodeItem));
    } else if (p.mode == pa::Mode::kPrefill) {
        std::memcpy(base + p.off_items, p.prefill_items.data(),
                    p.prefill_items.size() * sizeof(pa::PrefillItem));
    } else if (p.mode == pa::Mode::kAppend) {
        std::memcpy(base + p.off_items, p.append_items.data(),
                    p.append_items.size() * sizeof(pa::AppendItem));
    }
    return PA_OK;
}

// Checks shared by the execute calls (workspace size and alignment, work lists present).
pa_status check_execute(const pa_op* op, const unsigned char* ws, uint64_t ws_size) {
    const pa::Plan& p = op->plan;
    if (ws_size < p.workspace_bytes)
        return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                    "workspace of " + std::to_string(ws_size) + " bytes, need " +
                        std::to_string(p.workspace_bytes));
    if (p.workspace_bytes > 0 && ws == nullptr) return fail(PA_ERR_NULLPTR, "workspace is NULL");
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return fail(PA_ERR_PARAM_INVALID, "workspace must be 256-byte aligned");
    if (p.items_bytes == 0 || op->lists.dev != nullptr) return PA_OK;
    return fail(PA_ERR_HIP, op->planned_without_device
                                ? "the op was planned without a HIP device: plan it again"
                                : "the op has no work lists");
}

// ------------------------------------------------------- static scratch
// Workspace of pa_paged_attention_static, for callers that cannot allocate: a file-scope
// device array of kScratchBytes, one copy per device (each GPU the library runs on holds
// its own until the process ends).  Host code never uses the array's name as an address
// (on the host it is only a stand-in for the symbol): the device address of each copy is
// taken once per device with hipGetSymbolAddress, with that device current, and kept.
constexpr uint64_t kScratchBytes = uint64_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch_ptr[kMaxScratchDevices] = {};

pa_status scratch_on_device(int dev, unsigned char** out) {
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(PA_ERR_PARAM_INVALID, "device " + std::to_string(dev) + " out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || ptr == nullptr)
            return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                            "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = static_cast<unsigned char*>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return PA_OK;
}

pa_status execute_attention(pa_op* op, unsigned char* ws, uint64_t workspaceSize, hipStream_t s);

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
    pa_status st = pa::plan(query, key, value, blockTables, mask, seqLen, kvSeqLen, slopes,
                            maskType, headNum, kvHeadNum, qkScale, keyAntiquantScale,
                            valueAntiquantScale, keyAntiquantOffset, valueAntiquantOffset,
                            keyAntiquantMode, valueAntiquantMode, attnOut, lse, plan_config(),
                            h->plan, err);
    if (st != PA_OK) {
        delete h;
        return fail(st, err);
    }
    st = make_host_lists(h);
    if (st != PA_OK) {
        delete h;
        return st;
    }
    *workspaceSize = h->plan.workspace_bytes;
    *op = h;
    g_last_error.clear();
    return PA_OK;
}

pa_status pa_paged_attention(void* workspace, uint64_t workspaceSize, pa_op* op, void* stream) {
    if (op == nullptr) return fail(PA_ERR_NULLPTR, "op is NULL");
    if (op->plan.mode == pa::Mode::kAppend)
        return fail(PA_ERR_PARAM_INVALID, "op is a KV-cache append plan: run it with pa_kv_cache_append");
    return execute_attention(op, static_cast<unsigned char*>(workspace), workspaceSize,
                             static_cast<hipStream_t>(stream));
}

pa_status pa_paged_attention_static(pa_op* op, void* stream) {
    if (op == nullptr) return fail(PA_ERR_NULLPTR, "op is NULL");
    const pa::Plan& p = op->plan;
    if (p.mode == pa::Mode::kAppend)
        return fail(PA_ERR_PARAM_INVALID, "op is a KV-cache append plan: run it with pa_kv_cache_append");
    if (p.mode == pa::Mode::kNoop) return PA_OK;
    if (p.workspace_bytes > kScratchBytes)
        return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                    "the op needs " + std::to_string(p.workspace_bytes) +
                        " bytes of workspace; the static scratch holds " + std::to_string(kScratchBytes) +
                        ": call pa_paged_attention with a workspace");
    hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = -1;
    hipError_t e = hipStreamGetDevice(s, &dev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    unsigned char* ws = nullptr;
    pa_status st = scratch_on_device(dev, &ws);
    if (st != PA_OK) return st;
    return execute_attention(op, ws, kScratchBytes, s);
}

}  // extern "C"

namespace {

// Phase 2 of an attention op with the workspace `ws` (device memory of ws_size bytes).
pa_status execute_attention(pa_op* op, unsigned char* ws, uint64_t workspaceSize, hipStream_t s) {
    const pa::Plan& p = op->plan;
    if (p.mode == pa::Mode::kNoop) return PA_OK;
    pa_status st = check_execute(op, ws, workspaceSize);
    if (st != PA_OK) return st;
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

    const unsigned char* lists = op->lists.dev;
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
        a.part_o = p.partial_slots ? reinterpret_cast<float*>(ws + p.off_part_o) : nullptr;
        a.part_ml = p.partial_slots ? reinterpret_cast<float*>(ws + p.off_part_ml) : nullptr;
        a.comb = p.partial_slots ? reinterpret_cast<pa::CombineItem*>(ws + p.off_combine) : nullptr;
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
        const bool combine = !p.combine_items.empty();
        e = pa::launch_decode(a, static_cast<int>(p.decode_items.size()), p.head_size, bf16, i8, f8,
                              s, op->t_start[0], op->t_stop[0]);
        if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
        if (combine) {
            pa::CombineArgs c{};
            c.items = a.comb;
            c.part_o = a.part_o;
            c.part_ml = a.part_ml;
            c.out = p.out;
            c.lse = p.lse;
            c.out_tok_stride = p.out_tok_stride;
            c.out_head_stride = p.out_head_stride;
            c.lse_tok_stride = p.lse_tok_stride;
            c.group = p.group;
            e = pa::launch_combine(c, static_cast<int>(p.combine_items.size()), p.head_size, bf16, s,
                                   op->t_start[1], op->t_stop[1]);
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
                               s, op->t_start[0], op->t_stop[0]);
        if (e != hipSuccess) return hip_fail(e, "prefill kernel launch");
    }
    // the kernels read the op's pinned work lists: mark their last use
    if (op->lists.done == nullptr) return PA_OK;
    e = hipEventRecord(op->lists.done, s);
    return e == hipSuccess ? PA_OK : hip_fail(e, "hipEventRecord(done)");
}

}  // namespace

extern "C" {

pa_status pa_kv_cache_append_plan(const pa_tensor* keyNew, const pa_tensor* valueNew,
                                  const pa_tensor* keyCache, const pa_tensor* valueCache,
                                  const pa_tensor* blockTables, const pa_tensor* seqLen,
                                  const pa_tensor* kvSeqLen, pa_op** op) {
    if (op == nullptr) return fail(PA_ERR_NULLPTR, "op must not be NULL");
    *op = nullptr;
    pa_op* h = new (std::nothrow) pa_op();
    if (h == nullptr) return fail(PA_ERR_HOST_ALLOC, "cannot allocate the operator");
    std::string err;
    pa_status st =
        pa::plan_append(keyNew, valueNew, keyCache, valueCache, blockTables, seqLen, kvSeqLen, h->plan, err);
    if (st != PA_OK) {
        delete h;
        return fail(st, err);
    }
    st = make_host_lists(h);
    if (st != PA_OK) {
        delete h;
        return st;
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
    pa_status st = check_execute(op, nullptr, 0);
    if (st != PA_OK) return st;
    hipError_t e;
    pa::AppendArgs a{};
    a.items = reinterpret_cast<const pa::AppendItem*>(op->lists.dev + p.off_items);
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
    e = pa::launch_append(a, static_cast<int>(p.append_items.size()), s, op->t_start[0],
                          op->t_stop[0]);
    if (e != hipSuccess) return hip_fail(e, "append kernel launch");
    if (op->lists.done == nullptr) return PA_OK;
    e = hipEventRecord(op->lists.done, s);
    return e == hipSuccess ? PA_OK : hip_fail(e, "hipEventRecord(done)");
}

void pa_op_destroy(pa_op* op) {
    if (op == nullptr) return;
    // the pinned work lists go back to the pool; they are handed out again only once the
    // kernels enqueued by this op's executes have run (their event has completed)
    release_lists(op->lists);
    delete op;
}

pa_status pa_set_plan_option(int option, int32_t value) {
    if (option < PA_OPT_DECODE_CHUNK_TILES || option > PA_OPT_COMPUTE_UNITS)
        return fail(PA_ERR_PARAM_INVALID, "unknown plan option " + std::to_string(option));
    const bool flag = option == PA_OPT_DECODE_WAVE_HEADS || option == PA_OPT_PREFILL_PAIR ||
                      option == PA_OPT_PREFILL_XCD_ORDER;
    if (value < -1 || (flag && value > 1) || (!flag && value > (1 << 20)) || (!flag && value == 0))
        return fail(PA_ERR_PARAM_INVALID, "value " + std::to_string(value) +
                                              " out of range for plan option " + std::to_string(option));
    g_options[option].store(value + 1, std::memory_order_relaxed);
    return PA_OK;
}

int32_t pa_get_plan_option(int option) {
    if (option < PA_OPT_DECODE_CHUNK_TILES || option > PA_OPT_COMPUTE_UNITS) return -1;
    return ::option(option);
}

pa_status pa_op_set_timing_events(pa_op* op, int kernel, void* start, void* stop) {
    if (op == nullptr) return fail(PA_ERR_NULLPTR, "op is NULL");
    if (kernel != PA_TIMED_MAIN && kernel != PA_TIMED_COMBINE)
        return fail(PA_ERR_PARAM_INVALID, "kernel must be PA_TIMED_MAIN or PA_TIMED_COMBINE");
    op->t_start[kernel] = static_cast<hipEvent_t>(start);
    op->t_stop[kernel] = static_cast<hipEvent_t>(stop);
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
    s += ", \"items_bytes\": " + std::to_string(p.items_bytes);
    s += ", \"compute_units\": " + std::to_string(p.compute_units);
    s += ", \"decode_items\": [";
    for (size_t i = 0; i < p.decode_items.size(); ++i) {
        const pa::DecodeItem& d = p.decode_items[i];
        if (i) s += ", ";
        s += "[" + std::to_string(d.b) + ", " + std::to_string(d.kvh) + ", " + std::to_string(d.hg) +
             ", " + std::to_string(d.t0) + ", " + std::to_string(d.t1) + ", " +
             std::to_string(d.slot) + ", " + std::to_string(d.qrow) + ", " +
             std::to_string(d.kvlen) + ", " + std::to_string(d.heads) + ", " +
             std::to_string(d.slot_stride) + ", " + std::to_string(d.comb) + ", " +
             std::to_string(d.nsplit) + "]";
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
