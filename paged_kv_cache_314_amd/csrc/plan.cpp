// Phase 1: argument validation and work planning.  No HIP calls, no device memory:
// runs (and is unit-tested) on a machine without a GPU.
//
// Checks follow the pages where they state one (PrefixEncoder, Members; the constraint
// sections of aclnnFusedInferAttentionScoreV3/V4); each message names the argument.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <sstream>
#include <tuple>
#include <utility>
#include <vector>

#include "pa_internal.h"

namespace pa {

namespace {

struct Fail {
    pa_status status;
    std::string msg;
};

int64_t numel(const pa_tensor* t) {
    int64_t n = 1;
    for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
    return n;
}

int elem_bytes(int32_t dt) {
    switch (dt) {
        case PA_F16:
        case PA_BF16: return 2;
        case PA_I8:
        case PA_F8E4M3: return 1;
        case PA_F32:
        case PA_I32: return 4;
        default: return 0;
    }
}

const char* dtype_name(int32_t dt) {
    switch (dt) {
        case PA_F16: return "f16";
        case PA_BF16: return "bf16";
        case PA_I8: return "i8";
        case PA_F8E4M3: return "f8e4m3";
        case PA_F32: return "f32";
        case PA_I32: return "i32";
        default: return "?";
    }
}

#define REQUIRE(cond, st, text)                     \
    do {                                            \
        if (!(cond)) {                              \
            std::ostringstream os_;                 \
            os_ << text;                            \
            throw Fail{st, os_.str()};              \
        }                                           \
    } while (0)

void check_desc(const pa_tensor* t, const char* name) {
    REQUIRE(t->ndim >= 1 && t->ndim <= 4, PA_ERR_PARAM_INVALID,
            name << ": ndim " << t->ndim << " not in [1, 4]");
    for (int i = 0; i < t->ndim; ++i)
        REQUIRE(t->shape[i] >= 0, PA_ERR_PARAM_INVALID, name << ": negative shape[" << i << "]");
    REQUIRE(elem_bytes(t->dtype) > 0, PA_ERR_PARAM_INVALID, name << ": unknown dtype " << t->dtype);
}

// Contiguous in the C sense (strides of a dense row-major array), ignoring size-1 dims.
bool is_contiguous(const pa_tensor* t) {
    int64_t expect = 1;
    for (int i = t->ndim - 1; i >= 0; --i) {
        if (t->shape[i] != 1 && t->stride[i] != expect) return false;
        expect *= t->shape[i];
    }
    return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [rows, heads, headSize] view of a query/out-like tensor (3-D, or 2-D with heads folded).
struct RowView {
    int64_t rows = 0, heads = 0, d = 0;
    int64_t row_stride = 0, head_stride = 0;
};

RowView row_view(const pa_tensor* t, const char* name, int64_t heads) {
    RowView v;
    if (t->ndim == 3) {
        REQUIRE(t->shape[1] == heads, PA_ERR_PARAM_INVALID,
                name << ": shape[1] = " << t->shape[1] << " but headNum = " << heads);
        REQUIRE(t->stride[2] == 1 || t->shape[2] == 1, PA_ERR_PARAM_INVALID,
                name << ": last dimension must be contiguous");
        v.rows = t->shape[0];
        v.heads = heads;
        v.d = t->shape[2];
        v.row_stride = t->stride[0];
        v.head_stride = t->stride[1];
    } else if (t->ndim == 2) {
        REQUIRE(heads > 0 && t->shape[1] % heads == 0, PA_ERR_PARAM_INVALID,
                name << ": hidden size " << t->shape[1] << " not divisible by headNum " << heads);
        REQUIRE(t->stride[1] == 1 || t->shape[1] == 1, PA_ERR_PARAM_INVALID,
                name << ": last dimension must be contiguous");
        v.rows = t->shape[0];
        v.heads = heads;
        v.d = t->shape[1] / heads;
        v.row_stride = t->stride[0];
        v.head_stride = v.d;
    } else {
        REQUIRE(false, PA_ERR_PARAM_INVALID,
                name << ": expected [nTokens, headNum, headSize] or [nTokens, headNum*headSize]");
    }
    return v;
}

// [blocks, slots, kvHeads, headSize] view of the paged key/value pool.
struct PoolView {
    int64_t blocks = 0, slots = 0, heads = 0, d = 0;
    int64_t blk_stride = 0, slot_stride = 0, head_stride = 0;
};

PoolView pool_view(const pa_tensor* t, const char* name, int64_t kv_heads) {
    PoolView v;
    if (t->ndim == 4) {
        REQUIRE(t->shape[2] == kv_heads, PA_ERR_PARAM_INVALID,
                name << ": shape[2] = " << t->shape[2] << " but kvHeadNum = " << kv_heads);
        REQUIRE(t->stride[3] == 1 || t->shape[3] == 1, PA_ERR_PARAM_INVALID,
                name << ": last dimension must be contiguous");
        v.blocks = t->shape[0];
        v.slots = t->shape[1];
        v.heads = kv_heads;
        v.d = t->shape[3];
        v.blk_stride = t->stride[0];
        v.slot_stride = t->stride[1];
        v.head_stride = t->stride[2];
    } else if (t->ndim == 3) {
        REQUIRE(kv_heads > 0 && t->shape[2] % kv_heads == 0, PA_ERR_PARAM_INVALID,
                name << ": kv hidden " << t->shape[2] << " not divisible by kvHeadNum " << kv_heads);
        REQUIRE(t->stride[2] == 1 || t->shape[2] == 1, PA_ERR_PARAM_INVALID,
                name << ": last dimension must be contiguous");
        v.blocks = t->shape[0];
        v.slots = t->shape[1];
        v.heads = kv_heads;
        v.d = t->shape[2] / kv_heads;
        v.blk_stride = t->stride[0];
        v.slot_stride = t->stride[1];
        v.head_stride = v.d;
    } else {
        REQUIRE(false, PA_ERR_PARAM_INVALID,
                name << ": expected [numBlocks, blockSize, kvHeadNum, headSize] or "
                        "[numBlocks, blockSize, kvHeadNum*headSize]");
    }
    return v;
}

// a 0 / 1 override (< 0: the automatic choice)
bool pick(int32_t override_value, bool automatic) {
    return override_value < 0 ? automatic : override_value != 0;
}

uint64_t align256(uint64_t x) { return (x + 255u) & ~uint64_t(255); }

// Workgroups are handed to the 8 XCDs of the chip round-robin by index (workgroup i runs
// on XCD i % 8), and each XCD has its own L2.  The query tiles of one (sequence, head
// block) all read the same K/V, so they are placed on one XCD at neighbouring dispatch
// positions: they start together, walk the keys at the same pace and share each K/V
// tile through that L2 instead of each fetching it from HBM.  Clusters go to the least
// loaded XCD, heaviest first; the per-XCD lists are padded to equal length with no-op
// items (heads == 0) so that list x, entry k lands at position 8 * k + x.
// Stable counting sort of `v` by key(x) descending (keys in [0, max_key]); the plans' sort
// keys (tile counts, head indices) are small integers, so this replaces a comparison sort
// of the work list in the per-step planning cost.  Falls back to std::stable_sort for a
// key range above 2^16.
template <typename T, typename Key>
void counting_sort_desc(std::vector<T>& v, Key key) {
    int64_t max_key = 0;
    for (const T& x : v) max_key = std::max<int64_t>(max_key, key(x));
    // a key range far above the element count: the prefix pass would dominate
    if (max_key > (int64_t(1) << 16) || max_key > 8 * static_cast<int64_t>(v.size()) + 64) {
        std::stable_sort(v.begin(), v.end(), [&](const T& a, const T& b) { return key(a) > key(b); });
        return;
    }
    std::vector<uint32_t> start(static_cast<size_t>(max_key) + 2, 0);
    for (const T& x : v) ++start[static_cast<size_t>(max_key - key(x)) + 1];
    for (size_t k = 1; k < start.size(); ++k) start[k] += start[k - 1];
    // plain structs: an uninitialised buffer, filled once, copied back
    std::unique_ptr<T[]> out(new T[v.size()]);
    for (const T& x : v) out[start[static_cast<size_t>(max_key - key(x))]++] = x;
    std::copy(out.get(), out.get() + v.size(), v.begin());
}

// cost[i]: the estimated cost of items[i]
std::vector<PrefillItem> xcd_order(const std::vector<PrefillItem>& items, const std::vector<int64_t>& cost,
                                   const PlanConfig& cfg, bool lpt_within) {
    const int kXcds = cfg.compute_units % kCusPerXcd == 0
                          ? std::max(1, std::min(8, cfg.compute_units / kCusPerXcd)) : 1;
    const size_t cus_per_xcd = static_cast<size_t>(cfg.compute_units / kXcds);
    const size_t n = items.size();
    // clusters: the items of one (sequence, head block), in arrival order (heaviest
    // first), at most 1/8 of the items each, so that a few large clusters (one long
    // sequence, few heads) still spread over every XCD
    const size_t cap = std::max<size_t>(1, (n + kXcds - 1) / kXcds);
    int32_t maxb = 0, maxh = 0;
    for (const PrefillItem& it : items) {
        maxb = std::max(maxb, it.b);
        maxh = std::max(maxh, it.h);
    }
    const size_t nh = static_cast<size_t>(maxh) + 1;
    std::vector<int32_t> open((static_cast<size_t>(maxb) + 1) * nh, -1);   // key -> open cluster
    std::vector<int32_t> cid(n);
    std::vector<int64_t> work;
    std::vector<uint32_t> size;
    work.reserve(n);
    size.reserve(n);
    for (size_t i = 0; i < n; ++i) {
        const PrefillItem& it = items[i];
        int32_t& c = open[static_cast<size_t>(it.b) * nh + static_cast<size_t>(it.h)];
        if (c < 0 || size[c] == cap) {
            c = static_cast<int32_t>(work.size());
            work.push_back(0);
            size.push_back(0);
        }
        cid[i] = c;
        work[c] += cost[i];
        ++size[c];
    }
    const size_t nc = work.size();
    // cluster members in arrival order (counting by cluster)
    std::vector<uint32_t> first(nc + 1, 0);
    for (size_t c = 0; c < nc; ++c) first[c + 1] = first[c] + size[c];
    std::vector<uint32_t> fill(first.begin(), first.end() - 1);
    std::vector<uint32_t> members(n);
    for (size_t i = 0; i < n; ++i) members[fill[cid[i]]++] = static_cast<uint32_t>(i);
    // clusters heaviest first (creation order breaks ties), each to the least loaded XCD
    std::vector<int32_t> order(nc);
    for (size_t c = 0; c < nc; ++c) order[c] = static_cast<int32_t>(c);
    counting_sort_desc(order, [&](int32_t c) { return work[c]; });
    std::vector<std::vector<uint32_t>> lists(kXcds);     // positions in items
    for (auto& l : lists) l.reserve(cap + cap / 2);
    std::vector<int64_t> load(kXcds, 0);
    std::vector<int32_t> xcd_of(nc);
    for (const int32_t c : order) {
        int x = 0;
        for (int i = 1; i < kXcds; ++i)
            if (load[i] < load[x]) x = i;
        load[x] += work[c];
        xcd_of[c] = x;
        if (!lpt_within)
            for (uint32_t k = first[c]; k < first[c + 1]; ++k) lists[x].push_back(members[k]);
    }
    // lpt_within (ALiBi, whose items' costs spread widely with the head's slope): each
    // XCD's list in the items' own order, heaviest first, rather than cluster by cluster;
    // the query tiles of one head still start close together, within the round of
    // workgroups that holds them (ALiBi prefix workload: 121 -> 119 us)
    if (lpt_within)
        for (size_t i = 0; i < n; ++i) lists[xcd_of[cid[i]]].push_back(static_cast<uint32_t>(i));
    // An XCD's list that fits one round (at most two workgroups per CU) is placed so that
    // each CU's pair of workgroups is one heavy and one light item: the hardware gives
    // every CU of the XCD its first workgroup before any CU gets a second, so positions
    // k and k + (CUs per XCD) share a CU.  Heaviest first, then the rest lightest first,
    // lets the long items run most of their tiles without a partner wave on their SIMDs
    // (measured: the causal 512-token, 4-sequence GQA workload runs 16% faster than with
    // equal-weight pairs).  Longer lists keep the cluster order (or, under lpt_within, the
    // cost order), which lets the query tiles of one (sequence, head block) share its K/V
    // tiles through the L2.
    if (pick(cfg.prefill_pair, true)) {
        for (auto& l : lists) {
            if (l.size() <= cus_per_xcd || l.size() > 2 * cus_per_xcd) continue;
            counting_sort_desc(l, [&](uint32_t i) { return int64_t(items[i].ktiles); });
            std::reverse(l.begin() + cus_per_xcd, l.end());
        }
    }
    size_t len = 0;
    for (const auto& l : lists) len = std::max(len, l.size());
    std::vector<PrefillItem> out(len * kXcds);   // value-initialised: heads == 0 = no-op
    for (int x = 0; x < kXcds; ++x)
        for (size_t k = 0; k < lists[x].size(); ++k) out[k * kXcds + x] = items[lists[x][k]];
    return out;
}

void plan_impl(const pa_tensor* query, const pa_tensor* key, const pa_tensor* value,
               const pa_tensor* blockTables, const pa_tensor* mask, const pa_tensor* seqLen,
               const pa_tensor* kvSeqLen, const pa_tensor* slopes, int maskType,
               int32_t headNum, int32_t kvHeadNum, float qkScale,
               const pa_tensor* keyScale, const pa_tensor* valueScale,
               const pa_tensor* keyOffset, const pa_tensor* valueOffset, int kmode, int vmode,
               const pa_tensor* attnOut, const pa_tensor* lse, const PlanConfig& cfg, Plan& p) {
    // -- required descriptors (aclnnFusedInferAttentionScoreV3, Constraints: null inputs)
    p.compute_units = cfg.compute_units;
    REQUIRE(query, PA_ERR_NULLPTR, "query is NULL");
    REQUIRE(key, PA_ERR_NULLPTR, "key is NULL");
    REQUIRE(value, PA_ERR_NULLPTR, "value is NULL");
    REQUIRE(blockTables, PA_ERR_NULLPTR, "blockTables is NULL");
    REQUIRE(seqLen, PA_ERR_NULLPTR, "seqLen is NULL");
    REQUIRE(kvSeqLen, PA_ERR_NULLPTR, "kvSeqLen is NULL");
    REQUIRE(attnOut, PA_ERR_NULLPTR, "attnOut is NULL");
    check_desc(query, "query");
    check_desc(attnOut, "attnOut");
    REQUIRE(headNum > 0, PA_ERR_PARAM_INVALID, "headNum must be > 0, got " << headNum);
    REQUIRE(kvHeadNum >= 0, PA_ERR_PARAM_INVALID, "kvHeadNum must be >= 0, got " << kvHeadNum);
    const int32_t kvh_num = kvHeadNum == 0 ? headNum : kvHeadNum;

    // -- empty query/out: nothing to do, verification skipped
    //    (aclnnFusedInferAttentionScoreV4, Constraints, processing when empty)
    if (numel(query) == 0 && numel(attnOut) == 0) {
        p.mode = Mode::kNoop;
        return;
    }

    REQUIRE(query->dtype == PA_F16 || query->dtype == PA_BF16, PA_ERR_PARAM_INVALID,
            "query dtype must be f16 or bf16, got " << dtype_name(query->dtype));
    REQUIRE(attnOut->dtype == query->dtype, PA_ERR_PARAM_INVALID,
            "attnOut dtype " << dtype_name(attnOut->dtype) << " differs from query "
                             << dtype_name(query->dtype));
    const RowView qv = row_view(query, "query", headNum);
    const RowView ov = row_view(attnOut, "attnOut", headNum);
    REQUIRE(qv.rows == ov.rows && qv.d == ov.d, PA_ERR_PARAM_INVALID,
            "attnOut shape differs from query shape");
    REQUIRE(qv.rows > 0 && qv.d > 0, PA_ERR_PARAM_INVALID,
            "query has zero elements but attnOut does not (or the reverse)");
    REQUIRE(ov.row_stride >= ov.heads * ov.d || ov.rows == 1, PA_ERR_PARAM_INVALID,
            "attnOut rows overlap (token stride " << ov.row_stride << ")");
    REQUIRE(std::llabs(ov.head_stride) >= ov.d || ov.heads == 1, PA_ERR_PARAM_INVALID,
            "attnOut heads overlap (head stride " << ov.head_stride << ")");

    p.qtype = static_cast<pa_dtype>(query->dtype);
    p.head_num = headNum;
    p.kv_head_num = kvh_num;
    p.head_size = static_cast<int32_t>(qv.d);
    p.n_tokens = static_cast<int32_t>(qv.rows);
    p.q = query->data;
    p.out = attnOut->data;
    p.q_tok_stride = qv.row_stride;
    p.q_head_stride = qv.head_stride;
    p.out_tok_stride = ov.row_stride;
    p.out_head_stride = ov.head_stride;
    REQUIRE(qv.rows < (int64_t(1) << 31), PA_ERR_UNSUPPORTED, "nTokens >= 2^31");
    REQUIRE(query->data != nullptr, PA_ERR_NULLPTR, "query->data is NULL");
    REQUIRE(attnOut->data != nullptr, PA_ERR_NULLPTR, "attnOut->data is NULL");

    if (lse) {
        check_desc(lse, "lse");
        REQUIRE(lse->dtype == PA_F32, PA_ERR_PARAM_INVALID,
                "lse dtype must be f32, got " << dtype_name(lse->dtype));
        const bool shape_ok = (lse->ndim == 2 || (lse->ndim == 3 && lse->shape[2] == 1)) &&
                              lse->shape[0] == qv.rows && lse->shape[1] == headNum;
        REQUIRE(shape_ok, PA_ERR_PARAM_INVALID, "lse must be [nTokens, headNum] (or [.., .., 1])");
        REQUIRE(lse->stride[1] == 1 || headNum == 1, PA_ERR_PARAM_INVALID,
                "lse head dimension must be contiguous");
        REQUIRE(lse->stride[0] >= headNum || qv.rows == 1, PA_ERR_PARAM_INVALID,
                "lse rows overlap");
        REQUIRE(lse->data != nullptr, PA_ERR_NULLPTR, "lse->data is NULL");
        p.lse = static_cast<float*>(lse->data);
        p.lse_tok_stride = lse->stride[0];
    }

    // -- empty key/value: out = 0, lse = +inf, verification skipped
    check_desc(key, "key");
    check_desc(value, "value");
    if (numel(key) == 0 || numel(value) == 0) {
        p.mode = Mode::kFill;
        return;
    }

    // ------------------------------------------------------------ full checks
    REQUIRE(mask == nullptr, PA_ERR_UNSUPPORTED,
            "mask tensors are not supported; maskType 3 builds the ALiBi bias from slopes");
    REQUIRE(maskType == PA_MASK_NONE || maskType == PA_MASK_CAUSAL || maskType == PA_MASK_ALIBI ||
                maskType == PA_MASK_ALIBI_SQRT || maskType == PA_MASK_ALIBI_LEFT_ALIGN,
            PA_ERR_PARAM_INVALID, "maskType " << maskType << " is not 0, 3, 4, 5 or 9");
    REQUIRE(maskType != PA_MASK_ALIBI_SQRT && maskType != PA_MASK_ALIBI_LEFT_ALIGN,
            PA_ERR_UNSUPPORTED, "maskType " << maskType << " (ALiBi sqrt / left-align) is not implemented");
    REQUIRE(std::isfinite(qkScale), PA_ERR_PARAM_INVALID, "qkScale must be finite");
    REQUIRE(headNum % kvh_num == 0, PA_ERR_PARAM_INVALID,
            "headNum " << headNum << " is not a multiple of kvHeadNum " << kvh_num);
    REQUIRE(qv.d == 64 || qv.d == 128, PA_ERR_UNSUPPORTED,
            "headSize " << qv.d << " not supported (64 or 128)");

    // key / value
    // one-byte caches: INT8 and FLOAT8_E4M3FN (aclnnFusedInferAttentionScoreV3, Constraints,
    // fake-quantization scenario), both dequantised with antiquant scales
    const bool kv_f8 = key->dtype == PA_F8E4M3;
    const bool kv_i8 = key->dtype == PA_I8 || kv_f8;
    REQUIRE(key->dtype == query->dtype || kv_i8, PA_ERR_PARAM_INVALID,
            "key dtype " << dtype_name(key->dtype) << " must equal the query dtype or be i8 / f8e4m3");
    REQUIRE(value->dtype == key->dtype, PA_ERR_PARAM_INVALID, "value dtype differs from key dtype");
    const PoolView kv = pool_view(key, "key", kvh_num);
    const PoolView vv = pool_view(value, "value", kvh_num);
    REQUIRE(key->ndim == value->ndim, PA_ERR_PARAM_INVALID, "key and value shapes differ");
    for (int i = 0; i < key->ndim; ++i)
        REQUIRE(key->shape[i] == value->shape[i], PA_ERR_PARAM_INVALID, "key and value shapes differ");
    REQUIRE(kv.d == qv.d, PA_ERR_PARAM_INVALID,
            "key headSize " << kv.d << " differs from query headSize " << qv.d);
    const int64_t bs = kv.slots;
    const int64_t bs_align = kv_i8 ? 32 : 16;   // aclnnFusedInferAttentionScoreV3: 16 (f16/bf16), 32 (int8, fp8)
    REQUIRE(bs > 0 && bs % bs_align == 0, PA_ERR_PARAM_INVALID,
            "blockSize " << bs << " must be a positive multiple of " << bs_align);
    REQUIRE(bs <= 4096, PA_ERR_UNSUPPORTED, "blockSize " << bs << " > 4096");
    REQUIRE(key->data != nullptr && value->data != nullptr, PA_ERR_NULLPTR, "key/value data is NULL");

    // alignment of every vector access: 16-byte rows
    const int eb_q = 2, eb_kv = kv_i8 ? 1 : 2;
    REQUIRE(aligned16(query->data) && aligned16(attnOut->data) && aligned16(key->data) &&
                aligned16(value->data),
            PA_ERR_PARAM_INVALID, "query/attnOut/key/value data must be 16-byte aligned");
    auto mult16 = [](int64_t stride, int eb) { return (stride * eb) % 16 == 0; };
    REQUIRE(mult16(qv.row_stride, eb_q) && mult16(qv.head_stride, eb_q) &&
                mult16(ov.row_stride, eb_q) && mult16(ov.head_stride, eb_q),
            PA_ERR_PARAM_INVALID, "query/attnOut strides must be multiples of 16 bytes");
    // the kernels address rows inside a block with 32-bit byte offsets
    REQUIRE(kv.slot_stride >= 0 && vv.slot_stride >= 0 && kv.blk_stride >= 0 &&
                vv.blk_stride >= 0 && kv.head_stride >= 0 && vv.head_stride >= 0,
            PA_ERR_PARAM_INVALID, "key/value strides must be non-negative");
    REQUIRE((bs * std::max(kv.slot_stride, vv.slot_stride) + qv.d) * eb_kv < (int64_t(1) << 31),
            PA_ERR_UNSUPPORTED, "a cache block must span less than 2 GiB");
    REQUIRE(mult16(kv.blk_stride, eb_kv) && mult16(kv.slot_stride, eb_kv) &&
                mult16(kv.head_stride, eb_kv) && mult16(vv.blk_stride, eb_kv) &&
                mult16(vv.slot_stride, eb_kv) && mult16(vv.head_stride, eb_kv),
            PA_ERR_PARAM_INVALID, "key/value strides must be multiples of 16 bytes");

    // lengths (host)
    check_desc(seqLen, "seqLen");
    check_desc(kvSeqLen, "kvSeqLen");
    REQUIRE(seqLen->dtype == PA_I32 && kvSeqLen->dtype == PA_I32, PA_ERR_PARAM_INVALID,
            "seqLen and kvSeqLen must be int32");
    REQUIRE(seqLen->ndim == 1 && kvSeqLen->ndim == 1, PA_ERR_PARAM_INVALID,
            "seqLen and kvSeqLen must be 1-D");
    const int64_t B = seqLen->shape[0];
    REQUIRE(kvSeqLen->shape[0] == B, PA_ERR_PARAM_INVALID,
            "seqLen has " << B << " entries, kvSeqLen " << kvSeqLen->shape[0]);
    REQUIRE(B > 0, PA_ERR_PARAM_INVALID, "batch must be > 0");
    REQUIRE(seqLen->data != nullptr && kvSeqLen->data != nullptr, PA_ERR_NULLPTR,
            "seqLen/kvSeqLen data is NULL");
    const int32_t* ql = static_cast<const int32_t*>(seqLen->data);
    const int32_t* kl = static_cast<const int32_t*>(kvSeqLen->data);
    const int64_t qls = seqLen->stride[0], kls = kvSeqLen->stride[0];
    int64_t qsum = 0, need_blocks = 0, max_blocks = 0;
    int32_t max_q = 0;
    for (int64_t b = 0; b < B; ++b) {
        const int32_t q = ql[b * qls], k = kl[b * kls];
        REQUIRE(q >= 0, PA_ERR_PARAM_INVALID, "seqLen[" << b << "] = " << q << " < 0");
        REQUIRE(k >= 0, PA_ERR_PARAM_INVALID, "kvSeqLen[" << b << "] = " << k << " < 0");
        qsum += q;
        max_q = std::max(max_q, q);
        const int64_t nb = (k + bs - 1) / bs;
        need_blocks += nb;
        max_blocks = std::max(max_blocks, nb);
    }
    REQUIRE(qsum == qv.rows, PA_ERR_PARAM_INVALID,
            "sum(seqLen) = " << qsum << " but query has " << qv.rows << " rows");

    // block table (aclnnFusedInferAttentionScoreV3, Constraints, paged attention scenario)
    check_desc(blockTables, "blockTables");
    REQUIRE(blockTables->dtype == PA_I32, PA_ERR_PARAM_INVALID, "blockTables must be int32");
    REQUIRE(blockTables->ndim == 2, PA_ERR_PARAM_INVALID, "blockTables must be 2-D");
    REQUIRE(blockTables->shape[0] == B, PA_ERR_PARAM_INVALID,
            "blockTables has " << blockTables->shape[0] << " rows, batch is " << B);
    REQUIRE(blockTables->shape[1] >= max_blocks, PA_ERR_PARAM_INVALID,
            "blockTables has " << blockTables->shape[1] << " columns, a sequence needs " << max_blocks);
    REQUIRE(blockTables->stride[1] == 1 || blockTables->shape[1] <= 1, PA_ERR_PARAM_INVALID,
            "blockTables columns must be contiguous");
    REQUIRE(kv.blocks >= need_blocks, PA_ERR_PARAM_INVALID,
            "numBlocks " << kv.blocks << " < blocks the sequences need (" << need_blocks << ")");
    REQUIRE(blockTables->data != nullptr || max_blocks == 0, PA_ERR_NULLPTR, "blockTables data is NULL");

    // antiquant parameters (int8 only; aclnnFusedInferAttentionScoreV3, Constraints on
    // the KV antiquant parameters)
    int32_t max_kv = 0;
    for (int64_t b = 0; b < B; ++b) max_kv = std::max(max_kv, kl[b * kls]);
    if (kv_i8) {
        REQUIRE(keyScale != nullptr && valueScale != nullptr, PA_ERR_NULLPTR,
                "int8 / f8e4m3 key/value need keyAntiquantScale and valueAntiquantScale");
        REQUIRE((kmode == PA_ANTIQUANT_PER_CHANNEL || kmode == PA_ANTIQUANT_PER_TOKEN) &&
                    (vmode == PA_ANTIQUANT_PER_CHANNEL || vmode == PA_ANTIQUANT_PER_TOKEN),
                PA_ERR_PARAM_INVALID, "antiquant modes must be 0 (per-channel) or 1 (per-token)");
        REQUIRE(kmode == vmode || (kmode == PA_ANTIQUANT_PER_CHANNEL && vmode == PA_ANTIQUANT_PER_TOKEN),
                PA_ERR_PARAM_INVALID,
                "key and value antiquant modes must be equal, or key per-channel with value per-token");
        REQUIRE((keyOffset == nullptr) == (valueOffset == nullptr), PA_ERR_PARAM_INVALID,
                "keyAntiquantOffset and valueAntiquantOffset must both be given or both be NULL");
        // FLOAT8_E4M3FN: per-channel scales only, no offsets (Constraints on the KV
        // antiquant parameters, per-channel mode)
        REQUIRE(!kv_f8 || (kmode == PA_ANTIQUANT_PER_CHANNEL && vmode == PA_ANTIQUANT_PER_CHANNEL &&
                           keyOffset == nullptr),
                PA_ERR_PARAM_INVALID, "f8e4m3 key/value take per-channel antiquant scales without offsets");
        // one scale (or offset) tensor: shape / dtype for its mode; returns the row stride
        // of a per-token tensor (0 for per-channel)
        auto check_aq = [&](const pa_tensor* t, int mode, const char* name) -> int64_t {
            check_desc(t, name);
            REQUIRE(t->data != nullptr, PA_ERR_NULLPTR, name << " data is NULL");
            if (mode == PA_ANTIQUANT_PER_CHANNEL) {
                REQUIRE(numel(t) == kvh_num * qv.d, PA_ERR_PARAM_INVALID,
                        name << " (per-channel) must hold kvHeadNum*headSize = " << kvh_num * qv.d
                             << " elements, got " << numel(t));
                REQUIRE(is_contiguous(t), PA_ERR_PARAM_INVALID, name << " must be contiguous");
                REQUIRE(t->dtype == PA_F32 || t->dtype == query->dtype, PA_ERR_PARAM_INVALID,
                        name << " (per-channel) dtype must be f32 or the query dtype");
                REQUIRE(reinterpret_cast<uintptr_t>(t->data) % elem_bytes(t->dtype) == 0,
                        PA_ERR_PARAM_INVALID, name << " data must be aligned to its element size");
                return 0;
            }
            REQUIRE(t->dtype == PA_F32, PA_ERR_PARAM_INVALID, name << " (per-token) must be f32");
            const bool lead1 = t->ndim == 3 && t->shape[0] == 1;
            REQUIRE(t->ndim == 2 || lead1, PA_ERR_PARAM_INVALID,
                    name << " (per-token) must be (batch, S) or (1, batch, S)");
            const int r = t->ndim - 2;
            REQUIRE(t->shape[r] == B, PA_ERR_PARAM_INVALID,
                    name << " (per-token) has " << t->shape[r] << " rows, batch is " << B);
            REQUIRE(t->shape[r + 1] >= max_kv, PA_ERR_PARAM_INVALID,
                    name << " (per-token) has " << t->shape[r + 1] << " columns, max kvSeqLen is " << max_kv);
            REQUIRE(t->stride[r + 1] == 1 || t->shape[r + 1] <= 1, PA_ERR_PARAM_INVALID,
                    name << " (per-token) columns must be contiguous");
            REQUIRE(t->stride[r] >= 0 && (t->stride[r] >= t->shape[r + 1] || B == 1),
                    PA_ERR_PARAM_INVALID, name << " (per-token) rows overlap");
            REQUIRE(reinterpret_cast<uintptr_t>(t->data) % 4 == 0, PA_ERR_PARAM_INVALID,
                    name << " (per-token) data must be 4-byte aligned");
            return t->stride[r];
        };
        p.ktok_stride = check_aq(keyScale, kmode, "keyAntiquantScale");
        p.vtok_stride = check_aq(valueScale, vmode, "valueAntiquantScale");
        if (kmode == vmode && kmode == PA_ANTIQUANT_PER_CHANNEL)
            REQUIRE(keyScale->dtype == valueScale->dtype, PA_ERR_PARAM_INVALID,
                    "key and value antiquant scales differ in dtype");
        if (keyOffset != nullptr) {
            for (auto [off, sc, mode, row_stride, name] :
                 {std::tuple{keyOffset, keyScale, kmode, p.ktok_stride, "keyAntiquantOffset"},
                  std::tuple{valueOffset, valueScale, vmode, p.vtok_stride, "valueAntiquantOffset"}}) {
                const int64_t st = check_aq(off, mode, name);
                bool same_shape = off->ndim == sc->ndim;
                for (int i = 0; same_shape && i < off->ndim; ++i) same_shape = off->shape[i] == sc->shape[i];
                REQUIRE(off->dtype == sc->dtype && same_shape && st == row_stride, PA_ERR_PARAM_INVALID,
                        name << " must have the shape, strides and dtype of its scale");
            }
            p.koff = keyOffset->data;
            p.voff = valueOffset->data;
        }
        p.kscale = keyScale->data;
        p.vscale = valueScale->data;
        p.scale_type = static_cast<pa_dtype>(keyScale->dtype);
        p.vscale_type = static_cast<pa_dtype>(valueScale->dtype);
        p.kmode = kmode;
        p.vmode = vmode;
    } else {
        REQUIRE(keyScale == nullptr && valueScale == nullptr, PA_ERR_PARAM_INVALID,
                "antiquant scales given for non-int8 key/value");
        REQUIRE(keyOffset == nullptr && valueOffset == nullptr, PA_ERR_PARAM_INVALID,
                "antiquant offsets given for non-int8 key/value");
        REQUIRE(kmode == PA_ANTIQUANT_PER_CHANNEL && vmode == PA_ANTIQUANT_PER_CHANNEL,
                PA_ERR_PARAM_INVALID, "antiquant modes other than per-channel need int8 key/value");
    }

    // slopes
    if (maskType == PA_MASK_ALIBI) {
        REQUIRE(slopes != nullptr, PA_ERR_NULLPTR, "maskType 3 (ALiBi) needs slopes");
        check_desc(slopes, "slopes");
        REQUIRE(slopes->dtype == PA_F32, PA_ERR_PARAM_INVALID, "slopes must be f32");
        REQUIRE(numel(slopes) == headNum && is_contiguous(slopes), PA_ERR_PARAM_INVALID,
                "slopes must be a contiguous [headNum] tensor");
        REQUIRE(slopes->data != nullptr, PA_ERR_NULLPTR, "slopes data is NULL");
        p.slopes = static_cast<const float*>(slopes->data);
    } else {
        REQUIRE(slopes == nullptr, PA_ERR_PARAM_INVALID, "slopes given but maskType is not 3");
    }

    // ------------------------------------------------------------------ plan
    p.kvtype = static_cast<pa_dtype>(key->dtype);
    p.batch = static_cast<int32_t>(B);
    p.group = headNum / kvh_num;
    p.head_groups = (p.group + kHeadPack - 1) / kHeadPack;
    p.block_size = static_cast<int32_t>(bs);
    p.num_blocks = static_cast<int32_t>(std::min<int64_t>(kv.blocks, INT32_MAX));
    p.mask_type = maskType;
    p.qk_scale = qkScale;
    p.k = key->data;
    p.v = value->data;
    p.table = static_cast<const int32_t*>(blockTables->data);
    p.table_stride = blockTables->stride[0];
    p.k_blk_stride = kv.blk_stride;
    p.k_slot_stride = kv.slot_stride;
    p.k_head_stride = kv.head_stride;
    p.v_blk_stride = vv.blk_stride;
    p.v_slot_stride = vv.slot_stride;
    p.v_head_stride = vv.head_stride;

    std::vector<int32_t> q0(B + 1, 0);
    for (int64_t b = 0; b < B; ++b) q0[b + 1] = q0[b] + ql[b * qls];

    uint64_t off = 0;
    if (max_q <= 1) {
        // ---- decode: split each (sequence, kv head, head group) into tile ranges
        p.mode = Mode::kDecode;
        int64_t total_tiles = 0;
        for (int64_t b = 0; b < B; ++b)
            if (ql[b * qls] == 1) total_tiles += (kl[b * kls] + kDecodeTile - 1) / kDecodeTile;
        total_tiles *= static_cast<int64_t>(kvh_num) * p.head_groups;
        // wave-per-kv-head items when kv heads come in fours and a kv group fits one
        // MFMA column block: the four waves of a workgroup read neighbouring head slices
        // of the same token rows.  Only with enough work to fill the GPU: on short
        // batches splitting one kv head's range over four waves gives the shorter
        // critical path.  The decode_wave_heads option turns it off / on regardless.
        const bool wph_ok = kvh_num % 4 == 0 && p.head_groups == 1;
        const int64_t cus = std::max(1, cfg.compute_units);
        const bool wph_auto = total_tiles >= 64 * cus;
        const bool wph = wph_ok && pick(cfg.decode_wave_heads, wph_auto);
        p.decode_wave_heads = wph ? 1 : 0;
        // About `target` workgroups in all.  Wave-per-head items cover four kv heads.
        // The path is bound by HBM, which stays saturated while about one workgroup per
        // CU is still streaming, and every item pays a start-up latency: so few, long
        // items.  With nearly equal sequence lengths: one item per CU (fewer concurrent
        // streams also keep more DRAM page locality); uneven lengths: three per CU, the
        // lone ones at the end absorbing the imbalance.  The general-antiquant kernel
        // (per-token scales or offsets) needs two workgroups per CU to hide its latency:
        // two and four per CU.
        int64_t max_tiles = 0, n_dec = 0;
        for (int64_t b = 0; b < B; ++b) {
            if (ql[b * qls] != 1) continue;
            max_tiles = std::max<int64_t>(max_tiles, (kl[b * kls] + kDecodeTile - 1) / kDecodeTile);
            ++n_dec;
        }
        const bool even = n_dec > 0 &&
                          4 * max_tiles * n_dec * kvh_num * p.head_groups <= 5 * total_tiles;
        const bool lean_bytes = p.kvtype != PA_F16 && p.kvtype != PA_BF16 &&
                                p.kmode == PA_ANTIQUANT_PER_CHANNEL &&
                                p.vmode == PA_ANTIQUANT_PER_CHANNEL && p.koff == nullptr;
        const bool general_antiquant = (p.kvtype == PA_I8 || p.kvtype == PA_F8E4M3) && !lean_bytes;
        const int rounds = wph ? (even ? (general_antiquant ? 2 : 1) : (general_antiquant ? 4 : 3)) : 0;
        const int target = cfg.decode_target_items > 0
                               ? cfg.decode_target_items
                               : static_cast<int>(wph ? rounds * cus : 8 * cus);
        // Splits per sequence.  A forced chunk size (plan option) gives
        // ceil(tiles / chunk).  Otherwise the target item count is shared out by largest
        // remainder: every sequence gets at least one split and at most one per 8 tiles,
        // and each further split goes to the sequence whose splits are longest, so the
        // items come out nearly equal in length and as many as targeted (a fixed chunk
        // leaves lengths between half a chunk and a chunk, and rounds the count down).
        const int64_t groups_all = int64_t(kvh_num) * p.head_groups;
        const int64_t per_split = wph ? (groups_all + 3) / 4 : groups_all;   // items per split
        std::vector<int32_t> nsplit_of(static_cast<size_t>(B), 1);
        int32_t max_chunk = 0;
        if (cfg.decode_chunk_tiles > 0) {
            const int32_t chunk = cfg.decode_chunk_tiles;
            for (int64_t b = 0; b < B; ++b) {
                if (ql[b * qls] != 1) continue;
                const int32_t tiles = (kl[b * kls] + kDecodeTile - 1) / kDecodeTile;
                nsplit_of[b] = std::max<int32_t>(1, (tiles + chunk - 1) / chunk);
            }
            max_chunk = chunk;
        } else if (n_dec > 0) {
            const int64_t want = std::max<int64_t>(n_dec, (target + per_split / 2) / per_split);
            const int64_t seq_tiles = total_tiles / groups_all;          // tiles over all sequences
            int64_t have = 0;
            for (int64_t b = 0; b < B; ++b) {
                if (ql[b * qls] != 1) continue;
                const int64_t tiles = (kl[b * kls] + kDecodeTile - 1) / kDecodeTile;
                const int64_t cap = std::max<int64_t>(1, tiles / 8);
                const int64_t share = seq_tiles > 0 ? tiles * want / seq_tiles : 1;
                nsplit_of[b] = static_cast<int32_t>(std::min(cap, std::max<int64_t>(1, share)));
                have += nsplit_of[b];
            }
            // the remaining splits, one at a time, to the sequence with the longest splits
            // that may still take one (ties: lowest index, for a deterministic plan)
            using Entry = std::pair<int64_t, int64_t>;    // (tiles * 2^20 / nsplit, -b)
            std::vector<Entry> heap;
            auto key = [&](int64_t b) {
                const int64_t tiles = (kl[b * kls] + kDecodeTile - 1) / kDecodeTile;
                return Entry((tiles << 20) / nsplit_of[b], -b);
            };
            for (int64_t b = 0; b < B; ++b) {
                if (ql[b * qls] != 1) continue;
                const int64_t tiles = (kl[b * kls] + kDecodeTile - 1) / kDecodeTile;
                if (nsplit_of[b] < std::max<int64_t>(1, tiles / 8)) heap.push_back(key(b));
            }
            std::make_heap(heap.begin(), heap.end());
            while (have < want && !heap.empty()) {
                std::pop_heap(heap.begin(), heap.end());
                const int64_t b = -heap.back().second;
                heap.pop_back();
                ++nsplit_of[b];
                ++have;
                const int64_t tiles = (kl[b * kls] + kDecodeTile - 1) / kDecodeTile;
                if (nsplit_of[b] < std::max<int64_t>(1, tiles / 8)) {
                    heap.push_back(key(b));
                    std::push_heap(heap.begin(), heap.end());
                }
            }
        }
        int32_t slots = 0;
        {
            size_t n_items = 0, n_comb = 0;
            for (int64_t b = 0; b < B; ++b) {
                if (ql[b * qls] != 1) continue;
                const int32_t tiles = (kl[b * kls] + kDecodeTile - 1) / kDecodeTile;
                const int64_t nsplit = nsplit_of[b];
                max_chunk = std::max<int32_t>(max_chunk, static_cast<int32_t>((tiles + nsplit - 1) / nsplit));
                n_items += static_cast<size_t>(per_split * nsplit);
                if (nsplit > 1) n_comb += static_cast<size_t>(groups_all);
            }
            p.decode_items.reserve(n_items);
            p.combine_items.reserve(n_comb);
        }
        p.decode_chunk_tiles = max_chunk;
        std::vector<int32_t> bounds;
        for (int64_t b = 0; b < B; ++b) {
            if (ql[b * qls] != 1) continue;
            const int32_t klen = kl[b * kls];
            const int32_t tiles = (klen + kDecodeTile - 1) / kDecodeTile;
            const int32_t nsplit = nsplit_of[b];
            const int32_t groups = kvh_num * p.head_groups;
            // (kv head, head group) g owns partial slots slots + g*nsplit + s.  Items are
            // emitted head-major: the splits of one kv head (or head quad) launch together.
            const int32_t gstep = wph ? 4 : 1;
            const int32_t comb0 = static_cast<int32_t>(p.combine_items.size());
            // split s covers tiles [tiles * s / nsplit, tiles * (s + 1) / nsplit), the same
            // for every kv head of the sequence
            bounds.resize(static_cast<size_t>(nsplit) + 1);
            for (int32_t s = 0; s <= nsplit; ++s)
                bounds[s] = static_cast<int32_t>(int64_t(tiles) * s / nsplit);
            for (int32_t g = 0; g < groups; g += gstep) {
                for (int32_t s = 0; s < nsplit; ++s) {
                    DecodeItem it{};
                    it.b = static_cast<int32_t>(b);
                    it.kvh = g / p.head_groups;
                    it.hg = g % p.head_groups;
                    it.t0 = bounds[s];
                    it.t1 = bounds[s + 1];
                    it.slot = nsplit > 1 ? slots + g * nsplit + s : -1;
                    it.qrow = q0[b];
                    it.kvlen = klen;
                    it.heads = gstep;
                    it.slot_stride = nsplit;
                    it.comb = nsplit > 1 ? comb0 + g : -1;
                    it.nsplit = nsplit;
                    p.decode_items.push_back(it);
                }
            }
            if (nsplit > 1) {
                for (int32_t g = 0; g < groups; ++g) {
                    CombineItem c{};
                    c.kvh = g / p.head_groups;
                    c.hg = g % p.head_groups;
                    c.slot0 = slots + g * nsplit;
                    c.nsplit = nsplit;
                    c.qrow = q0[b];
                    p.combine_items.push_back(c);
                }
                slots += groups * nsplit;
            }
        }
        p.partial_slots = slots;
        // longest ranges first: the hardware hands out workgroups in launch order, so
        // this is a greedy longest-processing-time schedule and shortens the tail
        counting_sort_desc(p.decode_items, [](const DecodeItem& x) { return int64_t(x.t1 - x.t0); });
        const int64_t geff = std::min<int32_t>(p.group, kHeadPack);
        // work list: in the op's pinned host buffer; partials and combine items: in the
        // device workspace
        p.off_items = 0;
        p.items_bytes = align256(p.decode_items.size() * sizeof(DecodeItem));
        p.off_part_o = off;
        off = align256(off + uint64_t(slots) * geff * qv.d * sizeof(float));
        p.off_part_ml = off;
        off = align256(off + uint64_t(slots) * geff * 2 * sizeof(float));
        p.off_combine = off;
        off = align256(off + p.combine_items.size() * sizeof(CombineItem));
        p.workspace_bytes = slots > 0 ? off : 0;
    } else {
        // ---- prefill: (sequence, query-head block, query-row tile) items, heaviest first.
        // A workgroup covers up to 4 query heads of one kv group (so each K/V tile is
        // staged once for all of them) and kPrefillBM / heads query rows.
        p.mode = Mode::kPrefill;
        const bool causal = maskType == PA_MASK_CAUSAL || maskType == PA_MASK_ALIBI;
        const int32_t hpw = (p.group % 4 == 0) ? 4 : (p.group % 2 == 0 ? 2 : 1);
        const int32_t rows = kPrefillBM / hpw;
        for (int64_t b = 0; b < B; ++b) {
            const int32_t qlen = ql[b * qls], klen = kl[b * kls];
            for (int32_t qb = 0; qb < qlen; qb += rows) {
                int64_t last_key;   // last key index any row of the tile can see
                if (causal) {
                    const int64_t last_row = std::min<int64_t>(qb + rows, qlen) - 1;
                    last_key = std::min<int64_t>(int64_t(klen) - qlen + last_row, int64_t(klen) - 1);
                } else {
                    last_key = int64_t(klen) - 1;
                }
                const int32_t ktiles =
                    last_key < 0 ? 0 : static_cast<int32_t>((last_key + kPrefillBN) / kPrefillBN);
                for (int32_t h = 0; h < headNum; h += hpw) {
                    PrefillItem it{};
                    it.b = static_cast<int32_t>(b);
                    it.h = h;
                    it.qbeg = qb;
                    it.qlen = qlen;
                    it.kvlen = klen;
                    it.qrow0 = q0[b];
                    it.ktiles = ktiles;
                    it.heads = hpw;
                    p.prefill_items.push_back(it);
                }
            }
        }
        // Heaviest first (the hardware hands out workgroups in launch order, so this is a
        // longest-processing-time schedule).  An item costs its key tiles, except that
        // under ALiBi the prefix tiles far enough from its rows for their bias alone to
        // make them negligible cost only a bound on their K rows' norms, about a seventh
        // of a computed tile (measured): 20 units a computed tile, 3 a far one.  Which
        // tiles are far depends on the slopes, which live in device memory out of the
        // planner's reach; the usual geometric slopes 2^(-8(h+1)/headNum) are assumed and
        // the kernel's rule applied (other slopes only change the order).
        const bool alibi = maskType == PA_MASK_ALIBI;
        // reach[h] = kFarTileBias / (head h's assumed slope in log2 units): a key is far
        // for head h beyond that distance (the smallest slope of an item's heads is its
        // last head's)
        std::vector<double> reach(alibi ? headNum : 0);
        for (int32_t h = 0; h < static_cast<int32_t>(reach.size()); ++h)
            reach[h] = double(kFarTileBias) /
                       (std::exp2(-8.0 * double(h + 1) / double(headNum)) * 1.4426950408889634);
        auto item_cost = [&](const PrefillItem& x) -> int64_t {
            int64_t far = 0;
            if (alibi && x.ktiles > 0) {
                const int64_t shift = int64_t(x.kvlen) - x.qlen, T = x.ktiles - 1;
                const int64_t P = std::min<int64_t>(shift > 0 ? shift / kPrefillBN : 0, T);
                // tile t (< P) is far iff (pmin - (64 t + 63)) > reach, i.e. 64 t < y: the
                // ceil(y / 64) tiles t >= 0 below that bound
                const double y = double(shift + x.qbeg - (kPrefillBN - 1)) - reach[x.h + x.heads - 1];
                if (y > 0.0) far = std::min<int64_t>(P, static_cast<int64_t>(std::ceil(y * (1.0 / kPrefillBN))));
            }
            return 20 * (int64_t(x.ktiles) - far) + 3 * far;
        };
        const size_t n_items = p.prefill_items.size();
        std::vector<int64_t> cost(n_items);
        for (size_t i = 0; i < n_items; ++i) cost[i] = item_cost(p.prefill_items[i]);
        {
            // heaviest first (stable): positions sorted by cost, then gathered
            std::vector<uint32_t> pos(n_items);
            for (size_t i = 0; i < n_items; ++i) pos[i] = static_cast<uint32_t>(i);
            counting_sort_desc(pos, [&](uint32_t i) { return cost[i]; });
            std::vector<PrefillItem> sorted(n_items);
            std::vector<int64_t> sorted_cost(n_items);
            for (size_t k = 0; k < n_items; ++k) {
                sorted[k] = p.prefill_items[pos[k]];
                sorted_cost[k] = cost[pos[k]];
            }
            p.prefill_items.swap(sorted);
            cost.swap(sorted_cost);
        }
        if (pick(cfg.prefill_xcd_order, true))
            p.prefill_items = xcd_order(p.prefill_items, cost, cfg, alibi);
        p.off_items = 0;
        p.items_bytes = align256(p.prefill_items.size() * sizeof(PrefillItem));
        p.workspace_bytes = 0;
    }
}

}  // namespace

namespace {

// KV-cache append: the new tokens of sequence b (seqLen[b] rows of keyNew / valueNew,
// packed in sequence order like the query) are its last positions,
// p = kvSeqLen[b] - seqLen[b] + i, written to block blockTables[b][p / blockSize],
// slot p % blockSize (aclnnFusedInferAttentionScoreV3, Constraints, paged attention
// scenario: the cache layout; PrefixEncoder, Members: kvSeqLen counts the cached prefix
// plus the new tokens).
void plan_append_impl(const pa_tensor* keyNew, const pa_tensor* valueNew, const pa_tensor* keyCache,
                      const pa_tensor* valueCache, const pa_tensor* blockTables,
                      const pa_tensor* seqLen, const pa_tensor* kvSeqLen, Plan& p) {
    REQUIRE(keyNew && valueNew && keyCache && valueCache && blockTables && seqLen && kvSeqLen,
            PA_ERR_NULLPTR, "keyNew, valueNew, keyCache, valueCache, blockTables, seqLen and "
                            "kvSeqLen are required");
    for (auto [t, name] : {std::pair{keyNew, "keyNew"}, std::pair{valueNew, "valueNew"},
                           std::pair{keyCache, "keyCache"}, std::pair{valueCache, "valueCache"}})
        check_desc(t, name);
    REQUIRE(keyNew->ndim == 3 && valueNew->ndim == 3, PA_ERR_PARAM_INVALID,
            "keyNew / valueNew must be [nTokens, kvHeadNum, headSize]");
    for (int i = 0; i < 3; ++i)
        REQUIRE(keyNew->shape[i] == valueNew->shape[i], PA_ERR_PARAM_INVALID,
                "keyNew and valueNew shapes differ");
    const int64_t T = keyNew->shape[0], hkv = keyNew->shape[1], d = keyNew->shape[2];
    p.mode = Mode::kAppend;
    if (T == 0) {
        p.mode = Mode::kNoop;
        return;
    }
    REQUIRE(hkv > 0 && d > 0, PA_ERR_PARAM_INVALID, "kvHeadNum and headSize must be > 0");
    REQUIRE(keyNew->dtype == keyCache->dtype && valueNew->dtype == valueCache->dtype &&
                keyCache->dtype == valueCache->dtype,
            PA_ERR_PARAM_INVALID, "new tokens and caches must share one dtype");
    REQUIRE(keyCache->dtype == PA_F16 || keyCache->dtype == PA_BF16 || keyCache->dtype == PA_I8 ||
                keyCache->dtype == PA_F8E4M3,
            PA_ERR_PARAM_INVALID, "cache dtype must be f16, bf16, i8 or f8e4m3");
    const int eb = elem_bytes(keyCache->dtype);
    REQUIRE((d * eb) % 16 == 0, PA_ERR_PARAM_INVALID, "headSize * element size must be a multiple of 16 bytes");
    REQUIRE(keyNew->stride[2] == 1 && valueNew->stride[2] == 1, PA_ERR_PARAM_INVALID,
            "keyNew / valueNew last dimension must be contiguous");
    const PoolView kc = pool_view(keyCache, "keyCache", hkv);
    const PoolView vc = pool_view(valueCache, "valueCache", hkv);
    REQUIRE(kc.d == d && vc.d == d && kc.slots == vc.slots && kc.blocks == vc.blocks, PA_ERR_PARAM_INVALID,
            "caches must be [numBlocks, blockSize, kvHeadNum, headSize] matching the new tokens");
    auto mult16 = [&](int64_t stride) { return (stride * eb) % 16 == 0; };
    REQUIRE(mult16(keyNew->stride[0]) && mult16(keyNew->stride[1]) && mult16(valueNew->stride[0]) &&
                mult16(valueNew->stride[1]) && mult16(kc.blk_stride) && mult16(kc.slot_stride) &&
                mult16(kc.head_stride) && mult16(vc.blk_stride) && mult16(vc.slot_stride) &&
                mult16(vc.head_stride),
            PA_ERR_PARAM_INVALID, "strides must be multiples of 16 bytes");
    REQUIRE(aligned16(keyNew->data) && aligned16(valueNew->data) && aligned16(keyCache->data) &&
                aligned16(valueCache->data),
            PA_ERR_PARAM_INVALID, "data must be 16-byte aligned");
    REQUIRE(keyNew->data && valueNew->data && keyCache->data && valueCache->data, PA_ERR_NULLPTR,
            "a tensor's data is NULL");
    const int64_t bs = kc.slots;
    REQUIRE(bs > 0 && bs <= 4096, PA_ERR_PARAM_INVALID, "blockSize must be in [1, 4096]");
    REQUIRE((bs * std::max(kc.slot_stride, vc.slot_stride) + d) * eb < (int64_t(1) << 31),
            PA_ERR_UNSUPPORTED, "a cache block must span less than 2 GiB");

    check_desc(seqLen, "seqLen");
    check_desc(kvSeqLen, "kvSeqLen");
    REQUIRE(seqLen->dtype == PA_I32 && kvSeqLen->dtype == PA_I32 && seqLen->ndim == 1 &&
                kvSeqLen->ndim == 1 && seqLen->shape[0] == kvSeqLen->shape[0] && seqLen->shape[0] > 0,
            PA_ERR_PARAM_INVALID, "seqLen and kvSeqLen must be int32 [batch], batch > 0");
    REQUIRE(seqLen->data && kvSeqLen->data, PA_ERR_NULLPTR, "seqLen/kvSeqLen data is NULL");
    const int64_t B = seqLen->shape[0];
    const int32_t* ql = static_cast<const int32_t*>(seqLen->data);
    const int32_t* kl = static_cast<const int32_t*>(kvSeqLen->data);
    check_desc(blockTables, "blockTables");
    REQUIRE(blockTables->dtype == PA_I32 && blockTables->ndim == 2 && blockTables->shape[0] == B &&
                (blockTables->stride[1] == 1 || blockTables->shape[1] <= 1),
            PA_ERR_PARAM_INVALID, "blockTables must be int32 [batch, maxBlockNum], columns contiguous");
    int64_t row = 0;
    for (int64_t b = 0; b < B; ++b) {
        const int32_t q = ql[b * seqLen->stride[0]], k = kl[b * kvSeqLen->stride[0]];
        REQUIRE(q >= 0 && k >= q, PA_ERR_PARAM_INVALID,
                "sequence " << b << ": need 0 <= seqLen (" << q << ") <= kvSeqLen (" << k << ")");
        REQUIRE(blockTables->shape[1] * bs >= k, PA_ERR_PARAM_INVALID,
                "blockTables has " << blockTables->shape[1] << " columns, sequence " << b << " needs "
                                   << (k + bs - 1) / bs);
        for (int32_t i = 0; i < q; i += kAppendRows) {
            AppendItem it{};
            it.b = static_cast<int32_t>(b);
            it.row0 = static_cast<int32_t>(row + i);
            it.pos0 = k - q + i;
            it.count = std::min(kAppendRows, q - i);
            p.append_items.push_back(it);
        }
        row += q;
    }
    REQUIRE(row == T, PA_ERR_PARAM_INVALID, "sum(seqLen) = " << row << " but keyNew has " << T << " rows");
    REQUIRE(blockTables->data != nullptr, PA_ERR_NULLPTR, "blockTables data is NULL");

    p.kvtype = static_cast<pa_dtype>(keyCache->dtype);
    p.elem_bytes = eb;
    p.batch = static_cast<int32_t>(B);
    p.kv_head_num = static_cast<int32_t>(hkv);
    p.head_size = static_cast<int32_t>(d);
    p.block_size = static_cast<int32_t>(bs);
    p.n_tokens = static_cast<int32_t>(T);
    p.knew = keyNew->data;
    p.vnew = valueNew->data;
    p.knew_tok_stride = keyNew->stride[0];
    p.knew_head_stride = keyNew->stride[1];
    p.vnew_tok_stride = valueNew->stride[0];
    p.vnew_head_stride = valueNew->stride[1];
    p.k = keyCache->data;
    p.v = valueCache->data;
    p.k_blk_stride = kc.blk_stride;
    p.k_slot_stride = kc.slot_stride;
    p.k_head_stride = kc.head_stride;
    p.v_blk_stride = vc.blk_stride;
    p.v_slot_stride = vc.slot_stride;
    p.v_head_stride = vc.head_stride;
    p.table = static_cast<const int32_t*>(blockTables->data);
    p.table_stride = blockTables->stride[0];
    p.off_items = 0;
    p.items_bytes = align256(p.append_items.size() * sizeof(AppendItem));
    p.workspace_bytes = 0;
}

}  // namespace

pa_status plan_append(const pa_tensor* keyNew, const pa_tensor* valueNew, const pa_tensor* keyCache,
                      const pa_tensor* valueCache, const pa_tensor* blockTables,
                      const pa_tensor* seqLen, const pa_tensor* kvSeqLen, Plan& p, std::string& err) {
    try {
        plan_append_impl(keyNew, valueNew, keyCache, valueCache, blockTables, seqLen, kvSeqLen, p);
    } catch (const Fail& f) {
        err = f.msg;
        return f.status;
    } catch (const std::bad_alloc&) {
        err = "host allocation failed while planning";
        return PA_ERR_HOST_ALLOC;
    }
    err.clear();
    return PA_OK;
}

pa_status plan(const pa_tensor* query, const pa_tensor* key, const pa_tensor* value,
               const pa_tensor* blockTables, const pa_tensor* mask, const pa_tensor* seqLen,
               const pa_tensor* kvSeqLen, const pa_tensor* slopes, int maskType,
               int32_t headNum, int32_t kvHeadNum, float qkScale,
               const pa_tensor* keyAntiquantScale, const pa_tensor* valueAntiquantScale,
               const pa_tensor* keyAntiquantOffset, const pa_tensor* valueAntiquantOffset,
               int keyAntiquantMode, int valueAntiquantMode,
               const pa_tensor* attnOut, const pa_tensor* lse, const PlanConfig& cfg, Plan& p,
               std::string& err) {
    try {
        plan_impl(query, key, value, blockTables, mask, seqLen, kvSeqLen, slopes, maskType,
                  headNum, kvHeadNum, qkScale, keyAntiquantScale, valueAntiquantScale,
                  keyAntiquantOffset, valueAntiquantOffset, keyAntiquantMode, valueAntiquantMode,
                  attnOut, lse, cfg, p);
    } catch (const Fail& f) {
        err = f.msg;
        return f.status;
    } catch (const std::bad_alloc&) {
        err = "host allocation failed while planning";
        return PA_ERR_HOST_ALLOC;
    }
    err.clear();
    return PA_OK;
}

}  // namespace pa
