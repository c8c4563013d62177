// Internal types shared by the host planner (plan.cpp) and the HIP launchers.
// Plain C++17: no HIP types, so the planner builds and runs without a GPU.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "pagedattn.h"

namespace pa {

// Token tile one wave consumes per step in the decode kernel.
constexpr int kDecodeTile = 32;
// Heads packed into one decode MFMA column block (the N dimension of 16x16x32).
constexpr int kHeadPack = 16;
// Waves per decode workgroup.
constexpr int kDecodeWaves = 4;
// Compute units per XCD (accelerator complex die) of gfx950: a full MI355X has 8 XCDs
// of 32 CUs; a partitioned one shows fewer whole XCDs.
constexpr int kCusPerXcd = 32;
// Prefill: query rows per workgroup and keys per step.
constexpr int kPrefillBM = 128;
constexpr int kPrefillBN = 64;
// ALiBi over 16-bit K/V: prefix tiles whose bias lies more than this many log2 units
// below that of the workgroup's nearest key, for every row and key, are far tiles, which
// a bound on the scores from their K rows' norms usually shows negligible (64: few far
// tiles then fail the bound and have to be computed).  The planner counts them in an
// item's cost.
constexpr float kFarTileBias = 64.0f;

// What the planner sizes work for, and the overrides of its automatic choices (a value
// < 0 means automatic).  Set by the C ABI from the current device and pa_set_plan_option.
struct PlanConfig {
    int32_t compute_units = 256;        // of the device the op will run on
    int32_t decode_chunk_tiles = -1;    // 32-token tiles per decode work item
    int32_t decode_target_items = -1;   // decode workgroups the planner aims for
    int32_t decode_wave_heads = -1;     // 0 / 1: items of four kv heads, one per wave
    int32_t prefill_pair = -1;          // 0 / 1: heavy + light prefill items per CU
    int32_t prefill_xcd_order = -1;     // 0 / 1: XCD-ordered prefill list
};

enum class Mode : int32_t { kNoop = 0, kFill = 1, kDecode = 2, kPrefill = 3, kAppend = 4 };

// KV-cache append: new tokens per workgroup
constexpr int kAppendRows = 16;

// One append workgroup: `count` consecutive new tokens of sequence b, rows row0 .. of the
// new-token tensors, positions pos0 .. in the sequence.
struct AppendItem {
    int32_t b;
    int32_t row0;
    int32_t pos0;
    int32_t count;
    int32_t pad[4];
};
static_assert(sizeof(AppendItem) == 32, "AppendItem layout");

// One decode workgroup: a range of 32-token tiles of one sequence and
//   heads == 1: one (kv head, head group), the four waves splitting the tile range, or
//   heads == 4: kv heads kvh .. kvh+3 (one head group each), wave w streaming the whole
//               range of kv head kvh + w, so that the four waves read 4 neighbouring
//               head slices of every token row together.
struct DecodeItem {
    int32_t b;        // sequence
    int32_t kvh;      // (first) kv head
    int32_t hg;       // group of up to 16 query heads sharing kvh (0 when heads == 4)
    int32_t t0, t1;   // tile range [t0, t1)
    int32_t slot;     // -1: write out/lse directly; >= 0: partial slot (of kv head kvh)
    int32_t qrow;     // query/out row of this sequence's decode token
    int32_t kvlen;    // kvSeqLen[b]
    int32_t heads;    // 1 or 4 (see above)
    int32_t slot_stride;  // heads == 4: slot of kv head kvh + w is slot + w * slot_stride
    int32_t comb;         // split sequences: index of the combine item of (kvh, hg) (of kv
                          // head kvh + w: comb + w); -1 when the sequence is not split
    int32_t nsplit;       // splits of the sequence (1: not split)
};
static_assert(sizeof(DecodeItem) == 48, "DecodeItem layout");

// One combine workgroup: merge nsplit consecutive partial slots into out/lse.
struct CombineItem {
    int32_t kvh, hg;
    int32_t slot0, nsplit;
    int32_t qrow;
    int32_t pad[3];
};
static_assert(sizeof(CombineItem) == 32, "CombineItem layout");

// One prefill workgroup: `heads` consecutive query heads of one kv group (1, 2 or 4)
// times kPrefillBM / heads query rows of one sequence; wave w takes head
// h + w % heads and rows qbeg + 32 * (w / heads) .. +31.
struct PrefillItem {
    int32_t b;
    int32_t h;        // first query head
    int32_t qbeg;     // first local query row of the tile
    int32_t qlen;     // seqLen[b]
    int32_t kvlen;    // kvSeqLen[b]
    int32_t qrow0;    // packed row of local query 0 of this sequence
    int32_t ktiles;   // key tiles (kPrefillBN) the tile must visit
    int32_t heads;    // query heads sharing the workgroup's K/V tiles
};
static_assert(sizeof(PrefillItem) == 32, "PrefillItem layout");

// Visiting order of a prefill wave's key tiles (plain constexpr arithmetic, used by the
// kernel and checked on the host).  The wave owns local query rows wave_q0 ..
// wave_q0 + 31 of a sequence with qlen queries and kvlen keys; its item visits key
// tiles 0 .. T = ktiles - 1 (tiles of kPrefillBN keys), one per step k = 0 .. T:
//   step 0: tile T, the one nearest the queries;
//   steps 1 .. P: the P tiles holding only keys before the new tokens (visible to every
//           query row under a causal mask), P - 1 down to 0;
//   steps P + 1 .. T: the rest of the diagonal, T - 1 down to P.
// Without a causal mask P = 0 and the order is T down to 0.  The wave computes only
// tiles t <= t_act (its rows see no key of a higher tile; -1: none), and k_first is its
// first computed step (its output accumulators are still zero there).
struct PrefillVisit {
    int T, t_act, P, k_first;
};

constexpr PrefillVisit prefill_visit(int ktiles, bool causal, int qlen, int kvlen, int wave_q0) {
    const int T = ktiles - 1;
    const int shift = kvlen - qlen;                 // position of local query 0
    const int wave_q1 = (wave_q0 + 31 < qlen - 1) ? wave_q0 + 31 : qlen - 1;
    const int wave_pmax = shift + wave_q1;          // highest position among the rows
    const bool live = wave_q0 < qlen;
    int t_act = -1;
    if (live) {
        if (!causal) t_act = T;
        else if (wave_pmax >= 0) t_act = (T < wave_pmax / kPrefillBN) ? T : wave_pmax / kPrefillBN;
    }
    int P = 0;
    if (causal && shift > 0) P = (shift / kPrefillBN < T) ? shift / kPrefillBN : T;
    if (P < 0) P = 0;
    // a live wave sees every prefix tile (t_act >= P), so after tile T the first tile it
    // computes is P - 1 if there is a prefix, else the first diagonal tile <= t_act
    const int k_first = (t_act == T) ? 0 : (P > 0 ? 1 : T - t_act);
    return PrefillVisit{T, t_act, P, k_first};
}

constexpr int prefill_tile_of(const PrefillVisit& v, int k) {
    return k == 0 ? v.T : (k <= v.P ? v.P - k : v.T - (k - v.P));
}

// Everything phase 2 needs; produced by plan().
struct Plan {
    Mode mode = Mode::kNoop;
    pa_dtype qtype = PA_F16;     // query / out dtype
    pa_dtype kvtype = PA_F16;    // key / value dtype
    pa_dtype scale_type = PA_F32;   // key antiquant scale dtype
    pa_dtype vscale_type = PA_F32;  // value antiquant scale dtype
    int32_t kmode = 0, vmode = 0;   // antiquant modes: 0 per-channel, 1 per-token
    int32_t batch = 0, head_num = 0, kv_head_num = 0, group = 1, head_groups = 1;
    int32_t head_size = 0, block_size = 0, num_blocks = 0, n_tokens = 0;
    int32_t mask_type = 0;
    float qk_scale = 1.0f;

    // device pointers captured in phase 1
    const void* q = nullptr;
    const void* k = nullptr;
    const void* v = nullptr;
    const int32_t* table = nullptr;
    void* out = nullptr;
    float* lse = nullptr;
    const float* slopes = nullptr;
    const void* kscale = nullptr;
    const void* vscale = nullptr;
    const void* koff = nullptr;     // antiquant offsets (NULL: symmetric)
    const void* voff = nullptr;
    int64_t ktok_stride = 0, vtok_stride = 0;   // per-token scale / offset row strides

    // strides in elements
    int64_t q_tok_stride = 0, q_head_stride = 0, out_tok_stride = 0, out_head_stride = 0;
    int64_t lse_tok_stride = 0;
    int64_t k_blk_stride = 0, k_slot_stride = 0, k_head_stride = 0;
    int64_t v_blk_stride = 0, v_slot_stride = 0, v_head_stride = 0;
    int64_t table_stride = 0;

    // work lists (the kernels read them from the op's pinned host buffer)
    std::vector<DecodeItem> decode_items;
    std::vector<CombineItem> combine_items;
    std::vector<PrefillItem> prefill_items;
    std::vector<AppendItem> append_items;

    // KV-cache append: new-token tensors [nTokens, kvHeadNum, headSize] (strides in
    // elements) and the caches written (k / v above are the caches, kvtype their dtype)
    const void* knew = nullptr;
    const void* vnew = nullptr;
    int64_t knew_tok_stride = 0, knew_head_stride = 0, vnew_tok_stride = 0, vnew_head_stride = 0;
    int32_t elem_bytes = 0;
    int32_t decode_chunk_tiles = 0;
    int32_t decode_wave_heads = 0;   // 1: items of 4 kv heads, one per wave
    int32_t partial_slots = 0;
    int32_t compute_units = 0;       // the device size the lists were made for

    // work lists: in the op's pinned, device-mapped host buffer (offset off_items,
    // items_bytes); the device workspace holds the split-KV partials (off_part_o,
    // off_part_ml) and the combine items, written there by the decode kernel's first
    // split of each (sequence, kv head, head group) (off_combine); all 256-aligned
    uint64_t off_items = 0, items_bytes = 0;
    uint64_t off_part_o = 0, off_part_ml = 0, off_combine = 0, workspace_bytes = 0;
};

// KV-cache append planning (validation + work list).  On failure returns a status and
// sets `err`.
pa_status plan_append(const pa_tensor* keyNew, const pa_tensor* valueNew, const pa_tensor* keyCache,
                      const pa_tensor* valueCache, const pa_tensor* blockTables,
                      const pa_tensor* seqLen, const pa_tensor* kvSeqLen, Plan& p, std::string& err);

// Validation + planning for the device described by `cfg`.  On failure returns a status and sets `err`.
pa_status plan(const pa_tensor* query, const pa_tensor* key, const pa_tensor* value,
               const pa_tensor* blockTables, const pa_tensor* mask,
               const pa_tensor* seqLen, const pa_tensor* kvSeqLen, const pa_tensor* slopes,
               int maskType, int32_t headNum, int32_t kvHeadNum, float qkScale,
               const pa_tensor* keyAntiquantScale, const pa_tensor* valueAntiquantScale,
               const pa_tensor* keyAntiquantOffset, const pa_tensor* valueAntiquantOffset,
               int keyAntiquantMode, int valueAntiquantMode,
               const pa_tensor* attnOut, const pa_tensor* lse, const PlanConfig& cfg, Plan& p,
               std::string& err);

}  // namespace pa
