// Seeded random fuzz of the host planner (phase 1), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_native_checks.py.  Plain C++: it links the
// planner alone and hands it descriptors with fake, aligned device addresses (the
// planner never dereferences them) and real host length arrays.
//
// For every valid random call it checks that the work lists cover the problem exactly
// once: decode -- every (sequence with one query, kv head, head group) has tile ranges
// partitioning [0, ceil(kvSeqLen / 32)), split groups own consecutive partial slots and
// one combine item, which the group's first split hands on; prefill -- every (sequence,
// query head, query row) lies in exactly one item, whose key-tile count is that of its
// rows' last visible key, and no-op padding items only end a per-XCD list.  Random
// invalid calls must be refused with an error status.  Exit status 0 = all passed.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "pa_internal.h"

namespace {

int g_failures = 0;

#define CHECK(cond, ...)                                                  \
    do {                                                                  \
        if (!(cond)) {                                                    \
            std::fprintf(stderr, "case %d: check failed: %s: ", g_case, #cond); \
            std::fprintf(stderr, __VA_ARGS__);                           \
            std::fprintf(stderr, "\n");                                   \
            ++g_failures;                                                 \
            return;                                                       \
        }                                                                 \
    } while (0)

int g_case = 0;
constexpr uintptr_t kFake = 0x7f0000000000ull;   // 256-aligned, never dereferenced

pa_tensor desc(std::vector<int64_t> shape, int32_t dtype, uintptr_t ptr = kFake,
               std::vector<int64_t> stride = {}) {
    pa_tensor t{};
    t.data = reinterpret_cast<void*>(ptr);
    t.dtype = dtype;
    t.ndim = static_cast<int32_t>(shape.size());
    if (stride.empty()) {
        stride.assign(shape.size(), 1);
        for (int i = static_cast<int>(shape.size()) - 2; i >= 0; --i)
            stride[i] = stride[i + 1] * shape[i + 1];
    }
    for (size_t i = 0; i < shape.size(); ++i) {
        t.shape[i] = shape[i];
        t.stride[i] = stride[i];
    }
    return t;
}

struct Call {
    std::vector<int32_t> ql, kl;
    int H = 1, Hkv = 1, D = 64, bs = 16, mask = 0, table_w = 1;
    int32_t qtype = PA_F16, kvtype = PA_F16;
    int64_t blocks = 1;
    bool lse = false, head_major = false, two_d_query = false;
};

pa_status run_plan(const Call& c, const pa::PlanConfig& cfg, pa::Plan& p, std::string& err) {
    int64_t T = 0;
    for (int32_t q : c.ql) T += q;
    const int B = static_cast<int>(c.ql.size());
    pa_tensor q = c.two_d_query ? desc({T, int64_t(c.H) * c.D}, c.qtype)
                                : desc({T, c.H, c.D}, c.qtype);
    pa_tensor out = desc({T, c.H, c.D}, c.qtype);
    pa_tensor k, v;
    if (c.head_major) {   // (blocks, kvHeads, slots, D) storage passed as its permuted view
        const std::vector<int64_t> st = {int64_t(c.Hkv) * c.bs * c.D, c.D, int64_t(c.bs) * c.D, 1};
        k = desc({c.blocks, c.bs, c.Hkv, c.D}, c.kvtype, kFake, st);
        v = desc({c.blocks, c.bs, c.Hkv, c.D}, c.kvtype, kFake, st);
    } else {
        k = desc({c.blocks, c.bs, c.Hkv, c.D}, c.kvtype);
        v = desc({c.blocks, c.bs, c.Hkv, c.D}, c.kvtype);
    }
    pa_tensor table = desc({B, c.table_w}, PA_I32);
    pa_tensor sl = desc({B}, PA_I32, reinterpret_cast<uintptr_t>(c.ql.data()));
    pa_tensor kvl = desc({B}, PA_I32, reinterpret_cast<uintptr_t>(c.kl.data()));
    pa_tensor slopes = desc({c.H}, PA_F32);
    pa_tensor lse = desc({T, c.H}, PA_F32);
    const bool one_byte = c.kvtype == PA_I8 || c.kvtype == PA_F8E4M3;
    pa_tensor ks = desc({c.Hkv, c.D}, PA_F32), vs = desc({c.Hkv, c.D}, PA_F32);
    return pa::plan(&q, &k, &v, &table, nullptr, &sl, &kvl,
                    c.mask == PA_MASK_ALIBI ? &slopes : nullptr, c.mask, c.H, c.Hkv, 0.125f,
                    one_byte ? &ks : nullptr, one_byte ? &vs : nullptr, nullptr, nullptr, 0, 0,
                    &out, c.lse ? &lse : nullptr, cfg, p, err);
}

void check_decode(const Call& c, const pa::Plan& p) {
    const int geff_groups = (c.H / c.Hkv + pa::kHeadPack - 1) / pa::kHeadPack;
    std::map<std::tuple<int, int, int>, std::vector<std::tuple<int, int, int>>> parts;
    std::set<int> written;
    for (const pa::DecodeItem& it : p.decode_items) {
        CHECK(it.heads == 1 || it.heads == 4, "heads %d", it.heads);
        CHECK(it.t0 >= 0 && it.t1 >= it.t0, "range %d..%d", it.t0, it.t1);
        for (int w = 0; w < it.heads; ++w) {
            const int slot = it.slot < 0 ? -1 : it.slot + w * it.slot_stride;
            parts[{it.b, it.kvh + w, it.hg}].emplace_back(it.t0, it.t1, slot);
            if (it.comb >= 0 && it.t0 == 0) {
                const size_t ci = static_cast<size_t>(it.comb + w);
                CHECK(ci < p.combine_items.size(), "combine index %zu", ci);
                const pa::CombineItem& cb = p.combine_items[ci];
                CHECK(cb.kvh == it.kvh + w && cb.hg == it.hg && cb.slot0 == slot &&
                          cb.nsplit == it.nsplit && cb.qrow == it.qrow,
                      "combine item %zu does not match its first split", ci);
                CHECK(written.insert(static_cast<int>(ci)).second, "combine item %zu twice", ci);
            }
        }
    }
    CHECK(written.size() == p.combine_items.size(), "%zu of %zu combine items handed on",
          written.size(), p.combine_items.size());
    std::set<int> slots;
    for (size_t b = 0; b < c.ql.size(); ++b) {
        for (int kvh = 0; kvh < c.Hkv; ++kvh) {
            for (int hg = 0; hg < geff_groups; ++hg) {
                auto itp = parts.find({static_cast<int>(b), kvh, hg});
                if (c.ql[b] != 1) {
                    CHECK(itp == parts.end(), "items for sequence %zu without a query", b);
                    continue;
                }
                CHECK(itp != parts.end(), "no item for (%zu, %d, %d)", b, kvh, hg);
                auto v = itp->second;
                std::sort(v.begin(), v.end());
                int cur = 0;
                for (auto& [t0, t1, slot] : v) {
                    CHECK(t0 == cur, "gap or overlap at tile %d", t0);
                    cur = t1;
                    if (v.size() > 1) CHECK(slots.insert(slot).second, "slot %d reused", slot);
                    else CHECK(slot == -1, "single split with a slot");
                }
                CHECK(cur == (c.kl[b] + 31) / 32, "tiles %d of %d", cur, (c.kl[b] + 31) / 32);
                parts.erase(itp);
            }
        }
    }
    CHECK(parts.empty(), "items for unknown groups");
    CHECK(static_cast<int>(slots.size()) == p.partial_slots, "slots %zu vs %d", slots.size(),
          p.partial_slots);
    for (int s : slots) CHECK(s >= 0 && s < p.partial_slots, "slot %d out of range", s);
}

void check_prefill(const Call& c, const pa::Plan& p, const pa::PlanConfig& cfg) {
    // per-XCD lists interleaved by position (none when the XCD order is switched off)
    const int xcds = cfg.prefill_xcd_order == 0 ? 1
                     : cfg.compute_units % pa::kCusPerXcd == 0
                         ? std::max(1, std::min(8, cfg.compute_units / pa::kCusPerXcd)) : 1;
    const auto& items = p.prefill_items;
    CHECK(items.size() % xcds == 0, "%zu items for %d XCDs", items.size(), xcds);
    const bool causal = c.mask == PA_MASK_CAUSAL || c.mask == PA_MASK_ALIBI;
    std::vector<int64_t> q0(c.ql.size() + 1, 0);
    for (size_t b = 0; b < c.ql.size(); ++b) q0[b + 1] = q0[b] + c.ql[b];
    std::set<std::tuple<int, int, int>> covered;
    for (size_t pos = 0; pos < items.size(); ++pos) {
        const pa::PrefillItem& it = items[pos];
        if (it.heads == 0) {
            for (size_t q = pos; q < items.size(); q += xcds)
                CHECK(items[q].heads == 0, "padding item %zu inside an XCD list", pos);
            continue;
        }
        CHECK(it.heads == 1 || it.heads == 2 || it.heads == 4, "heads %d", it.heads);
        const int g = c.H / c.Hkv;
        CHECK(g % it.heads == 0 && it.h / g == (it.h + it.heads - 1) / g, "heads cross kv groups");
        CHECK(it.b >= 0 && it.b < static_cast<int>(c.ql.size()), "sequence %d", it.b);
        CHECK(it.qlen == c.ql[it.b] && it.kvlen == c.kl[it.b] && it.qrow0 == q0[it.b],
              "lengths of sequence %d", it.b);
        const int rows = pa::kPrefillBM / it.heads;
        const int r1 = std::min(it.qbeg + rows, it.qlen);
        int64_t last = -1;
        for (int i = it.qbeg; i < r1; ++i) {
            for (int h = it.h; h < it.h + it.heads; ++h)
                CHECK(covered.insert({it.b, h, i}).second, "row (%d, %d, %d) twice", it.b, h, i);
            last = std::max<int64_t>(last, causal ? std::min<int64_t>(int64_t(it.kvlen) - it.qlen + i,
                                                                      it.kvlen - 1)
                                                  : it.kvlen - 1);
        }
        const int want = last < 0 ? 0 : static_cast<int>(last / pa::kPrefillBN + 1);
        CHECK(it.ktiles == want, "ktiles %d, want %d", it.ktiles, want);
    }
    size_t expect = 0;
    for (size_t b = 0; b < c.ql.size(); ++b) expect += size_t(c.ql[b]) * c.H;
    CHECK(covered.size() == expect, "%zu of %zu rows covered", covered.size(), expect);
}

Call random_call(std::mt19937_64& rng, bool decode) {
    auto pick = [&](std::initializer_list<int> xs) {
        std::vector<int> v(xs);
        return v[std::uniform_int_distribution<size_t>(0, v.size() - 1)(rng)];
    };
    auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
    Call c;
    const int B = uni(1, decode ? 70 : 12);
    c.Hkv = pick({1, 2, 3, 4, 8});
    c.H = c.Hkv * pick({1, 2, 4, 8, 12, 24, 32});
    c.D = pick({64, 128});
    c.kvtype = pick({PA_F16, PA_BF16, PA_I8, PA_F8E4M3});
    c.qtype = (c.kvtype == PA_F16 || c.kvtype == PA_BF16) ? c.kvtype : pick({PA_F16, PA_BF16});
    const bool one_byte = c.kvtype == PA_I8 || c.kvtype == PA_F8E4M3;
    c.bs = one_byte ? pick({32, 64, 96, 128, 256}) : pick({16, 32, 48, 64, 80, 128, 1024});
    c.mask = pick({PA_MASK_NONE, PA_MASK_CAUSAL, PA_MASK_ALIBI});
    c.lse = uni(0, 1) == 1;
    c.head_major = uni(0, 1) == 1;
    c.two_d_query = uni(0, 3) == 0;
    int64_t need = 0;
    int maxb = 0;
    for (int b = 0; b < B; ++b) {
        const int kl = pick({0, 1, 31, 32, 33}) + (uni(0, 3) ? uni(0, decode ? 20000 : 3000) : 0);
        int ql = decode ? uni(0, 1) : (uni(0, 4) == 0 ? 0 : uni(1, 600));
        if (!decode && uni(0, 2) == 0) ql = std::min(ql, kl);   // a prefix before the new tokens
        c.ql.push_back(ql);
        c.kl.push_back(kl);
        need += (kl + c.bs - 1) / c.bs;
        maxb = std::max(maxb, (kl + c.bs - 1) / c.bs);
    }
    int64_t T = 0;
    for (int32_t q : c.ql) T += q;
    if (T == 0) c.ql[0] = 1;
    if (!decode) {
        bool big = false;
        for (int32_t q : c.ql) big = big || q > 1;
        if (!big) c.ql[0] = 2;
    }
    c.blocks = std::max<int64_t>(need + uni(0, 5), 1);
    c.table_w = std::max(maxb + uni(0, 3), 1);
    return c;
}

pa::PlanConfig random_config(std::mt19937_64& rng) {
    auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
    pa::PlanConfig cfg;
    const int cus[] = {256, 256, 256, 128, 64, 32, 80, 304};
    cfg.compute_units = cus[uni(0, 7)];
    if (uni(0, 3) == 0) cfg.decode_chunk_tiles = uni(1, 64);
    if (uni(0, 5) == 0) cfg.decode_target_items = uni(1, 5000);
    if (uni(0, 3) == 0) cfg.decode_wave_heads = uni(0, 1);
    if (uni(0, 3) == 0) cfg.prefill_pair = uni(0, 1);
    if (uni(0, 3) == 0) cfg.prefill_xcd_order = uni(0, 1);
    return cfg;
}

// A valid call broken in one place: the planner must refuse it.
void invalid_case(std::mt19937_64& rng) {
    Call c = random_call(rng, std::uniform_int_distribution<int>(0, 1)(rng) == 0);
    pa::PlanConfig cfg;
    const int kind = std::uniform_int_distribution<int>(0, 6)(rng);
    switch (kind) {
        case 0: c.kl[0] = -1 - c.kl[0]; break;                  // negative length
        case 1: c.ql.back() = -1; break;
        case 2: c.table_w = 0; c.kl[0] = std::max(c.kl[0], 1); break;   // table too narrow
        case 3: c.blocks = 0; c.kl[0] = std::max(c.kl[0], 1); break;   // empty pool
        case 4: c.D = 96; break;                                  // unsupported head size
        case 5: c.bs = 24; break;                                 // block size not a multiple of 16
        case 6: c.Hkv = std::max(c.Hkv, 2); c.H = c.Hkv * 3 + 1; break;   // GQA not divisible
    }
    pa::Plan p;
    std::string err;
    // a zero-block pool is the empty-K/V rule (fill), not an error
    const pa_status st = run_plan(c, cfg, p, err);
    if (kind == 3) {
        CHECK(st == PA_OK && p.mode == pa::Mode::kFill, "empty pool: status %d", st);
        return;
    }
    int64_t T = 0;
    for (int32_t q : c.ql) T += q;
    if (T == 0) {   // an empty query skips verification (the empty-input rule)
        CHECK(st == PA_OK && p.mode == pa::Mode::kNoop, "empty query: status %d", st);
        return;
    }
    CHECK(st != PA_OK, "invalid call (kind %d) accepted", kind);
    CHECK(!err.empty(), "no message for kind %d", kind);
}

}  // namespace

int main(int argc, char** argv) {
    const int n = argc > 1 ? std::atoi(argv[1]) : 300;
    const uint64_t seed = argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 314;
    std::mt19937_64 rng(seed);
    int decode_n = 0, prefill_n = 0;
    for (g_case = 0; g_case < n; ++g_case) {
        const bool decode = g_case % 2 == 0;
        const Call c = random_call(rng, decode);
        const pa::PlanConfig cfg = random_config(rng);
        pa::Plan p;
        std::string err;
        const pa_status st = run_plan(c, cfg, p, err);
        if (st != PA_OK) {
            std::fprintf(stderr, "case %d: valid call refused (%d): %s\n", g_case, st, err.c_str());
            ++g_failures;
            continue;
        }
        if (p.mode == pa::Mode::kDecode) {
            check_decode(c, p);
            ++decode_n;
        } else if (p.mode == pa::Mode::kPrefill) {
            check_prefill(c, p, cfg);
            ++prefill_n;
        }
        if (g_case % 4 == 0) invalid_case(rng);
    }
    std::printf("plan_fuzz: %d cases (%d decode, %d prefill plans), %d failures\n", n, decode_n,
                prefill_n, g_failures);
    return g_failures == 0 ? 0 : 1;
}
