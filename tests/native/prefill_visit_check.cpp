// Exhaustive host check of the prefill kernel's key-tile visiting order
// (pa::prefill_visit / pa::prefill_tile_of, the constexpr arithmetic the kernel calls),
// over causal and unmasked items: every query length, key length and item / wave
// position in the ranges below.  For each wave of each item it checks that
//   - steps 0 .. T visit every key tile 0 .. T exactly once;
//   - t_act is the highest tile any of the wave's rows can see (-1: none);
//   - k_first is the first step whose tile the wave computes (<= t_act);
//   - the tiles of steps 1 .. P hold only keys visible to every query row (keys before
//     the new tokens), and P is the number of such whole tiles (at most T).
// Exit status 0 = all passed.
#include <algorithm>
#include <cstdio>
#include <vector>

#include "pa_internal.h"

int main() {
    long checked = 0, failures = 0;
    auto fail = [&](const char* what, int qlen, int kvlen, int qbeg, int heads, int wave,
                    bool causal) {
        if (++failures <= 20)
            std::fprintf(stderr, "%s: qlen %d kvlen %d qbeg %d heads %d wave %d causal %d\n", what,
                         qlen, kvlen, qbeg, heads, wave, causal ? 1 : 0);
    };
    const int BN = pa::kPrefillBN;
    for (int causal_i = 0; causal_i < 2; ++causal_i) {
        const bool causal = causal_i == 1;
        for (int qlen = 1; qlen <= 300; qlen += (qlen < 70 ? 1 : 7)) {
            for (int kvlen = 0; kvlen <= 1100; kvlen += (kvlen < 200 ? 1 : 13)) {
                const int shift = kvlen - qlen;
                for (int heads : {1, 2, 4}) {
                    const int rows = pa::kPrefillBM / heads;
                    for (int qbeg = 0; qbeg < qlen; qbeg += rows) {
                        // the planner's key-tile count for the item's rows
                        const int r1 = std::min(qbeg + rows, qlen);
                        long last = -1;
                        for (int i = qbeg; i < r1; ++i)
                            last = std::max<long>(last, causal ? std::min(shift + i, kvlen - 1)
                                                               : kvlen - 1);
                        const int ktiles = last < 0 ? 0 : static_cast<int>(last / BN + 1);
                        for (int wave = 0; wave < 4; ++wave) {
                            const int wq0 = qbeg + 32 * (wave / heads);
                            const pa::PrefillVisit v =
                                pa::prefill_visit(ktiles, causal, qlen, kvlen, wq0);
                            ++checked;
                            if (v.T != ktiles - 1) fail("T", qlen, kvlen, qbeg, heads, wave, causal);
                            // every tile exactly once
                            std::vector<int> seen(std::max(ktiles, 0), 0);
                            bool ok = true;
                            for (int k = 0; k <= v.T; ++k) {
                                const int t = pa::prefill_tile_of(v, k);
                                if (t < 0 || t > v.T || seen[t]++) ok = false;
                            }
                            if (!ok) fail("tiles not a permutation", qlen, kvlen, qbeg, heads, wave, causal);
                            // t_act: the highest tile a row of the wave sees
                            int want = -1;
                            for (int i = wq0; i < std::min(wq0 + 32, qlen); ++i) {
                                const int lk = causal ? std::min(shift + i, kvlen - 1) : kvlen - 1;
                                if (lk >= 0) want = std::max(want, lk / BN);
                            }
                            if (v.t_act != want) fail("t_act", qlen, kvlen, qbeg, heads, wave, causal);
                            // k_first: the first step with a computed tile
                            if (v.t_act >= 0) {
                                int first = -1;
                                for (int k = 0; k <= v.T && first < 0; ++k)
                                    if (pa::prefill_tile_of(v, k) <= v.t_act) first = k;
                                if (v.k_first != first)
                                    fail("k_first", qlen, kvlen, qbeg, heads, wave, causal);
                            }
                            // steps 1 .. P: prefix-only tiles, and all of them
                            if (!causal && v.P != 0) fail("P without mask", qlen, kvlen, qbeg, heads, wave, causal);
                            if (causal) {
                                const int whole = shift > 0 ? std::min(shift / BN, v.T) : 0;
                                if (v.P != std::max(whole, 0)) fail("P", qlen, kvlen, qbeg, heads, wave, causal);
                                for (int k = 1; k <= v.P; ++k)
                                    if ((pa::prefill_tile_of(v, k) + 1) * BN > shift)
                                        fail("prefix tile", qlen, kvlen, qbeg, heads, wave, causal);
                            }
                        }
                    }
                }
            }
        }
    }
    std::printf("prefill_visit_check: %ld waves checked, %ld failures\n", checked, failures);
    return failures == 0 ? 0 : 1;
}
