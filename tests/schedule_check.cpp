// Host-side check of the library's scheduling maps and tile selector, built
// and run by tests/test_host_schedule.py (no GPU needed).  Compiled with
// hipcc together with csrc/tile_select.cpp; the maps come from bf16_common.h,
// the same inline functions the kernels call.
//
// stdin: "maps" runs the exhaustive map checks; otherwise one query per line,
//   d causal has_key_lens bh Lq Lk num_cus general
// and the selected tile's name is printed per line.
#include <stdio.h>
#include <string.h>

#include <vector>

#include "sdpa_internal.h"
#include "bf16_common.h"

using sdpa::bf16k::causal_items_per_unit;
using sdpa::bf16k::cu_pair_renumber;
using sdpa::bf16k::item_block;
using sdpa::bf16k::unit_of_workgroup;

namespace {

long check_unit_map(int max_nwg) {
    long bad = 0;
    for (int nwg = 1; nwg <= max_nwg; ++nwg) {
        std::vector<char> seen(nwg, 0);
        for (int g = 0; g < nwg; ++g) {
            const int u = unit_of_workgroup(nwg, g);
            if (u < 0 || u >= nwg || seen[u]++) ++bad;
            // the workgroups of one XCD (same g mod 8) take consecutive units
            if (g >= 8 && unit_of_workgroup(nwg, g) != unit_of_workgroup(nwg, g - 8) + 1) ++bad;
        }
    }
    return bad;
}

long check_cu_pairs(int C, int max_nwg, long* active) {
    long bad = 0;
    for (int nwg = 1; nwg <= max_nwg; ++nwg) {
        std::vector<int> unit(nwg);
        std::vector<char> seen(nwg, 0);
        for (int g = 0; g < nwg; ++g) {
            const int u = cu_pair_renumber(nwg, g, C, unit_of_workgroup(nwg, g));
            unit[g] = u;
            if (u < 0 || u >= nwg || seen[u]++) ++bad;
        }
        // where the renumbering applies, the XCD's local workgroups k and k + C
        // (one compute unit) hold units lo + 2k and lo + 2k + 1
        const int per = nwg >> 3, rem = nwg & 7;
        for (int x = 0; x < 8 && x < nwg; ++x) {
            const int R = per + (x < rem ? 1 : 0);
            const int lo = x * per + (x < rem ? x : rem);
            if (R <= C || R > 2 * C || (lo & 1)) continue;
            ++*active;
            for (int k = 0; k < R - C; ++k) {
                const int g0 = 8 * k + x, g1 = 8 * (k + C) + x;
                if (unit[g0] != lo + 2 * k || unit[g1] != lo + 2 * k + 1) ++bad;
            }
        }
    }
    return bad;
}

template <bool CAUSAL>
long check_item_block() {
    long bad = 0;
    const int slices = 3;
    for (int nqb = 1; nqb <= 40; ++nqb) {
        std::vector<char> seen(slices * nqb, 0);
        for (int item = 0; item < slices * nqb; ++item) {
            int bh, qb;
            item_block<CAUSAL>(item, nqb, &bh, &qb);
            if (bh < 0 || bh >= slices || qb < 0 || qb >= nqb || seen[bh * nqb + qb]++) ++bad;
            if (bh != item / nqb) ++bad;
            // causal: items 2i and 2i + 1 of a slice take (qb + 1) key tiles
            // each, nqb + 1 together
            if (CAUSAL && (item % nqb) % 2 == 1) {
                int bh0, qb0;
                item_block<CAUSAL>(item - 1, nqb, &bh0, &qb0);
                if (bh0 != bh || (qb0 + 1) + (qb + 1) != nqb + 1) ++bad;
            }
        }
    }
    return bad;
}

long check_items_per_unit() {
    long bad = 0;
    // fits the resident slots: one item each
    bad += causal_items_per_unit(512, 512, 819, 32, 8) != 1;
    // up to the single-item limit: one item each
    bad += causal_items_per_unit(800, 512, 819, 32, 8) != 1;
    // beyond it, long items: pairs
    bad += causal_items_per_unit(12288, 512, 819, 64, 8) != 2;
    // short items whose pairs would end in a round at most 60% full: single
    // (1300 items -> 650 pairs -> 138 in the last of 512 slots)
    bad += causal_items_per_unit(1300, 512, 819, 4, 8) != 1;
    // the same with a full last round: pairs (2048 items -> 1024 pairs, 0 left over)
    bad += causal_items_per_unit(2048, 512, 819, 4, 8) != 2;
    // short_steps = 0 (the backward's rule): pairs past the single-item limit
    bad += causal_items_per_unit(1300, 512, 639, 4, 0) != 2;
    return bad;
}

}  // namespace

int main() {
    char line[256];
    while (fgets(line, sizeof line, stdin)) {
        if (strncmp(line, "maps", 4) == 0) {
            long active = 0;
            printf("unit_map %ld\n", check_unit_map(20000));
            const long c32 = check_cu_pairs(32, 8 * 2 * 32 + 64, &active);
            const long c38 = check_cu_pairs(38, 8 * 2 * 38 + 64, &active);
            printf("cu_pairs %ld active %ld\n", c32 + c38, active);
            printf("item_block_causal %ld\n", check_item_block<true>());
            printf("item_block_plain %ld\n", check_item_block<false>());
            printf("items_per_unit %ld\n", check_items_per_unit());
            continue;
        }
        int d, causal, lens, Lq, Lk, cus, general;
        long long bh;
        if (sscanf(line, "%d %d %d %lld %d %d %d %d", &d, &causal, &lens, &bh, &Lq, &Lk, &cus, &general) != 8)
            continue;
        sdpa::Bf16Tile t;
        if (!sdpa::select_bf16_tile(d, causal, lens, bh, Lq, Lk, cus, general != 0, &t)) {
            printf("none\n");
            continue;
        }
        printf("%s\n", t.name);
    }
    return 0;
}
