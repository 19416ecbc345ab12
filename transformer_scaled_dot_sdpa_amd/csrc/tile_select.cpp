// Tile / occupancy selection for the bf16 forward kernel.
//
// Head sizes 64 (the base model's 8 heads of 64: cookipedia article
// "Attention Is All You Need", section "原論文でのエンコーダ") and 128
// (GPT-3's heads, formula page "トランスフォーマーの注意機構", section 起源)
// are compiled.  The choice depends on how the problem fills the GPU:
//
//   items  = B*H * ceil(Lq / 128)       query blocks of 128 rows
//   cus    = compute units; the default tile keeps 2 workgroups per CU
//   steps  = key tiles of 64 in a row's longest range (Lk; for causal,
//            min(Lq, Lk))
//   whole  = the 256-row blocks of the 8-wavefront tile cover no more rows
//            than the 128-row blocks (B*H*ceil(Lq/256) * 2 == items)
//
//   bf16_d*_bc64_w4       default: 4 wavefronts (128 rows) per workgroup,
//                         2 per CU; the only tile with d_v != d_k and masks.
//                         Between one and two rounds of slots it runs one
//                         item per workgroup, renumbered so that the two
//                         workgroups of a CU take a long and a short item
//                         (cu_pair_unit), which balances causal blocks and
//                         ranked key lengths alike.
//   bf16_d*_bc64_w4_ks2   two groups of 4 wavefronts take alternate key
//                         tiles of the same 128 rows: half the tile steps
//                         per item (d128: 1 workgroup per CU; d64: 4
//                         wavefronts per SIMD, 2 workgroups per CU).  Wins
//                         with at most one item per CU and long enough key
//                         ranges (d128: >= 10 steps causal, >= 16 otherwise;
//                         d64: >= 9 causal, >= 12 otherwise, >= 16 with key
//                         lengths), causal with up to two items per CU from
//                         32 steps (d128, an even number of query blocks
//                         per slice) or 20 steps (d64), and at d64 also with
//                         more items: causal from 32 steps, non-causal from
//                         24 steps up to 6.5 items per CU.
//   bf16_d*_bc64_w8       8 wavefronts (256 rows) share each K/V tile: half
//                         the L2->LDS bytes per flop (d128: 1 workgroup per
//                         CU; d64: 4 wavefronts per SIMD, 2 workgroups per
//                         CU).  Only without key lengths and with whole
//                         256-row blocks where rows would be wasted, it wins
//                         at d128 non-causal with 1..2 items per CU, at d128
//                         causal with 2.4..4 items per CU, >= 30 steps and an
//                         even number of 256-row blocks per slice, at
//                         d64 causal with 3..4.2 items per CU (one or an even
//                         number of 256-row blocks per slice; ahead of the
//                         key split's 32-step rule), and at d64
//                         non-causal from 2 items per CU (where the key split
//                         does not).
//   bf16_d*_bc64_w4_pairs per-batch key lengths, no causal mask: batches
//                         ranked by length, each workgroup runs the i-th
//                         longest and the i-th shortest item.  Wins with more
//                         than 2 items per CU and >= 16 steps.
//
// The thresholds come from timing every tile on MI355X (interleaved batches,
// median of 3) on 43 chosen shapes, 320 shapes drawn at random and a grid of
// causal shapes around the key-split boundaries; the design notes list the
// tables and the check on further random shapes that none of the
// thresholds was fitted to.
#include <string.h>

#include "sdpa_internal.h"

namespace sdpa {

namespace {
// Every compiled configuration; the first entry per head size is the default,
// the only one that also takes d_v != d_k and an additive mask.
const Bf16Tile kTiles[] = {
    {128, 64, 4, 1, 0, "bf16_d128_bc64_w4"},
    {128, 64, 4, 1, 1, "bf16_d128_bc64_w4_pairs"},
    {128, 64, 4, 2, 0, "bf16_d128_bc64_w4_ks2"},
    {128, 64, 8, 1, 0, "bf16_d128_bc64_w8"},
    {64, 64, 4, 1, 0, "bf16_d64_bc64_w4"},
    {64, 64, 4, 1, 1, "bf16_d64_bc64_w4_pairs"},
    {64, 64, 4, 2, 0, "bf16_d64_bc64_w4_ks2"},
    {64, 64, 8, 1, 0, "bf16_d64_bc64_w8"},
};

const Bf16Tile* tile_named(int d, const char* name) {
    for (const Bf16Tile& t : kTiles)
        if (t.d == d && strcmp(name, t.name) == 0) return &t;
    return nullptr;
}
}  // namespace

bool find_bf16_tile(int d, const char* name, Bf16Tile* out) {
    if (name == nullptr) return false;
    const Bf16Tile* t = tile_named(d, name);
    if (t == nullptr) return false;
    *out = *t;
    return true;
}

bool select_bf16_tile(int d, int causal, int has_key_lens, long long bh, int Lq, int Lk, int num_cus,
                      bool general, Bf16Tile* out) {
    if (d != 64 && d != 128) return false;
    const long long cus = num_cus > 0 ? num_cus : 256;
    const long long items = bh * ((Lq + 127) / 128);
    const bool whole = 2 * (bh * ((Lq + 255) / 256)) == items;
    const long long steps = ((causal ? (Lq < Lk ? Lq : Lk) : Lk) + 63) / 64;
    const bool lens = has_key_lens != 0;
    enum { W4, PAIRS, KS2, W8 } t = W4;
    if (lens && !causal) {
        if (items > 2 * cus && steps >= 16) t = PAIRS;
        else if (items <= cus && steps >= 16) t = KS2;
    } else if (d == 128) {
        if (items <= cus && steps >= (causal ? 10 : 16)) t = KS2;
        // up to two items per CU the split's single workgroup per CU runs
        // long/short pairs, balanced only when a slice has an even number
        // of query blocks (pairs do not then straddle two slices)
        else if (causal && items <= 2 * cus && steps >= 32 && ((Lq + 127) / 128) % 2 == 0) t = KS2;
        else if (!lens && whole && !causal && items > cus && items <= 2 * cus) t = W8;
        // causal 256-row blocks pair up long/short within a slice only when
        // a slice has an even number of them (measured: 10 of 10 such shapes
        // faster with w8, 3 of 4 odd ones slower)
        else if (!lens && causal && 5 * items >= 12 * cus && items <= 4 * cus && steps >= 30 &&
                 ((Lq + 255) / 256) % 2 == 0)
            t = W8;
    } else if (causal) {
        // w8 needs one or an even number of 256-row blocks per slice (with an
        // odd count above one the pairs straddle slices, as at d128: 4 of 5
        // such shapes slower with w8); where it applies it also beats the
        // key split from 32 steps (4 of 4 shapes measured)
        const bool w8 = !lens && whole && items >= 3 * cus && 5 * items <= 21 * cus &&
                        (((Lq + 255) / 256) % 2 == 0 || Lq <= 256);
        if ((items <= cus && steps >= 9) || (items <= 2 * cus && steps >= 20)) t = KS2;
        else if (w8) t = W8;
        else if (steps >= 32) t = KS2;
    } else {
        if ((items <= cus && steps >= 12) || (steps >= 24 && 2 * items <= 13 * cus)) t = KS2;
        else if (!lens && whole && items > 2 * cus) t = W8;
    }
    // d_v != d_k and additive masks run in the default geometry only
    if (general && t != PAIRS) t = W4;
    static const char* const kNames[2][4] = {
        {"bf16_d64_bc64_w4", "bf16_d64_bc64_w4_pairs", "bf16_d64_bc64_w4_ks2", "bf16_d64_bc64_w8"},
        {"bf16_d128_bc64_w4", "bf16_d128_bc64_w4_pairs", "bf16_d128_bc64_w4_ks2", "bf16_d128_bc64_w8"}};
    *out = *tile_named(d, kNames[d == 128][t]);
    return true;
}

}  // namespace sdpa
