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
//                         per item.  d128: 1 workgroup per CU; wins with at
//                         most one item per CU and long key ranges (>= 32
//                         steps causal, >= 16 otherwise).  d64: 4 wavefronts
//                         per SIMD (128 registers), 2 workgroups per CU;
//                         wins with at most one item per CU and >= 16 steps,
//                         or causal with at most two and >= 32 steps.
//   bf16_d*_bc64_w8       8 wavefronts (256 rows) share each K/V tile:
//                         half the L2->LDS bytes per flop.  d128: 1
//                         workgroup per CU; d64: four wavefronts per SIMD,
//                         2 workgroups per CU.  Wins with no key lengths for
//                         2..4 items per CU (causal: above 2) with >= 16
//                         steps (d64: at most 64 steps, and >= 32 above 2
//                         items per CU), and at d64 from 4 items per CU on.
//   bf16_d*_bc64_w4_pairs per-batch key lengths, no causal mask: batches
//                         ranked by length, each workgroup runs the i-th
//                         longest and the i-th shortest item.  Wins when the
//                         items need between two and four rounds of slots.
//
// The thresholds come from timing every tile on 42 shapes on MI355X
// (interleaved batches, median of 3); the design notes list the table.  On
// all of them the choice is within 2% of the fastest tile.
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
    const long long steps = ((causal ? (Lq < Lk ? Lq : Lk) : Lk) + 63) / 64;
    const char* name = d == 128 ? "bf16_d128_bc64_w4" : "bf16_d64_bc64_w4";
    if (has_key_lens && !causal && items > 2 * cus && items <= 4 * cus) {
        name = d == 128 ? "bf16_d128_bc64_w4_pairs" : "bf16_d64_bc64_w4_pairs";
    } else if (!general && d == 128 && items <= cus && steps >= (causal ? 32 : 16)) {
        name = "bf16_d128_bc64_w4_ks2";
    } else if (!general && d == 64 && (causal ? items <= 2 * cus && steps >= 32 : items <= cus && steps >= 16)) {
        name = "bf16_d64_bc64_w4_ks2";
    } else if (!general && !has_key_lens &&
               (((causal ? items > 2 * cus : items >= 2 * cus) && items <= 4 * cus && steps >= 16 &&
                 (d == 128 || (steps <= 64 && (items <= 2 * cus || steps >= 32)))) ||
                (d == 64 && items >= 4 * cus))) {
        name = d == 128 ? "bf16_d128_bc64_w8" : "bf16_d64_bc64_w8";
    }
    *out = *tile_named(d, name);
    return true;
}

}  // namespace sdpa
