// Tile / occupancy selection for the bf16 forward kernel.
//
// Head sizes 64 (the base model's 8 heads of 64: cookipedia article
// "Attention Is All You Need", section "原論文でのエンコーダ") and 128
// (GPT-3's heads, formula page "トランスフォーマーの注意機構", section 起源)
// are compiled.  The environment variable SDPA_FORCE_TILE may name one
// compiled configuration (e.g. "bf16_d128_bc64_w4") to override the choice,
// for tuning runs.
#include <stdlib.h>
#include <string.h>

#include "sdpa_internal.h"

namespace sdpa {

namespace {
// First entry per head size is the default.
const Bf16Tile kTiles[] = {
    {128, 64, 4, 0, "bf16_d128_bc64_w4"},
    {128, 64, 4, 1, "bf16_d128_pipe_w4"},
    {128, 64, 8, 2, "bf16_d128_pp_w8"},
    {128, 64, 8, 0, "bf16_d128_bc64_w8"},
    {128, 64, 4, 3, "bf16_d128_wide_w4"},
    {128, 64, 8, 4, "bf16_d128_mix_w8"},
    {64, 64, 4, 0, "bf16_d64_bc64_w4"},
    {64, 64, 4, 1, "bf16_d64_pipe_w4"},
    {64, 64, 8, 2, "bf16_d64_pp_w8"},
    {64, 128, 4, 0, "bf16_d64_bc128_w4"},
    {64, 64, 8, 0, "bf16_d64_bc64_w8"},
    {64, 64, 4, 3, "bf16_d64_wide_w4"},
    {64, 64, 8, 4, "bf16_d64_mix_w8"},
};
}  // namespace

bool select_bf16_tile(int d, int causal, long long bh, int Lq, int Lk, int num_cus,
                      Bf16Tile* out) {
    (void)causal; (void)bh; (void)Lq; (void)Lk; (void)num_cus;
    const char* force = getenv("SDPA_FORCE_TILE");
    if (force != nullptr && force[0] != '\0') {
        for (const Bf16Tile& t : kTiles)
            if (t.d == d && strcmp(force, t.name) == 0) {
                *out = t;
                return true;
            }
    }
    for (const Bf16Tile& t : kTiles)
        if (t.d == d) {
            *out = t;
            return true;
        }
    return false;
}

}  // namespace sdpa
