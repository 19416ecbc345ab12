"""Every bf16 tile configuration the library ships, not only the default one,
against the CPU oracle through the C ABI.

The tile is chosen by name with the SDPA_FORCE_TILE environment variable,
which the library reads on every call.  The cases cover several key tiles, a
ragged tail, key lengths (empty, short, full), causal with Lq > Lk and
Lq < Lk, query blocks that end inside a tile, and scores that grow along the
keys far enough to make the kernels redo a workgroup with a running maximum.
"""
import os

import numpy as np
import pytest

from gpu_util import announce, assert_close, generate, oracle_ref, require_gpu, run_gpu
from transformer_scaled_dot_sdpa_amd import inputs

pytestmark = pytest.mark.gpu

ALT_TILES = {
    128: ["bf16_d128_bc64_w8", "bf16_d128_pipe_w4", "bf16_d128_pp_w8", "bf16_d128_wide_w4",
          "bf16_d128_mix_w8"],
    64: ["bf16_d64_bc64_w8", "bf16_d64_bc128_w4", "bf16_d64_pipe_w4", "bf16_d64_pp_w8",
         "bf16_d64_wide_w4", "bf16_d64_mix_w8"],
}
TILE_PARAMS = [(d, t) for d, ts in ALT_TILES.items() for t in ts]

CASES = [
    # B, H, Lq, Lk, causal, key_lens
    (1, 1, 7, 7, False, None),
    (2, 3, 300, 300, True, None),
    (2, 2, 129, 200, False, [77, 200]),
    (3, 2, 64, 64, False, [0, 1, 64]),
    (1, 2, 300, 130, True, None),
    (1, 2, 100, 333, True, None),
    (2, 1, 520, 520, True, [300, 520]),
]


@pytest.fixture
def forced_tile(request):
    require_gpu()
    old = os.environ.get("SDPA_FORCE_TILE")
    os.environ["SDPA_FORCE_TILE"] = request.param
    yield request.param
    if old is None:
        os.environ.pop("SDPA_FORCE_TILE", None)
    else:
        os.environ["SDPA_FORCE_TILE"] = old


def _check_selected(d, tile):
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    q = torch.empty((1, 1, 8, d), dtype=torch.bfloat16, device="cuda")
    assert sdpa.kernel_name(q, q, False, False) == tile


@pytest.mark.parametrize("d,forced_tile", TILE_PARAMS, indirect=["forced_tile"],
                         ids=[t for _, t in TILE_PARAMS])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}q{}k{}c{}L{}".format(*c[:5], c[5]))
def test_tile_matches_oracle(d, forced_tile, case):
    _check_selected(d, forced_tile)
    B, H, Lq, Lk, causal, kl = case
    seed = 500 + d + Lq + 3 * Lk
    announce(f"tile {forced_tile}: B{B} H{H} Lq{Lq} Lk{Lk} causal={causal} key_lens={kl} seed={seed}")
    q, k, v, _ = generate(B, H, Lq, Lk, d, "bf16", seed)
    o, l = run_gpu(q, k, v, "bf16", causal, kl)
    ro, rl = oracle_ref(q, k, v, "bf16", causal, kl)
    assert_close(o, l, ro, rl, "bf16", f"{forced_tile} {case}")
    if kl is not None:
        for b, n in enumerate(kl):
            if n <= 0:
                assert np.all(o[b] == 0) and np.all(np.isneginf(l[b]))


@pytest.mark.parametrize("d,forced_tile", TILE_PARAMS, indirect=["forced_tile"],
                         ids=[t for _, t in TILE_PARAMS])
@pytest.mark.parametrize("causal", [False, True])
def test_tile_scores_growing_along_keys(d, forced_tile, causal):
    """Batch 0: scores rise with the key index far past the first tile's
    maximum; batch 1: random rows in the same launch."""
    _check_selected(d, forced_tile)
    B, H, L = 2, 2, 512
    q, k, v, _ = generate(B, H, L, L, d, "bf16", 31 + d)
    qf = np.zeros((H, L, d), np.float32)
    qf[:, :, 0] = 8.0
    kf = np.zeros((H, L, d), np.float32)
    kf[:, :, 0] = (0.25 if d == 128 else 0.125) * np.arange(L)[None, :]
    q[0] = inputs.f32_to_bf16_bits(qf)
    k[0] = inputs.f32_to_bf16_bits(kf)
    announce(f"tile {forced_tile}: growing scores causal={causal}")
    o, l = run_gpu(q, k, v, "bf16", causal)
    ro, rl = oracle_ref(q, k, v, "bf16", causal)
    assert_close(o, l, ro, rl, "bf16", f"{forced_tile} growing causal={causal}")
