"""Every bf16 tile configuration the library compiles, not only the ones the
selector picks for the workloads, against the CPU oracle through the C ABI.

A tile is forced by name through ``sdpa_forward_ex``'s ``tile`` field.  The
cases cover one key tile and many (odd and even counts, so that one group of
a key-split tile can have nothing to do in the last step, or in every step),
ragged tails, key lengths (empty, short, full, tied; odd item counts for the
tiles that pair items by key length), causal with Lq > Lk and
Lq < Lk, query blocks that end inside a tile, and scores that grow along the
keys far enough to make the kernels redo a workgroup with a running maximum.
"""
import numpy as np
import pytest

from gpu_util import announce, assert_close, generate, oracle_ref, require_gpu, to_device
from transformer_scaled_dot_sdpa_amd import inputs

pytestmark = pytest.mark.gpu

TILES = {
    128: ["bf16_d128_bc64_w4", "bf16_d128_bc64_w4_pairs", "bf16_d128_bc64_w4_ks2", "bf16_d128_bc64_w8"],
    64: ["bf16_d64_bc64_w4", "bf16_d64_bc64_w4_pairs", "bf16_d64_bc64_w4_ks2", "bf16_d64_bc64_w8"],
}
TILE_PARAMS = [(d, t) for d, ts in TILES.items() for t in ts]

CASES = [
    # B, H, Lq, Lk, causal, key_lens
    (1, 1, 7, 7, False, None),
    (2, 3, 300, 300, True, None),
    (2, 2, 129, 200, False, [77, 200]),
    (3, 2, 64, 64, False, [0, 1, 64]),
    (1, 2, 300, 130, True, None),
    (1, 2, 100, 333, True, None),
    (2, 1, 520, 520, True, [300, 520]),
    (2, 2, 256, 512, False, [64, 450]),
    (4, 2, 128, 192, False, None),
    (1, 3, 200, 64, True, None),
    # key lengths with ties, an empty batch and an odd number of items (the
    # pairs tiles rank batches by length and run the middle item alone)
    (5, 3, 200, 300, False, [300, 17, 300, 0, 150]),
    (3, 1, 100, 200, False, [5, 200, 100]),
    # causal, an even number of query blocks per slice and between one and
    # two blocks per compute unit: the default tile's compute-unit pairing
    # renumbers the units
    (2, 80, 256, 256, True, None),
    # key lengths, no causal mask, between one and two blocks per compute
    # unit, 5 key tiles: the default tile orders items by length rank
    # interleaved from both ends and pairs them per compute unit
    (8, 40, 100, 300, False, [300, 5, 0, 150, 299, 64, 1, 200]),
    # the same two schedules with an odd number of items (the middle item of
    # the length order, and XCD ranges that start at an odd unit and keep
    # the plain order)
    (3, 91, 100, 320, False, [320, 7, 200]),
    (1, 135, 256, 256, True, None),
    # causal, a few more items than resident workgroups: single items
    # rather than long/short pairs (pairs would leave slots idle), once
    # with up to 1.6 slots' worth of items and once with short items whose
    # pairs would end in a round under 60% full
    (1, 129, 512, 512, True, None),
    (2, 300, 256, 256, True, None),
    # causal long/short pairs with an odd number of query blocks per slice
    # (units of two items then span two slices)
    (2, 150, 300, 300, True, None),
]


def run_tile(q, k, v, causal, key_lens, tile):
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    kl = torch.from_numpy(np.asarray(key_lens, dtype=np.int32)).cuda() if key_lens is not None else None
    out, lse = sdpa.forward_ex(qd, kd, vd, causal=causal, key_lens=kl, tile=tile)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("d,tile", TILE_PARAMS, ids=[t for _, t in TILE_PARAMS])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}q{}k{}c{}L{}".format(*c[:5], c[5]))
def test_tile_matches_oracle(d, tile, case):
    require_gpu()
    B, H, Lq, Lk, causal, kl = case
    seed = 500 + d + Lq + 3 * Lk
    announce(f"tile {tile}: B{B} H{H} Lq{Lq} Lk{Lk} causal={causal} key_lens={kl} seed={seed}")
    q, k, v, _ = generate(B, H, Lq, Lk, d, "bf16", seed)
    o, l = run_tile(q, k, v, causal, kl, tile)
    ro, rl = oracle_ref(q, k, v, "bf16", causal, kl)
    assert_close(o, l, ro, rl, "bf16", f"{tile} {case}")
    if kl is not None:
        for b, n in enumerate(kl):
            if n <= 0:
                assert np.all(o[b] == 0) and np.all(np.isneginf(l[b]))


@pytest.mark.parametrize("d,tile", TILE_PARAMS, ids=[t for _, t in TILE_PARAMS])
@pytest.mark.parametrize("causal", [False, True])
def test_tile_scores_growing_along_keys(d, tile, causal):
    """Batch 0: scores rise with the key index far past the first tile's
    maximum; batch 1: random rows in the same launch."""
    require_gpu()
    B, H, L = 2, 2, 512
    q, k, v, _ = generate(B, H, L, L, d, "bf16", 31 + d)
    qf = np.zeros((H, L, d), np.float32)
    qf[:, :, 0] = 8.0
    kf = np.zeros((H, L, d), np.float32)
    kf[:, :, 0] = (0.25 if d == 128 else 0.125) * np.arange(L)[None, :]
    q[0] = inputs.f32_to_bf16_bits(qf)
    k[0] = inputs.f32_to_bf16_bits(kf)
    announce(f"tile {tile}: growing scores causal={causal}")
    o, l = run_tile(q, k, v, causal, None, tile)
    ro, rl = oracle_ref(q, k, v, "bf16", causal)
    assert_close(o, l, ro, rl, "bf16", f"{tile} growing causal={causal}")


@pytest.mark.parametrize("d,tile", TILE_PARAMS, ids=[t for _, t in TILE_PARAMS])
def test_tile_bitwise_deterministic(d, tile):
    """Two runs of one tile give the same bits (no atomics, fixed orders)."""
    require_gpu()
    q, k, v, _ = generate(2, 3, 333, 400, d, "bf16", 77 + d)
    announce(f"tile {tile}: determinism")
    o1, l1 = run_tile(q, k, v, True, [250, 400], tile)
    o2, l2 = run_tile(q, k, v, True, [250, 400], tile)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_tile_names_and_refusals():
    """Unknown names and non-default tiles asked for a mask or d_v != d_k are
    refused with NOT_SUPPORTED; the selector's names are compiled tiles."""
    require_gpu()
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    from transformer_scaled_dot_sdpa_amd.binding import NOT_SUPPORTED, SdpaError
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    v128 = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    mask = torch.zeros((64, 64), dtype=torch.float32, device="cuda")
    for bad in ("bf16_d64_nope", "bf16_d128_bc64_w4", "bf16_d64_bc128_w4"):
        with pytest.raises(SdpaError) as e:
            sdpa.forward_ex(q, q, q, tile=bad)
        assert e.value.status == NOT_SUPPORTED
    with pytest.raises(SdpaError) as e:
        sdpa.forward_ex(q, q, q, mask=mask, tile="bf16_d64_bc64_w8")
    assert e.value.status == NOT_SUPPORTED
    with pytest.raises(SdpaError) as e:
        sdpa.forward_ex(q, q, v128, tile="bf16_d64_bc64_w8")
    assert e.value.status == NOT_SUPPORTED
    sdpa.forward_ex(q, q, q, mask=mask, tile="bf16_d64_bc64_w4")
    sdpa.forward_ex(q, q, v128, tile="bf16_d64_bc64_w4")
    sdpa.forward_ex(q, q, v128, mask=mask, tile="bf16_d64_bc64_w4_pairs")
    torch.cuda.synchronize()
    for (B, H, Lq, Lk, d, causal) in [(4, 96, 4096, 4096, 128, True), (64, 8, 128, 128, 64, False),
                                      (32, 8, 256, 256, 64, True), (32, 8, 256, 512, 64, False),
                                      (1, 8, 1, 4096, 64, False)]:
        qq = torch.empty((B, H, Lq, d), dtype=torch.bfloat16, device="meta")
        kk = torch.empty((B, H, Lk, d), dtype=torch.bfloat16, device="meta")
        name = sdpa.binding.sdpa_kernel_name(sdpa.binding.handle_for(1, 0), B, H, Lq, Lk, d, causal, False)
        assert name in TILES[d], name


# One shape per rule of the tile selector (B, H, Lq, Lk, d_k, causal, key
# lengths given) and the tile it picks on a 256-CU MI355X.
SELECTOR_CASES = [
    ((4, 96, 4096, 4096, 128, True, False), "bf16_d128_bc64_w4"),        # many items
    ((1, 8, 4096, 4096, 128, True, False), "bf16_d128_bc64_w4_ks2"),     # <= 1 item per CU, long keys
    ((2, 16, 1024, 1024, 128, False, False), "bf16_d128_bc64_w4_ks2"),
    ((4, 16, 512, 512, 128, True, False), "bf16_d128_bc64_w4"),          # 8 key tiles: too short to split
    ((2, 13, 2048, 2048, 128, True, False), "bf16_d128_bc64_w4_ks2"),    # causal, 1..2 items per CU, even blocks
    ((8, 2, 2066, 2066, 128, True, False), "bf16_d128_bc64_w4"),         # same, odd blocks per slice
    ((2, 40, 512, 512, 128, False, False), "bf16_d128_bc64_w8"),         # 1..2 items per CU, whole blocks
    ((32, 3, 302, 302, 128, False, False), "bf16_d128_bc64_w4"),         # same, but 256-row blocks waste rows
    ((1, 10, 8192, 8192, 128, True, False), "bf16_d128_bc64_w8"),        # 2.5 items per CU, long keys
    ((16, 2, 2671, 2671, 128, True, False), "bf16_d128_bc64_w4"),        # same range, odd 256-row blocks
    ((8, 8, 1024, 1024, 128, True, True), "bf16_d128_bc64_w4"),          # key lengths: no w8
    ((4, 32, 1024, 1024, 128, False, True), "bf16_d128_bc64_w4_pairs"),  # key lengths, > 2 items per CU
    ((8, 8, 512, 2048, 64, False, True), "bf16_d64_bc64_w4_ks2"),        # key lengths, <= 1 item per CU
    ((64, 8, 128, 128, 64, False, False), "bf16_d64_bc64_w4"),           # encoder workload
    ((32, 8, 256, 256, 64, True, False), "bf16_d64_bc64_w4"),            # decoder workload
    ((32, 8, 256, 512, 64, False, True), "bf16_d64_bc64_w4"),            # cross-attention workload
    ((1, 8, 8192, 8192, 64, True, False), "bf16_d64_bc64_w4_ks2"),       # causal, >= 32 key tiles
    ((8, 4, 1280, 1280, 64, True, False), "bf16_d64_bc64_w4_ks2"),       # causal, <= 2 items per CU, 20 tiles
    ((16, 4, 1536, 1536, 64, True, False), "bf16_d64_bc64_w8"),          # causal, 3 items per CU
    ((8, 8, 2048, 2048, 64, True, False), "bf16_d64_bc64_w8"),           # same at 32 key tiles, even blocks
    ((8, 12, 1271, 1271, 64, True, False), "bf16_d64_bc64_w4"),          # 3.75 items per CU, 5 blocks: odd
    ((16, 2, 6600, 6600, 64, False, False), "bf16_d64_bc64_w4_ks2"),     # 6.5 items per CU, long keys
    ((64, 16, 512, 512, 64, False, False), "bf16_d64_bc64_w8"),          # many items, whole blocks
]


@pytest.mark.parametrize("case,expected", SELECTOR_CASES, ids=[e for _, e in SELECTOR_CASES])
def test_selector_choices(case, expected):
    require_gpu()
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the table is for a 256-CU device")
    B, H, Lq, Lk, d, causal, lens = case
    name = sdpa.binding.sdpa_kernel_name(sdpa.binding.handle_for(1, 0), B, H, Lq, Lk, d, causal, lens)
    assert name == expected, (case, name)
