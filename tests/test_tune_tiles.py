"""The tile tuner's random shapes (host logic only; the timing needs a GPU)."""
from transformer_scaled_dot_sdpa_amd.tune_tiles import SHAPES, random_shapes


def test_random_shapes_are_seeded_and_within_bounds():
    a = random_shapes(40, 7)
    assert a == random_shapes(40, 7)
    assert a != random_shapes(40, 8)
    assert len(a) == 40
    for (d, B, H, Lq, Lk, causal, kl) in a:
        assert d in (64, 128)
        assert B in (1, 2, 4, 8, 16, 32) and H >= 1
        assert 100 <= Lq <= 8192 and 1 <= Lk <= 8192
        if causal:
            assert Lk == Lq and kl is None
        if kl is not None:
            lo, hi = kl
            assert B > 1 and 1 <= lo <= hi == Lk
        work = 4.0 * B * H * Lq * Lk * d / (2 if causal else 1)
        assert work <= 2e12
        items = B * H * ((Lq + 127) // 128)
        # between 1/4 and 16 query blocks per compute unit, up to rounding
        # of B*H to a whole number
        assert items >= 1 and items <= 16 * 256 + 2 * ((Lq + 127) // 128) * B


def test_chosen_shapes_cover_both_head_sizes_and_forms():
    forms = {(d, causal, kl is not None) for (d, B, H, Lq, Lk, causal, kl) in SHAPES}
    for d in (64, 128):
        assert (d, True, False) in forms
        assert (d, False, False) in forms
        assert (d, False, True) in forms
