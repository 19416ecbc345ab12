"""Host logic of the seeded input generators (CPU)."""
import numpy as np

from transformer_scaled_dot_sdpa_amd import inputs


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 0.0, -0.0,
                  np.inf, -np.inf, 3.4e38], dtype=np.float32)
    b = inputs.f32_to_bf16_bits(f)
    back = inputs.bf16_bits_to_f32(b)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even (1.0)
    assert back[0] == 1.0 and back[1] == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even (1 + 2^-6)
    assert back[2] == np.float32(1.0 + 2**-6)
    assert back[3] == 1.0
    assert back[4] == -2.5 and back[5] == 0.0 and np.signbit(back[6])
    assert np.isposinf(back[7]) and np.isneginf(back[8])
    assert np.isinf(back[9])  # rounds past the largest bf16
    assert np.isnan(inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]


def test_bf16_rounding_is_nearest():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32)
    y = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(x))
    rel = np.abs(y - x) / np.abs(x)
    assert rel.max() <= 2.0**-8
    # y is the nearer of the two bf16 neighbours of x (truncation and the next one up)
    lo_bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    lo = inputs.bf16_bits_to_f32(lo_bits)
    hi = inputs.bf16_bits_to_f32(lo_bits + 1)
    d_lo, d_hi, d_y = np.abs(x - lo), np.abs(hi - x), np.abs(y - x)
    assert np.all(d_y <= np.minimum(d_lo, d_hi))
    # exact widening round trip
    assert np.array_equal(inputs.f32_to_bf16_bits(y), inputs.f32_to_bf16_bits(x))


def test_chunked_draw_equals_single_draw(monkeypatch):
    a = inputs.generate(2, 3, 40, 50, 16, "bf16", seed=7)
    monkeypatch.setattr(inputs, "_CHUNK", 1000)
    b = inputs.generate(2, 3, 40, 50, 16, "bf16", seed=7)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)
    rng = np.random.Generator(np.random.PCG64(7))
    q = rng.standard_normal((2, 3, 40, 16)).astype(np.float32)
    assert np.array_equal(a[0], inputs.f32_to_bf16_bits(q))


def test_generator_is_seeded_and_shaped():
    q, k, v, kl = inputs.generate(3, 2, 5, 9, 4, "fp32", seed=3, key_lens=(2, 9))
    assert q.shape == (3, 2, 5, 4) and k.shape == v.shape == (3, 2, 9, 4)
    assert q.dtype == np.float32 and kl.dtype == np.int32 and kl.shape == (3,)
    assert kl.min() >= 2 and kl.max() <= 9
    q2, *_ = inputs.generate(3, 2, 5, 9, 4, "fp32", seed=3, key_lens=(2, 9))
    assert np.array_equal(q, q2)
    q3, *_ = inputs.generate(3, 2, 5, 9, 4, "fp32", seed=4)
    assert not np.array_equal(q, q3)


def test_workload_table():
    w = inputs.WORKLOADS
    assert [w[n].seed for n in inputs.WORKLOAD_ORDER] == [0, 1, 2, 3, 4]
    big = w["large_causal_d128"]
    assert (big.B, big.H, big.Lq, big.d, big.causal, big.scale) == (4, 96, 4096, 128, True, 0.5)
    assert abs(big.flops - 4 * 4 * 96 * 4096 * 4096 * 128 / 2) < 1
    assert w["cross_padded_d64"].key_lens == (64, 512)
