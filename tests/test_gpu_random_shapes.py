"""Seeded random shapes through every entry point, against the CPU oracle.

The hand-picked cases elsewhere cover the boundaries one at a time; this file
draws sizes, flags and key lengths at random (fixed seeds, so every run is
the same) to catch combinations nobody thought of: ragged query and key
tails together, causal with Lq != Lk and key lengths at once, key lengths
of 0, 1, the full length, or outside [0, Lk] (the library clamps them).
Sizes stay small enough for the fp64 oracle to answer in well under a
second per case.  Tolerances are those of the other parity tests.
"""
import numpy as np
import pytest

from gpu_util import announce, assert_close, oracle_ref, require_gpu, run_gpu
from test_gpu_backward import check_case
from test_gpu_decode import run_decode
from test_gpu_forward_ex import draw, oracle_ex, run_ex
from transformer_scaled_dot_sdpa_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _key_lens(rng, B, Lk):
    """None, or B lengths mixing the edge values with uniform draws."""
    if rng.random() < 0.4:
        return None
    pool = [0, 1, Lk, Lk + 5, -3]
    return [int(rng.choice(pool)) if rng.random() < 0.4 else int(rng.integers(1, Lk + 1))
            for _ in range(B)]


def _shape(rng, max_l):
    B = int(rng.integers(1, 4))
    H = int(rng.integers(1, 4))
    Lq = int(rng.integers(1, max_l + 1))
    Lk = int(rng.integers(1, max_l + 1))
    causal = bool(rng.random() < 0.5)
    return B, H, Lq, Lk, causal, _key_lens(rng, B, Lk)


@pytest.mark.parametrize("seed", range(24))
def test_random_forward_bf16(seed):
    rng = np.random.default_rng(5000 + seed)
    B, H, Lq, Lk, causal, kl = _shape(rng, 400)
    d = int(rng.choice([64, 128]))
    what = f"random fwd bf16 seed={seed}: B{B} H{H} Lq{Lq} Lk{Lk} d{d} causal={causal} key_lens={kl}"
    announce(what)
    q, k, v, _ = inputs.generate(B, H, Lq, Lk, d, "bf16", 5000 + seed)
    o, l = run_gpu(q, k, v, "bf16", causal, kl)
    ro, rl = oracle_ref(q, k, v, "bf16", causal, kl)
    assert_close(o, l, ro, rl, "bf16", what)


@pytest.mark.parametrize("seed", range(12))
def test_random_forward_bf16_many_items(seed):
    """Enough query blocks (about 200 to 1100, i.e. up to four per CU) for the
    shape-dependent tiles and schedules: compute-unit pairing, key-length
    ranking, the key split and the 8-wavefront tiles."""
    rng = np.random.default_rng(5500 + seed)
    d = int(rng.choice([64, 128]))
    Lq = int(rng.integers(64, 513))
    Lk = int(rng.integers(64, 641))
    causal = bool(rng.random() < 0.5)
    B = int(rng.integers(1, 9))
    target = int(rng.integers(200, 1101))
    H = max(1, round(target / (B * ((Lq + 127) // 128))))
    kl = _key_lens(rng, B, Lk)
    what = (f"random fwd bf16 (many items) seed={seed}: B{B} H{H} Lq{Lq} Lk{Lk} d{d} causal={causal} "
            f"key_lens={kl}")
    announce(what)
    q, k, v, _ = inputs.generate(B, H, Lq, Lk, d, "bf16", 5500 + seed)
    o, l = run_gpu(q, k, v, "bf16", causal, kl)
    ro, rl = oracle_ref(q, k, v, "bf16", causal, kl)
    assert_close(o, l, ro, rl, "bf16", what)


@pytest.mark.parametrize("seed", range(8))
def test_random_forward_f32(seed):
    rng = np.random.default_rng(6000 + seed)
    B, H, Lq, Lk, causal, kl = _shape(rng, 150)
    d = int(rng.integers(1, 257))
    what = f"random fwd fp32 seed={seed}: B{B} H{H} Lq{Lq} Lk{Lk} d{d} causal={causal} key_lens={kl}"
    announce(what)
    q, k, v, _ = inputs.generate(B, H, Lq, Lk, d, "fp32", 6000 + seed)
    o, l = run_gpu(q, k, v, "fp32", causal, kl)
    ro, rl = oracle_ref(q, k, v, "fp32", causal, kl)
    assert_close(o, l, ro, rl, "fp32", what)


@pytest.mark.parametrize("seed", range(12))
def test_random_backward_bf16(seed):
    rng = np.random.default_rng(7000 + seed)
    B, H, Lq, Lk, causal, kl = _shape(rng, 300)
    d = int(rng.choice([64, 128]))
    check_case(B, H, Lq, Lk, d, "bf16", causal, kl, 7000 + seed, f"random bf16 seed={seed} d{d}")


@pytest.mark.parametrize("seed", range(10))
def test_random_backward_bf16_many_items(seed):
    """About 200 to 1100 query (and key) blocks, i.e. up to four per CU:
    the backward's schedules for causal problems (one block per workgroup
    with compute-unit pairing, single blocks just past one round, long/short
    pairs beyond) and its whole-row result stores at scale."""
    rng = np.random.default_rng(7200 + seed)
    d = int(rng.choice([64, 128]))
    L = int(rng.integers(64, 513))
    causal = bool(rng.random() < 0.6)
    B = int(rng.integers(1, 9))
    target = int(rng.integers(200, 1101))
    H = max(1, round(target / (B * ((L + 127) // 128))))
    kl = _key_lens(rng, B, L)
    check_case(B, H, L, L, d, "bf16", causal, kl, 7200 + seed,
               f"random bf16 backward (many items) seed={seed} B{B} H{H} L{L} d{d} causal={causal}")


@pytest.mark.parametrize("seed", range(4))
def test_random_backward_f32(seed):
    rng = np.random.default_rng(7500 + seed)
    B, H, Lq, Lk, causal, kl = _shape(rng, 120)
    d = int(rng.integers(1, 257))
    check_case(B, H, Lq, Lk, d, "fp32", causal, kl, 7500 + seed, f"random fp32 seed={seed} d{d}")


@pytest.mark.parametrize("seed", range(8))
def test_random_decode(seed):
    rng = np.random.default_rng(8000 + seed)
    B = int(rng.integers(1, 5))
    H = int(rng.integers(1, 5))
    Lq = int(rng.integers(1, 9))
    Lk = int(rng.integers(1, 3001))
    causal = bool(rng.random() < 0.2)
    kl = _key_lens(rng, B, Lk)
    d = int(rng.choice([64, 128]))
    what = f"random decode seed={seed}: B{B} H{H} Lq{Lq} Lk{Lk} d{d} causal={causal} key_lens={kl}"
    announce(what)
    q, k, v, _ = inputs.generate(B, H, Lq, Lk, d, "bf16", 8000 + seed)
    o, l, _ = run_decode(q, k, v, causal, kl)
    ro, rl = oracle_ref(q, k, v, "bf16", causal, kl)
    assert_close(o, l, ro, rl, "bf16", what)


@pytest.mark.parametrize("seed", range(8))
def test_random_forward_ex(seed):
    rng = np.random.default_rng(9000 + seed)
    B, H, Lq, Lk, causal, kl = _shape(rng, 300)
    dk = int(rng.choice([64, 128]))
    dv = int(rng.choice([64, 128]))
    layout = str(rng.choice(["contiguous", "interleaved"]))
    scale = None if rng.random() < 0.5 else float(rng.uniform(0.02, 0.3))
    # an additive fp32 bias over [Lq, Lk], shared by every (b, h)
    mask = rng.standard_normal((Lq, Lk)).astype(np.float32) if rng.random() < 0.4 else None
    what = (f"random forward_ex seed={seed}: B{B} H{H} Lq{Lq} Lk{Lk} dk{dk} dv{dv} {layout} "
            f"causal={causal} key_lens={kl} scale={scale} mask={mask is not None}")
    announce(what)
    base = 9000 + 10 * seed
    q = draw(B, H, Lq, dk, "bf16", base)
    k = draw(B, H, Lk, dk, "bf16", base + 1)
    v = draw(B, H, Lk, dv, "bf16", base + 2)
    o, l = run_ex(q, k, v, "bf16", layout, causal=causal, key_lens=kl, scale=scale, mask=mask)
    ro, rl = oracle_ex(q, k, v, "bf16", causal=causal, key_lens=kl, scale=scale, mask=mask)
    assert_close(o, l, ro, rl, "bf16", what)
