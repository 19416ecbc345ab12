"""Seeded synthetic inputs for attention workloads.

This module is the only thing shared by the GPU path's tests/benchmark and the
CPU oracle.  It draws random numbers and converts storage formats; it holds
none of the attention arithmetic.

Recipe (every workload):

* ``rng = numpy.random.Generator(numpy.random.PCG64(seed))``;
* Q, then K, then V are drawn as float64 ``standard_normal`` of shapes
  ``[B, H, Lq, d]``, ``[B, H, Lk, d]``, ``[B, H, Lk, d]`` (iid N(0, 1), the
  distribution the German translation's footnote 4 assumes for q and k), each
  multiplied by ``scale``;
* each is rounded to float32 (round to nearest even) and, for bf16 workloads,
  from float32 to bf16 (round to nearest even); bf16 is kept as uint16 bits;
* when the workload has padding, ``key_lens = rng.integers(lo, hi,
  endpoint=True, size=B)`` (int32) is drawn after V;
* for gradients, the upstream gradient dL/dO comes from a generator of its
  own, ``PCG64(SeedSequence([seed, 1]))``, iid N(0, 1) of shape
  ``[B, H, Lq, d]`` (not scaled), rounded the same way.

Large tensors are drawn in chunks from the same generator, which yields the
same stream as one draw (checked by the test suite).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

_CHUNK = 1 << 24  # elements per draw when filling large tensors


@dataclass(frozen=True)
class Workload:
    """One synthetic attention problem: shapes, dtype, masking and seed."""
    name: str
    B: int
    H: int
    Lq: int
    Lk: int
    d: int
    dtype: str            # "fp32" or "bf16"
    causal: bool = False
    key_lens: tuple | None = None   # (lo, hi) inclusive range for uniform lengths
    scale: float = 1.0
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def flops(self) -> float:
        """Headline flop count 4*B*H*Lq*Lk*d, halved for causal."""
        f = 4.0 * self.B * self.H * self.Lq * self.Lk * self.d
        return f / 2 if self.causal else f


# The five workloads.  Shapes come from the pages: the toy model's
# d_model 6 / 2 heads / source length 8 (cookipedia article, "トイモデル");
# the base model's 8 heads of d_k = 64 (cookipedia, "原論文でのエンコーダ";
# formula page, "起源"); GPT-3's 96 heads of d_k = 128 (formula page, "起源").
# Batch sizes, lengths and the padding range are not on the pages.
WORKLOADS = {
    "toy_f32": Workload("toy_f32", 1, 2, 8, 8, 3, "fp32", seed=0,
                        note="toy non-causal self-attention, fp32"),
    "encoder_d64": Workload("encoder_d64", 64, 8, 128, 128, 64, "bf16", seed=1,
                            note="base-model encoder self-attention"),
    "decoder_causal_d64": Workload("decoder_causal_d64", 32, 8, 256, 256, 64, "bf16",
                                   causal=True, seed=2,
                                   note="base-model decoder masked self-attention"),
    "cross_padded_d64": Workload("cross_padded_d64", 32, 8, 256, 512, 64, "bf16",
                                 key_lens=(64, 512), seed=3,
                                 note="cross-attention with per-batch key lengths"),
    "large_causal_d128": Workload("large_causal_d128", 4, 96, 4096, 4096, 128, "bf16",
                                  causal=True, scale=0.5, seed=4,
                                  note="large-model causal self-attention"),
}
# Decode-shaped workloads (one new query per step against the cached keys of
# every earlier position; cookipedia article, "全体").  Shapes: GPT-3's heads
# and its 2048-token context (formula page, "起源" and "応用"); the base
# model's 8 heads of 64 for a single long sequence.  Batch sizes and the
# length range are not on the pages.
DECODE_WORKLOADS = {
    "decode_d128": Workload("decode_d128", 16, 96, 1, 2048, 128, "bf16",
                            key_lens=(1024, 2048), seed=5,
                            note="decode step, 96 heads of 128, context 1024..2048"),
    "decode_d64_single": Workload("decode_d64_single", 1, 8, 1, 4096, 64, "bf16", seed=6,
                                  note="decode step, one sequence, 8 heads of 64, context 4096"),
}
WORKLOADS.update(DECODE_WORKLOADS)

WORKLOAD_ORDER = ["toy_f32", "encoder_d64", "decoder_causal_d64",
                  "cross_padded_d64", "large_causal_d128"]


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite and infinite values stay below 2^32 after the rounding add
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u
    r >>= 16
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _draw(rng: np.random.Generator, shape, scale: float, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    for start in range(0, n, _CHUNK):
        stop = min(n, start + _CHUNK)
        x = rng.standard_normal(stop - start)
        if scale != 1.0:
            x *= scale
        x32 = x.astype(np.float32)
        out[start:stop] = f32_to_bf16_bits(x32) if dtype == "bf16" else x32
    return out.reshape(shape)


def generate(B: int, H: int, Lq: int, Lk: int, d: int, dtype: str, seed: int,
             scale: float = 1.0, key_lens: tuple | None = None):
    """Draw (q, k, v, key_lens) by the module recipe.

    Returns numpy arrays: float32, or uint16 bf16 bits when ``dtype == "bf16"``;
    ``key_lens`` is an int32 array of shape [B] or None.
    """
    if dtype not in ("fp32", "bf16"):
        raise ValueError(dtype)
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _draw(rng, (B, H, Lq, d), scale, dtype)
    k = _draw(rng, (B, H, Lk, d), scale, dtype)
    v = _draw(rng, (B, H, Lk, d), scale, dtype)
    kl = None
    if key_lens is not None:
        lo, hi = key_lens
        kl = rng.integers(lo, hi, endpoint=True, size=B).astype(np.int32)
    return q, k, v, kl


def generate_dout(B: int, H: int, Lq: int, d: int, dtype: str, seed: int) -> np.ndarray:
    """Upstream gradient dL/dO for the inputs of ``seed`` (module recipe)."""
    if dtype not in ("fp32", "bf16"):
        raise ValueError(dtype)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1])))
    return _draw(rng, (B, H, Lq, d), 1.0, dtype)


def generate_workload(w: Workload):
    """Inputs of a named workload (see :data:`WORKLOADS`)."""
    return generate(w.B, w.H, w.Lq, w.Lk, w.d, w.dtype, w.seed, w.scale, w.key_lens)


def as_float(x, dtype: str) -> np.ndarray:
    """float32 view of generated data (bf16 bits widened exactly)."""
    return bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)
