"""Helpers for the GPU tests: upload seeded inputs, run the HIP path through
the C ABI binding, and compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from transformer_scaled_dot_sdpa_amd import inputs

# Tolerances fixed for this method: max-abs error of the output 1e-5 for
# fp32 inputs and 2e-2 for bf16 inputs (outputs of order 1), and 1e-3 for
# the log-sum-exp; rows with no valid key must give lse = -inf exactly.
TOL_OUT = {"fp32": 1e-5, "bf16": 2e-2}
TOL_LSE = 1e-3


def announce(msg: str) -> None:
    """Name the case on stderr before the GPU runs it."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def to_device(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to("cuda")


def run_gpu(q, k, v, dtype, causal=False, key_lens=None, lse=True):
    """Upload numpy inputs (fp32, or bf16 as uint16 bits), run, and return
    (out float32 numpy, lse float32 numpy or None)."""
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    qd, kd, vd = to_device(q, dtype), to_device(k, dtype), to_device(v, dtype)
    kl = torch.from_numpy(np.asarray(key_lens, dtype=np.int32)).to("cuda") if key_lens is not None else None
    out, l = sdpa.forward(qd, kd, vd, causal=causal, key_lens=kl, need_lse=lse)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    return o, (l.cpu().numpy() if l is not None else None)


def oracle_ref(q, k, v, dtype, causal=False, key_lens=None, tau=None):
    import oracle
    return oracle.sdpa(q, k, v, causal=causal, key_lens=key_lens, tau=tau, bf16=(dtype == "bf16"))


def assert_close(o_gpu, l_gpu, o_ref, l_ref, dtype, what=""):
    err = float(np.max(np.abs(o_gpu.astype(np.float64) - o_ref))) if o_ref.size else 0.0
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    assert err <= TOL_OUT[dtype], f"{what}: max |dO| = {err:.3g} > {TOL_OUT[dtype]}"
    if l_gpu is not None:
        fin = np.isfinite(l_ref)
        assert np.array_equal(np.isneginf(l_gpu), np.isneginf(l_ref)), f"{what}: -inf rows differ"
        assert np.all(np.isfinite(l_gpu[fin])), f"{what}: non-finite lse"
        lerr = float(np.max(np.abs(l_gpu[fin].astype(np.float64) - l_ref[fin]), initial=0.0))
        assert lerr <= TOL_LSE, f"{what}: max |dlse| = {lerr:.3g} > {TOL_LSE}"
    return err


def generate(B, H, Lq, Lk, d, dtype, seed, scale=1.0, key_lens=None):
    return inputs.generate(B, H, Lq, Lk, d, dtype, seed, scale=scale, key_lens=key_lens)
