"""``attention(q, k, v, causal=False, key_lens=None)``: the forward as a
differentiable PyTorch op.

The forward keeps its log-sum-exp per row; the backward hands it, the
output and the incoming gradient to :func:`~.binding.backward`, which
recomputes the weights from them.  Both directions run in the library's
HIP kernels (nothing here computes); this module only connects them to
torch's autograd.  Inputs are contiguous [B, H, L, d_k] GPU tensors as for
:func:`~.binding.forward`; ``key_lens`` is not differentiable.
"""
from __future__ import annotations

from . import binding


def _function():
    import torch

    class SdpaFunction(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, causal, key_lens):
            out, lse = binding.forward(q, k, v, causal=causal, key_lens=key_lens)
            ctx.causal = causal
            ctx.save_for_backward(q, k, v, out, lse, key_lens)
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, out, lse, key_lens = ctx.saved_tensors
            dq, dk, dv = binding.backward(q, k, v, out, lse, dout.contiguous(), causal=ctx.causal,
                                          key_lens=key_lens)
            return dq, dk, dv, None, None

    return SdpaFunction


_FN = None


def attention(q, k, v, causal: bool = False, key_lens=None):
    """softmax(q k^T / sqrt(d_k)) v with gradients for q, k and v."""
    global _FN
    if _FN is None:
        _FN = _function()
    return _FN.apply(q, k, v, bool(causal), key_lens)
