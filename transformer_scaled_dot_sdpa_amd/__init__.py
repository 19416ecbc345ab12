"""MI355X-native scaled dot-product attention forward (HIP, gfx950).

``forward(q, k, v, causal=False, key_lens=None)`` computes
softmax(q k^T / sqrt(d_k)) v for every (batch, head) slice in the library's
HIP kernels (see ``include/sdpa.h`` for the C ABI).  The shared library is
loaded on first use; ``python -m transformer_scaled_dot_sdpa_amd.build``
builds it.  ``backward(q, k, v, out, lse, dout, ...)`` returns the gradients
(dq, dk, dv) of that forward, also in HIP kernels; ``decode(q, k, v, ...)``
is the forward for 1..8 query rows, split over key chunks; ``forward_ex``
takes strided (e.g. head-interleaved) views, d_v != d_k, a scale and an
additive mask.  ``attention(q, k, v, causal=False, key_lens=None)`` is the
forward as a differentiable torch op whose backward runs ``backward``.
"""
from .autograd import attention  # noqa: F401
from .binding import (SdpaError, backward, decode, decode_workspace_size, forward,  # noqa: F401
                      forward_ex, kernel_name, load_library, LIB_PATH, EXPORTED)
