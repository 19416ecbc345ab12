"""MI355X-native scaled dot-product attention forward (HIP, gfx950).

``forward(q, k, v, causal=False, key_lens=None)`` computes
softmax(q k^T / sqrt(d_k)) v for every (batch, head) slice in the library's
HIP kernels (see ``include/sdpa.h`` for the C ABI).  The shared library is
loaded on first use; ``python -m transformer_scaled_dot_sdpa_amd.build``
builds it.  ``backward(q, k, v, out, lse, dout, ...)`` returns the gradients
(dq, dk, dv) of that forward, also in HIP kernels.
"""
from .binding import (SdpaError, backward, forward, kernel_name, load_library,  # noqa: F401
                      LIB_PATH, EXPORTED)
