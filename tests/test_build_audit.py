"""Build-time check of the forward kernels' memory instructions (CPU only:
hipcc cross-compiles gfx950 assembly without a GPU).

Every instance of the bf16 forward kernel may touch global memory only for
its Q fragments, the key length, the O rows and the lse value; all K/V tile
traffic and the key-split groups' exchange of (O, m, l) go through LDS.  A
generic pointer into LDS that the compiler fails to keep in the LDS address
space turns into global accesses at LDS addresses, which fault the GPU; the
audit in the build refuses such a library, and this test runs it.
"""
from transformer_scaled_dot_sdpa_amd import build


def test_forward_kernels_touch_global_memory_only_for_q_o_lse():
    assert build.audit_forward_isa() >= 40
