"""sdpa_decode_noalloc (the decode entry point that allocates nothing; its
split partials live in the library's fixed per-GPU array) against
sdpa_decode with a caller workspace, through the C ABI: two calls in a row,
the second with a smaller input, must give the same out and lse as the
workspace entry point.  Sizes beyond the array are refused."""
import ctypes

import numpy as np
import pytest

from gpu_util import announce, assert_close, oracle_ref, require_gpu, to_device
from transformer_scaled_dot_sdpa_amd import inputs

pytestmark = pytest.mark.gpu


def run_both(B, H, Lq, Lk, d, causal, kl, seed):
    import torch
    from transformer_scaled_dot_sdpa_amd import binding as b
    q, k, v, _ = inputs.generate(B, H, Lq, Lk, d, "bf16", seed)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    kld = torch.from_numpy(np.asarray(kl, dtype=np.int32)).cuda() if kl is not None else None
    klp = kld.data_ptr() if kld is not None else None
    h = b.handle_for(b.DTYPE_BF16, 0)
    need = b.sdpa_decode_workspace_size(h, B, H, Lq, Lk, d)
    assert 0 < need <= b.DECODE_NOALLOC_SCRATCH_BYTES   # the split path, within the array
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    out_ws, out_na = torch.empty_like(qd), torch.full_like(qd, float("nan"))
    lse_ws = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    lse_na = torch.full_like(lse_ws, float("nan"))
    s = torch.cuda.current_stream().cuda_stream
    assert b.sdpa_decode(h, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out_ws.data_ptr(), lse_ws.data_ptr(),
                         B, H, Lq, Lk, d, int(causal), klp, ws.data_ptr(), need, s) == b.SUCCESS
    assert b.sdpa_decode_noalloc(h, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out_na.data_ptr(),
                                 lse_na.data_ptr(), B, H, Lq, Lk, d, int(causal), klp, s) == b.SUCCESS
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()
    return q, k, v, f(out_ws), f(lse_ws), f(out_na), f(lse_na)


@pytest.mark.parametrize("d", [64, 128])
def test_noalloc_matches_workspace_entry_point_twice(d):
    require_gpu()
    # first call: 2 x 4 slices, 3 rows, 3000 keys, key lengths; second call
    # smaller (1 slice, 1 row, 700 keys): the array keeps the first call's
    # partials, which the second must not pick up
    for i, (B, H, Lq, Lk, causal, kl) in enumerate([(2, 4, 3, 3000, False, [2999, 1500]),
                                                    (1, 1, 1, 700, False, None)]):
        announce(f"decode_noalloc call {i}: d{d} B{B} H{H} Lq{Lq} Lk{Lk} key_lens={kl}")
        q, k, v, ow, lw, on, ln = run_both(B, H, Lq, Lk, d, causal, kl, 5100 + 10 * d + i)
        assert np.array_equal(on, ow) and np.array_equal(ln, lw), "noalloc differs from sdpa_decode"
        ro, rl = oracle_ref(q, k, v, "bf16", causal, kl)
        assert_close(on, ln, ro, rl, "bf16", f"decode_noalloc call {i}")


def test_noalloc_refuses_sizes_beyond_its_array():
    require_gpu()
    import torch
    from transformer_scaled_dot_sdpa_amd import binding as b
    h = b.handle_for(b.DTYPE_BF16, 0)
    # 64 slices x 8 rows x 65536 keys at d = 128 split into far more partials than 16 MiB hold
    B, H, Lq, Lk, d = 8, 8, 8, 65536, 128
    assert b.sdpa_decode_workspace_size(h, B, H, Lq, Lk, d) > b.DECODE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.uint8, device="cuda")   # never read: refused before any launch
    p = x.data_ptr()
    st = b.sdpa_decode_noalloc(h, p, p + 0, p, p, None, B, H, Lq, Lk, d, 0, None,
                               torch.cuda.current_stream().cuda_stream)
    assert st == b.NOT_SUPPORTED
