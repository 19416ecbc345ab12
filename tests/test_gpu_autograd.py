"""``attention`` (forward and backward joined through torch.autograd) against
the library's own forward and backward calls, through the C ABI.

The autograd op only connects the two entry points, whose results the
parity tests compare with the oracle; here its outputs and gradients must
equal theirs bit for bit (both run the same deterministic kernels).
"""
import numpy as np
import pytest

from gpu_util import announce, require_gpu, to_device
from transformer_scaled_dot_sdpa_amd import inputs

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, Lq, Lk, d, dtype, causal, key_lens
    (2, 3, 200, 200, 128, "bf16", True, None),
    (2, 2, 130, 300, 64, "bf16", False, [300, 77]),
    (1, 2, 9, 17, 5, "fp32", True, None),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}q{}k{}d{}{}c{}".format(*c[:7]))
def test_attention_autograd_matches_entry_points(case):
    require_gpu()
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    B, H, Lq, Lk, d, dtype, causal, kl = case
    seed = 1700 + Lq + d
    announce(f"autograd attention B{B} H{H} Lq{Lq} Lk{Lk} d{d} {dtype} causal={causal} seed={seed}")
    q, k, v, _ = inputs.generate(B, H, Lq, Lk, d, dtype, seed)
    dout = inputs.generate_dout(B, H, Lq, d, dtype, seed)
    qd, kd, vd, gd = (to_device(x, dtype) for x in (q, k, v, dout))
    klt = torch.from_numpy(np.asarray(kl, dtype=np.int32)).cuda() if kl is not None else None

    out_ref, lse_ref = sdpa.forward(qd, kd, vd, causal=causal, key_lens=klt)
    dq_ref, dk_ref, dv_ref = sdpa.backward(qd, kd, vd, out_ref, lse_ref, gd, causal=causal, key_lens=klt)

    qa, ka, va = (t.clone().requires_grad_(True) for t in (qd, kd, vd))
    out = sdpa.attention(qa, ka, va, causal=causal, key_lens=klt)
    # the incoming gradient as a transposed view: the op makes it contiguous
    gt = gd.transpose(2, 3).contiguous().transpose(2, 3)
    out.backward(gt)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), out_ref)
    assert torch.equal(qa.grad, dq_ref)
    assert torch.equal(ka.grad, dk_ref)
    assert torch.equal(va.grad, dv_ref)
