"""Library calls captured into a HIP graph (as a serving loop or the
benchmark's short-call timing does) and replayed: every replay must give
the eager result bit for bit.  Replays are separated by eager work of the
program's own (other library calls on other buffers) and synchronisations.
The calls record kernel launches only (no memset or allocation nodes)."""
import numpy as np
import pytest

from gpu_util import announce, require_gpu, to_device
from transformer_scaled_dot_sdpa_amd import inputs

pytestmark = pytest.mark.gpu


def _dev(x):
    return to_device(x, "bf16")


def _replay_and_check(torch, g, outputs, eager, other_work):
    for rep in range(3):
        for t in outputs:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        other_work()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, ref in zip(outputs, eager):
            assert torch.equal(t.view(torch.uint8), ref.view(torch.uint8)), f"replay {rep} differs"
        other_work()


def test_forward_and_backward_in_a_graph():
    require_gpu()
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    announce("graph: forward x3 and backward")
    sets = []
    for i, (B, H, Lq, Lk, d, causal) in enumerate([(2, 3, 200, 300, 64, False), (1, 4, 257, 257, 128, True),
                                                   (3, 2, 128, 128, 64, True)]):
        q, k, v, _ = inputs.generate(B, H, Lq, Lk, d, "bf16", 6000 + i)
        g = inputs.generate_dout(B, H, Lq, d, "bf16", 6000 + i)
        qd, kd, vd, gd = _dev(q), _dev(k), _dev(v), _dev(g)
        sets.append((qd, kd, vd, gd, causal, torch.empty_like(qd),
                     torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda"),
                     torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd),
                     torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")))
    kl = torch.tensor([150, 300], dtype=torch.int32, device="cuda")

    def calls():
        for j, (qd, kd, vd, gd, causal, out, lse, dq, dk, dv, delta) in enumerate(sets):
            lens = kl if j == 0 else None
            sdpa.forward(qd, kd, vd, causal=causal, key_lens=lens, out=out, lse=lse)
            sdpa.backward(qd, kd, vd, out, lse, gd, causal=causal, key_lens=lens, dq=dq, dk=dk, dv=dv, delta=delta)

    calls()
    torch.cuda.synchronize()
    outputs = [t for s in sets for t in s[5:]]
    eager = [t.clone() for t in outputs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    xq = torch.randn(1, 2, 64, 128, device="cuda").bfloat16()
    _replay_and_check(torch, graph, outputs, eager, lambda: sdpa.forward(xq, xq, xq, causal=True))


def test_decode_and_decode_noalloc_in_a_graph():
    require_gpu()
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    from transformer_scaled_dot_sdpa_amd import binding as b
    announce("graph: decode with a workspace and decode_noalloc (split over keys)")
    B, H, Lq, Lk, d = 1, 8, 2, 4096, 64
    q, k, v, _ = inputs.generate(B, H, Lq, Lk, d, "bf16", 6100)
    qd, kd, vd = _dev(q), _dev(k), _dev(v)
    need = sdpa.decode_workspace_size(qd, kd)
    assert 0 < need <= b.DECODE_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out1, out2 = torch.empty_like(qd), torch.empty_like(qd)
    lse1 = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    lse2 = torch.empty_like(lse1)
    h = b.handle_for(b.DTYPE_BF16, 0)

    def calls():
        sdpa.decode(qd, kd, vd, out=out1, lse=lse1, workspace=ws)
        st = b.sdpa_decode_noalloc(h, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out2.data_ptr(),
                                   lse2.data_ptr(), B, H, Lq, Lk, d, 0, None,
                                   torch.cuda.current_stream().cuda_stream)
        assert st == b.SUCCESS

    calls()
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    outputs = [out1, lse1, out2, lse2]
    eager = [t.clone() for t in outputs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    # eager work between replays, including the no-allocation decode on
    # other inputs (it shares the library's array with the graph's call)
    q2, k2, v2, _ = inputs.generate(1, 4, 1, 3000, d, "bf16", 6101)
    q2d, k2d, v2d = _dev(q2), _dev(k2), _dev(v2)
    o3 = torch.empty_like(q2d)

    def other():
        assert b.sdpa_decode_noalloc(h, q2d.data_ptr(), k2d.data_ptr(), v2d.data_ptr(), o3.data_ptr(), None,
                                     1, 4, 1, 3000, d, 0, None,
                                     torch.cuda.current_stream().cuda_stream) == b.SUCCESS
    _replay_and_check(torch, graph, outputs, eager, other)
