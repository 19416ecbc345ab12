"""Decode-shaped forward (sdpa_decode) vs the CPU oracle through the C ABI.

Same operation and tolerances as the main forward (max-abs 2e-2 on bf16
outputs, 1e-3 on lse, -inf rows exact).  The cases cover one and several
chunks per slice (few slices force a split over keys), every supported query
count, ragged chunk tails, key lengths 0 / 1 / full / clamped, causal rows and
the two decode workloads at full size.
"""
import numpy as np
import pytest

from gpu_util import announce, assert_close, oracle_ref, require_gpu, to_device
from transformer_scaled_dot_sdpa_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def run_decode(q, k, v, causal=False, key_lens=None, workspace_pad=0):
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    kl = torch.from_numpy(np.asarray(key_lens, dtype=np.int32)).to("cuda") if key_lens is not None else None
    need = sdpa.decode_workspace_size(qd, kd)
    ws = None
    if need:
        # poison the workspace: its contents on entry must not matter
        ws = torch.full((need + workspace_pad,), 0xFF, dtype=torch.uint8, device="cuda")
    out, lse = sdpa.decode(qd, kd, vd, causal=causal, key_lens=kl, workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), need


CASES = [
    # B, H, Lq, Lk, causal, key_lens
    (1, 1, 1, 1, False, None),
    (1, 1, 1, 7, False, None),
    (1, 2, 1, 4096, False, None),
    (1, 1, 3, 1000, False, None),
    (2, 2, 8, 777, False, [777, 300]),
    (3, 1, 2, 512, False, [0, 1, 512]),
    (2, 1, 4, 640, False, [-5, 10000]),
    (1, 2, 5, 300, True, None),
    (2, 3, 1, 2050, False, [2049, 1]),
    (64, 32, 1, 256, False, None),      # many slices: the forward kernel
]

# At least two slices per compute unit: sdpa_decode runs the main forward
# kernel, one workgroup per slice, with no workspace.  Several query rows,
# the causal flag and key lengths 0, 1, short, full and out of range.
FORWARD_CASES = [
    # B, H, Lq, Lk, causal, key_lens
    (64, 8, 5, 300, True, None),
    (64, 8, 8, 700, False, [0, 1, 2, 63, 64, 65, 699, 700, 701, -3] + [350] * 54),
    (64, 8, 2, 129, True, [0, 1, 64, 128, 129, 1000] + [100] * 58),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}q{}k{}c{}L{}".format(*c))
def test_decode_matches_oracle(d, case):
    B, H, Lq, Lk, causal, kl = case
    seed = 1300 + d + 7 * Lq + Lk
    announce(f"decode d{d} B{B} H{H} Lq{Lq} Lk{Lk} causal={causal} key_lens={kl} seed={seed}")
    q, k, v, _ = inputs.generate(B, H, Lq, Lk, d, "bf16", seed)
    o, l, need = run_decode(q, k, v, causal, kl)
    ro, rl = oracle_ref(q, k, v, "bf16", causal, kl)
    assert_close(o, l, ro, rl, "bf16", f"decode {case}")
    if kl is not None:
        for b, n in enumerate(kl):
            if n <= 0:
                assert np.all(o[b] == 0) and np.all(np.isneginf(l[b]))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", FORWARD_CASES, ids=lambda c: "B{}H{}q{}k{}c{}".format(*c[:5]))
def test_decode_forward_backed_matches_oracle(d, case):
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    B, H, Lq, Lk, causal, kl = case
    qe = torch.empty((B, H, Lq, d), dtype=torch.bfloat16, device="cuda")
    ke = torch.empty((B, H, Lk, d), dtype=torch.bfloat16, device="cuda")
    assert sdpa.decode_workspace_size(qe, ke) == 0      # the forward-backed path
    seed = 1400 + d + 7 * Lq + Lk
    announce(f"decode (forward kernel) d{d} B{B} H{H} Lq{Lq} Lk{Lk} causal={causal} seed={seed}")
    q, k, v, _ = inputs.generate(B, H, Lq, Lk, d, "bf16", seed)
    o, l, need = run_decode(q, k, v, causal, kl)
    assert need == 0
    ro, rl = oracle_ref(q, k, v, "bf16", causal, kl)
    assert_close(o, l, ro, rl, "bf16", f"decode forward-backed {case}")
    if kl is not None:
        for b, n in enumerate(kl):
            if n <= 0:
                assert np.all(o[b] == 0) and np.all(np.isneginf(l[b]))


def test_decode_split_and_single_chunk_both_exercised():
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    q = torch.empty((1, 2, 1, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((1, 2, 4096, 128), dtype=torch.bfloat16, device="cuda")
    assert sdpa.decode_workspace_size(q, k) > 0          # few slices: split over keys
    q = torch.empty((64, 32, 1, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((64, 32, 256, 128), dtype=torch.bfloat16, device="cuda")
    assert sdpa.decode_workspace_size(q, k) == 0         # many slices: the forward kernel
    q = torch.empty((2, 1, 1, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((2, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    assert sdpa.decode_workspace_size(q, k) == 0         # short keys: one chunk of the decode kernel
    q = torch.empty((16, 32, 1, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((16, 32, 8192, 128), dtype=torch.bfloat16, device="cuda")
    assert sdpa.decode_workspace_size(q, k) > 0          # d = 128, 8192 keys: split kernel


@pytest.mark.parametrize("name", ["decode_d128", "decode_d64_single"])
def test_decode_workload_full(name):
    w = inputs.WORKLOADS[name]
    announce(f"decode workload {name}: B{w.B} H{w.H} Lq{w.Lq} Lk{w.Lk} d{w.d} seed={w.seed}")
    q, k, v, kl = inputs.generate_workload(w)
    o, l, _ = run_decode(q, k, v, w.causal, kl)
    ro, rl = oracle_ref(q, k, v, "bf16", w.causal, kl)
    assert_close(o, l, ro, rl, "bf16", name)


def test_decode_workspace_reused_across_calls():
    """One workspace serves calls of different sizes in a row on one stream,
    each call's partial results overwriting the last call's."""
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    shapes = [(1, 2, 1, 4096, 64, None), (2, 3, 4, 2000, 128, [2000, 7]), (1, 8, 1, 4096, 64, None),
              (3, 1, 8, 999, 128, [0, 999, 500]), (1, 2, 1, 4096, 64, None)]
    cases = []
    for i, (B, H, Lq, Lk, d, kl) in enumerate(shapes):
        q, k, v, _ = inputs.generate(B, H, Lq, Lk, d, "bf16", 1500 + i)
        cases.append((q, k, v, kl, d))
    need = 0
    dev = []
    for q, k, v, kl, d in cases:
        qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
        need = max(need, sdpa.decode_workspace_size(qd, kd))
        dev.append((qd, kd, vd, torch.from_numpy(np.asarray(kl, np.int32)).cuda() if kl else None))
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    announce(f"decode: {len(cases)} calls sharing one {need}-byte workspace")
    outs = [sdpa.decode(qd, kd, vd, key_lens=klt, workspace=ws) for qd, kd, vd, klt in dev]
    torch.cuda.synchronize()
    for (q, k, v, kl, d), (o, l) in zip(cases, outs):
        ro, rl = oracle_ref(q, k, v, "bf16", False, kl)
        assert_close(o.float().cpu().numpy(), l.cpu().numpy(), ro, rl, "bf16", f"reused workspace {q.shape}")


def test_decode_agrees_with_forward():
    """Both entry points compute the same function; on the same inputs they
    differ only by rounding."""
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    q, k, v, kl = inputs.generate(2, 4, 4, 3000, 128, "bf16", 77, key_lens=(1, 3000))
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    klt = torch.from_numpy(kl).cuda()
    o1, l1 = sdpa.forward(qd, kd, vd, key_lens=klt)
    o2, l2 = sdpa.decode(qd, kd, vd, key_lens=klt)
    torch.cuda.synchronize()
    assert float((o1.float() - o2.float()).abs().max()) <= 2e-2
    assert float((l1 - l2).abs().max()) <= 1e-3


def test_decode_rejects_bad_workspace():
    import torch
    from transformer_scaled_dot_sdpa_amd import binding as b
    h = b.handle_for(b.DTYPE_BF16, 0)
    q = torch.zeros(1, 2, 1, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 2, 4096, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.zeros_like(q)
    need = b.sdpa_decode_workspace_size(h, 1, 2, 1, 4096, 128)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    p = lambda t: t.data_ptr()
    call = lambda **kw: b.sdpa_decode(**{**dict(handle=h, q=p(q), k=p(k), v=p(k), out=p(o), lse=None,
                                                B=1, H=2, Lq=1, Lk=4096, d_k=128, causal=0,
                                                key_lens=None, workspace=p(ws), workspace_bytes=need,
                                                stream=None), **kw})
    assert call() == b.SUCCESS
    torch.cuda.synchronize()
    assert call(workspace=None) == b.INVALID_VALUE
    assert call(workspace_bytes=need - 4) == b.INVALID_VALUE
    assert call(workspace=p(ws) + 2) == b.INVALID_VALUE          # misaligned
    assert call(workspace=p(k)) == b.INVALID_VALUE               # overlaps k
    assert call(Lq=9) == b.NOT_SUPPORTED
    assert call(d_k=96) == b.NOT_SUPPORTED
    hf = b.handle_for(b.DTYPE_FP32, 0)
    assert call(handle=hf) == b.NOT_SUPPORTED
    assert b.sdpa_decode_workspace_size(hf, 1, 2, 1, 4096, 128) == 0
