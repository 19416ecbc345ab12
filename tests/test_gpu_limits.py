"""The largest key/value spans the bf16 kernels accept, against the oracle on
sampled rows.

The forward kernels address one (batch, head) slice of k and v through
buffer loads with 32-bit byte offsets, so a slice may span just under 4 GiB;
the C ABI rejects more.  Three launches reach into the upper half of that
range:

* the general forward on the head-interleaved [B, L, H*d] layout, 15 heads of
  d_k = 128 and 2^20 keys: rows 3840 bytes apart, so each slice spans
  3.75 GiB and the last head's last rows sit just under 4 GiB from its base;
* the contiguous forward on one slice of 2^23 + 123 keys (2 GiB and a few
  KB), one query block, which the selector gives to the key-split tile;
* the decode path (split over key chunks, merged by their lse) on the same
  slice with three query rows.

Inputs: a seeded random block of 4096 keys (module recipe) repeated along the
keys, with feature 0 of q, k and v replaced by structure that makes every
result depend on where each key and value row was read from.  Every query has
feature 0 = 8 and key j has 10 j / Lk there, so the weights grow about
e^7-fold from the first key to the last; value j has 2 j / Lk in feature 0.
A row fetched from a wrong offset (wrapped at 2 or 4 GiB, or read as zeros
past a buffer's end) then moves the output's feature 0 and the lse by far
more than the tolerances (2e-2 and 1e-3); the output stays of order 1.
"""
import numpy as np
import pytest

from gpu_util import announce, assert_close, require_gpu
from transformer_scaled_dot_sdpa_amd import inputs

pytestmark = pytest.mark.gpu

BLOCK = 4096            # keys of the random block that is repeated
Q0, K0, V0 = 8.0, 10.0, 2.0


def ramp_bits(Lk: int, top: float) -> np.ndarray:
    """bf16 bits of top * j / Lk for j = 0 .. Lk-1."""
    return inputs.f32_to_bf16_bits((np.arange(Lk, dtype=np.float64) * (top / Lk)).astype(np.float32))


def structured(H: int, Lq: int, Lk: int, d: int, seed: int):
    """(q [1, H, Lq, d], k and v stored as [1, Lk, H, d]) as uint16 bf16 bits."""
    q, kb, vb, _ = inputs.generate(1, H, Lq, BLOCK, d, "bf16", seed)
    q[..., 0] = inputs.f32_to_bf16_bits(np.float32(Q0))
    reps = -(-Lk // BLOCK)
    k = np.tile(kb.transpose(0, 2, 1, 3), (1, reps, 1, 1))[:, :Lk]
    v = np.tile(vb.transpose(0, 2, 1, 3), (1, reps, 1, 1))[:, :Lk]
    k[0, :, :, 0] = ramp_bits(Lk, K0)[:, None]
    v[0, :, :, 0] = ramp_bits(Lk, V0)[:, None]
    return q, k, v


def check_rows(q, k, v, o_gpu, l_gpu, heads, rows, what):
    """Oracle on the given query rows of the given heads (k, v stored as
    [1, Lk, H, d]) against the GPU results o_gpu [1, H, Lq, d], l_gpu [1, H, Lq].
    One oracle call per row, run side by side on host threads (the oracle
    gives a handful of rows to a single thread, and a row of 8 M keys takes
    it about 20 s)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    for h in heads:
        kh = np.ascontiguousarray(k[:, :, h])[:, None]
        vh = np.ascontiguousarray(v[:, :, h])[:, None]
        qh = np.ascontiguousarray(q[:, h:h + 1])
        with ThreadPoolExecutor(len(rows)) as ex:
            res = list(ex.map(lambda r: oracle.sdpa_rows(qh, kh, vh, [r], bf16=True, nthreads=1), rows))
        ro = np.concatenate([o for o, _ in res])
        rl = np.concatenate([l for _, l in res])
        assert_close(o_gpu[0, h, rows], l_gpu[0, h, rows], ro, rl, "bf16", f"{what} head {h} rows {rows}")
        # the structure is there: the weights sit on the far keys
        assert np.all(ro[:, 0] > 1.2), ro[:, 0]


def test_interleaved_slice_spans_3_75_gib():
    require_gpu()
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    H, Lq, Lk, d = 15, 70, 1 << 20, 128
    seed = 4100
    span = ((Lk - 1) * H * d + d) * 2
    announce(f"limits: forward_ex interleaved H{H} Lq{Lq} Lk{Lk} d{d} seed={seed}, {span / 2**30:.3f} GiB per slice")
    q, k, v = structured(H, Lq, Lk, d, seed)
    qd = torch.from_numpy(q).view(torch.bfloat16).cuda()
    kd = torch.from_numpy(k).view(torch.bfloat16).cuda().transpose(1, 2)    # [1, H, Lk, d], rows H*d apart
    vd = torch.from_numpy(v).view(torch.bfloat16).cuda().transpose(1, 2)
    assert kd.stride(2) == H * d and span < 2**32 and span > 3 * 2**30
    o, l = sdpa.forward_ex(qd, kd, vd)
    torch.cuda.synchronize()
    o_gpu, l_gpu = o.float().cpu().numpy(), l.cpu().numpy()
    del qd, kd, vd, o, l
    torch.cuda.empty_cache()
    check_rows(q, k, v, o_gpu, l_gpu, heads=(0, 7, H - 1), rows=[0, 37, Lq - 1], what="interleaved 3.75 GiB")


@pytest.fixture(scope="module")
def long_slice():
    """One contiguous slice of 2^23 + 123 keys, d_k = 128: k and v span 2 GiB
    and 31 KB each.  Host copies (for the oracle) and device copies."""
    require_gpu()
    import torch
    H, Lq, Lk, d = 1, 70, (1 << 23) + 123, 128
    seed = 4101
    assert Lk * d * 2 > 2**31
    announce(f"limits: contiguous slice H{H} Lq{Lq} Lk{Lk} d{d} seed={seed}, {Lk * d * 2 / 2**30:.4f} GiB")
    q, k, v = structured(H, Lq, Lk, d, seed)
    dev = {"q": torch.from_numpy(q).view(torch.bfloat16).cuda(),
           "k": torch.from_numpy(k).view(torch.bfloat16).cuda().transpose(1, 2).contiguous(),
           "v": torch.from_numpy(v).view(torch.bfloat16).cuda().transpose(1, 2).contiguous()}
    yield q, k, v, dev
    dev.clear()
    torch.cuda.empty_cache()


def test_contiguous_slice_over_2_gib(long_slice):
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    q, k, v, dev = long_slice
    Lq = q.shape[2]
    name = sdpa.kernel_name(dev["q"], dev["k"], causal=False)
    announce(f"limits: forward on the 2 GiB slice, tile {name}")
    o, l = sdpa.forward(dev["q"], dev["k"], dev["v"])
    torch.cuda.synchronize()
    o_gpu, l_gpu = o.float().cpu().numpy(), l.cpu().numpy()
    check_rows(q, k, v, o_gpu, l_gpu, heads=(0,), rows=[0, 35, Lq - 1], what=f"contiguous 2 GiB ({name})")


def test_decode_slice_over_2_gib(long_slice):
    """The split-over-keys decode (key chunks merged by their lse) on the same
    slice, three query rows."""
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    q, k, v, dev = long_slice
    qd = dev["q"][:, :, :3].contiguous()
    ws = sdpa.decode_workspace_size(qd, dev["k"])
    announce(f"limits: decode on the 2 GiB slice, 3 rows, workspace {ws} bytes")
    assert ws > 0                       # the split kernel, not the main forward
    o, l = sdpa.decode(qd, dev["k"], dev["v"])
    torch.cuda.synchronize()
    o_gpu, l_gpu = o.float().cpu().numpy(), l.cpu().numpy()
    check_rows(np.ascontiguousarray(q[:, :, :3]), k, v, o_gpu, l_gpu, heads=(0,), rows=[0, 1, 2],
               what="decode 2 GiB")
