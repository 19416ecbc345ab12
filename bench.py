#!/usr/bin/env python3
"""Benchmark of the attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one ``sdpa_forward`` over the whole workload batch (every (b, h)
slice, the full hot path in one kernel launch), with inputs already resident
in HBM.  W untimed steps, then K timed steps bracketed by
``torch.cuda.synchronize()``.  Rank 0 prints one JSON line with:

* ``value``: headline TFLOP/s, flops = 4*B*H*Lq*Lk*d_k, halved for causal,
  divided by the wall time per step;
* ``roofline``: the kernel's algorithmic work per launch (4*d_k flops per
  valid (query, key) pair, or the compulsory bytes for a bandwidth-bound
  workload) over its average launch duration measured with HIP events on the
  launch stream, against the MI355X published peak (dense bf16 MFMA
  2.5 PFLOP/s, HBM 8 TB/s); ``traffic`` = HBM bytes per launch from the
  committed rocprofv3 counter summary when it was taken on the current kernel
  source, else null;
* ``cpu_baseline``: the fp64 CPU oracle timed on this host on a bounded
  sample of the same workload (whole (b, h) slices), TFLOP/s by the same
  headline formula;
* ``backward``: the same workload's ``sdpa_backward`` (gradients dq, dk, dv
  from dout, out and lse), timed the same way after the forward steps; its
  algorithmic work is 10*d_k flops per valid pair (five products of 2*d_k:
  S and dP recomputed once, dV, dQ, dK), reported against the same peak;
* ``decode``: ``sdpa_decode`` (1..8 query rows, split over key chunks) on the
  decode-shaped workloads (default ``decode_d128`` and ``decode_d64_single``),
  each timed as batches of back-to-back calls between two HIP events,
  reported as HBM GB/s of algorithmic bytes (the workloads are bandwidth
  bound), with ``sdpa_forward`` timed on the same inputs beside it;
* ``forward_ex``: ``sdpa_forward_ex`` on the main workload's own inputs in
  the head-interleaved [B, L, H*d] layout, and with an additive fp32 bias
  (a [Lq, Lk] matrix shared by every slice) on top of the causal mask, each
  timed with HIP events and reported in TFLOP/s by the headline formula;
* ``configs``: the other workloads of the benchmark set (toy fp32, encoder,
  decoder causal, cross-attention with key lengths), each timed as batches
  of 200 back-to-back calls between two HIP events on the launch stream,
  with at least 8 input/output sets rotated (more than the 256 MiB
  Infinity Cache together, so every call reads HBM); median of 5 batches,
  and the same with one set (hot cache) reported apart.  µs per call,
  TFLOP/s by the headline formula and algorithmic GB/s against 8 TB/s;
* ``vendor_gemm``: context for the MFMA roofline -- the rate torch.matmul
  (the vendor BLAS) reaches on a large square bf16 product on the same GPU in
  the same run, i.e. what dense matrix cores deliver in practice at the clock
  the chip holds under full MFMA load, and ``value`` as a fraction of it.

Before the W warm-up steps the GPU runs untimed calls for
``--clock-settle`` seconds (default 0.25): its clock takes tens of
milliseconds to ramp up from idle, which a handful of warm-up steps of the
default workload does not cover.  ``--all`` prints one JSON line per
workload instead (the main line first).

Only one GPU is used; ``--gpus`` above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # flop / byte
KERNEL_SOURCES = ["transformer_scaled_dot_sdpa_amd/csrc/sdpa_fwd_bf16.hip",
                  "transformer_scaled_dot_sdpa_amd/csrc/bf16_common.h",
                  "transformer_scaled_dot_sdpa_amd/csrc/tile_select.cpp"]
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_work(w, key_lens):
    """(flops, bytes) the method needs: 4*d per valid (query, key) pair;
    Q, valid K/V rows, O read/written once, lse written once."""
    import numpy as np
    e = 2 if w.dtype == "bf16" else 4
    per_b = []
    for b in range(w.B):
        n = w.Lk if key_lens is None else int(min(max(int(key_lens[b]), 0), w.Lk))
        if w.causal:
            i = np.arange(w.Lq)
            pairs = int(np.minimum(i + 1, n).sum())
            kv_rows = min(n, w.Lq)
        else:
            pairs = w.Lq * n
            kv_rows = n
        per_b.append((pairs, kv_rows))
    pairs = sum(p for p, _ in per_b) * w.H
    kv_rows = sum(r for _, r in per_b) * w.H
    flops = 4.0 * w.d * pairs
    nbytes = e * w.d * (2 * w.B * w.H * w.Lq + 2 * kv_rows) + 4 * w.B * w.H * w.Lq
    return flops, float(nbytes)


def read_traffic(workload: str):
    """HBM bytes per launch from profiles/<workload>_hbm_traffic.md, if that
    summary was taken on the current kernel source."""
    path = os.path.join(PROFILES, f"{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


def host_cpu():
    """Model name and thread counts of the host the oracle runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count(),
            "usable_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(w, q, k, v, key_lens, out_gpu, lse_gpu, target_s: float):
    """Time the CPU oracle on whole (b, h) slices of the workload."""
    import numpy as np
    import oracle
    threads = min(16, len(os.sched_getaffinity(0)))
    bf16 = w.dtype == "bf16"
    per_head_flops = w.flops / (w.B * w.H)

    def run(nheads):
        rows = np.arange(nheads * w.Lq, dtype=np.int64)
        t0 = time.perf_counter()
        o, l = oracle.sdpa_rows(q, k, v, rows, causal=w.causal, key_lens=key_lens,
                                bf16=bf16, nthreads=threads)
        return time.perf_counter() - t0, rows, o, l

    t1, rows, o, l = run(1)
    nheads = 1
    if t1 < target_s / 2:
        nheads = int(max(1, min(w.B * w.H, round(target_s / max(t1, 1e-6)))))
        if nheads > 1:
            t1, rows, o, l = run(nheads)
    value = nheads * per_head_flops / t1 / 1e12
    # the same oracle on one thread, over the first rows of slice 0 up to
    # about 2 million (query, key) pairs, with the flops of exactly those rows
    kl0 = w.Lk if key_lens is None else max(0, min(w.Lk, int(key_lens[0])))
    all_rows = np.arange(w.Lq, dtype=np.int64)
    valid = np.minimum(kl0, all_rows + 1) if w.causal else np.full(w.Lq, kl0)
    n1 = int(max(1, np.searchsorted(np.cumsum(valid), 2_000_000, side="right")))
    rows1 = all_rows[:n1]
    flops1 = 4.0 * w.d * float(valid[:n1].sum())
    t0 = time.perf_counter()
    oracle.sdpa_rows(q, k, v, rows1, causal=w.causal, key_lens=key_lens, bf16=bf16, nthreads=1)
    t_one = time.perf_counter() - t0
    og = out_gpu.reshape(-1, w.d)[rows]
    lg = lse_gpu.reshape(-1)[rows]
    fin = np.isfinite(l)
    return {
        "value": value,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{nheads} whole (b,h) slice(s) of {w.name} ({nheads * w.Lq} query rows, "
                   f"{nheads * per_head_flops / 1e9:.2f} GFLOP headline), fp64, "
                   f"{t1:.2f} s wall"),
        "seconds": t1,
        "host": host_cpu(),
        "one_thread": {"value": flops1 / t_one / 1e12, "unit": "TFLOP/s (algorithmic)",
                       "sample": f"query rows 0..{n1 - 1} of slice 0, {t_one:.2f} s wall"},
        "sample_max_abs_out_vs_gpu": float(np.max(np.abs(og - o))),
        "sample_max_abs_lse_vs_gpu": float(np.max(np.abs(lg[fin] - l[fin]), initial=0.0)),
    }


def copy_calibration(mib: int):
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_calibration_bytes": n, "copies": 3}


def vendor_gemm(torch, m: int = 16384, n: int = 16384, k: int = 8192, iters: int = 10):
    """TFLOP/s of torch.matmul on an (m x k) by (k x n) bf16 product (contiguous operands)."""
    a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(k, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    del a, b, c
    return {"value": 2.0 * m * n * k / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
            "kind": f"torch.matmul bf16 ({m}x{k}) by ({k}x{n})", "ms": ms}


def backward_leg(torch, sdpa, inputs, w, sets, tkl, stream, args, fwd_flops_alg):
    """Time sdpa_backward on the forward's own outputs (first input set)."""
    import numpy as np
    tq, tk, tv, out, lse = sets[0]
    g = torch.from_numpy(inputs.generate_dout(w.B, w.H, w.Lq, w.d, w.dtype, w.seed))
    dout = (g.view(torch.bfloat16) if w.dtype == "bf16" else g).cuda()
    sdpa.forward(tq, tk, tv, causal=w.causal, key_lens=tkl, out=out, lse=lse, stream=stream)
    dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
    delta = torch.empty_like(lse)

    def bstep():
        sdpa.backward(tq, tk, tv, out, lse, dout, causal=w.causal, key_lens=tkl, dq=dq, dk=dk,
                      dv=dv, delta=delta, stream=stream)

    steps = max(1, min(args.steps, 20))
    print(f"[bench] backward: warmup {min(args.warmup, 5)}, timed {steps}", file=sys.stderr,
          flush=True)
    for _ in range(min(args.warmup, 5)):
        bstep()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        bstep()
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms_wall = (time.perf_counter() - t0) * 1e3 / steps
    ms = float(np.mean([s.elapsed_time(e) for s, e in zip(starts, ends)]))
    flops = 2.5 * fwd_flops_alg   # 10*d_k per valid pair
    achieved = flops / (ms * 1e-3) / 1e12
    head = 2.5 * w.flops / (ms_wall * 1e-3) / 1e12
    print(f"[bench] backward {ms:.4f} ms/call, {achieved:.1f} TFLOP/s", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = backward_cpu_baseline(w, sets, dout, (dq, dk, dv), args.cpu_seconds / 2)
    del dq, dk, dv, delta, dout
    out = {"ms_per_call": ms, "ms_per_step_wall": ms_wall, "steps": steps,
            "value": head, "unit": "TFLOP/s",
            "flops_note": "10*d_k per pair (2.5x the forward's 4*d_k), halved for causal",
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                         "algorithmic_flops_per_call": flops,
                         "kernels": "bwd_dq_kernel (with D), bwd_dkdv_kernel"}}
    if cpu is not None:
        out["cpu_baseline"] = cpu
    return out


def backward_cpu_baseline(w, sets, dout, grads, target_s):
    """The oracle's fp64 backward on whole (b, h) slices (one thread per
    slice, as many slices as host threads, repeated up to the time target),
    TFLOP/s at 10*d_k flops per valid pair; plus the largest gradient
    difference against the GPU on the sample."""
    import numpy as np
    import oracle
    threads = min(16, len(os.sched_getaffinity(0)))
    nsl = min(threads, w.H)
    bits = lambda t: t[0:1, 0:nsl].contiguous().cpu().view(torch_int16()).numpy().view(np.uint16)
    tq, tk, tv = (bits(t) for t in sets[0][:3])
    g = bits(dout)
    t0 = time.perf_counter()
    ref = oracle.sdpa_bwd(tq, tk, tv, g, causal=w.causal, bf16=True, nthreads=threads)
    sec = time.perf_counter() - t0
    pairs_per_slice = (w.Lq * (w.Lq + 1) // 2) if (w.causal and w.Lq == w.Lk) else w.Lq * w.Lk
    flops = 10.0 * w.d * pairs_per_slice * nsl
    diff = max(float(np.max(np.abs(gr[0:1, 0:nsl].float().cpu().numpy() - r))) for gr, r in zip(grads, ref))
    return {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{nsl} whole (b,h) slice(s) of {w.name}, fp64 backward, {sec:.2f} s wall",
            "seconds": sec, "sample_max_abs_grad_vs_gpu": diff}


def torch_int16():
    import torch
    return torch.int16


def forward_ex_leg(torch, sdpa, w, sets, tkl, stream, args):
    """sdpa_forward_ex on the first input set: head-interleaved layout, then
    an additive bias on the scaled scores (plus the workload's own masks)."""
    import numpy as np
    tq, tk, tv = sets[0][:3]
    lse = torch.empty_like(sets[0][4])   # the main leg's outputs stay untouched
    il = lambda t: t.transpose(1, 2).contiguous().transpose(1, 2)
    iq, ik, iv = il(tq), il(tk), il(tv)
    iout = il(torch.empty_like(tq))
    gen = torch.Generator(device="cuda").manual_seed(w.seed)
    bias = torch.randn((w.Lq, w.Lk), device="cuda", generator=gen, dtype=torch.float32) * 0.5
    out = torch.empty_like(tq)

    def timed(fn):
        steps = max(1, min(args.steps, 20))
        for _ in range(min(args.warmup, 3)):
            fn()
        torch.cuda.synchronize()
        st = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        en = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for i in range(steps):
            st[i].record(stream)
            fn()
            en[i].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in zip(st, en)])), steps

    ms_il, steps = timed(lambda: sdpa.forward_ex(iq, ik, iv, causal=w.causal, key_lens=tkl, out=iout,
                                                 lse=lse, stream=stream))
    ms_mask, _ = timed(lambda: sdpa.forward_ex(tq, tk, tv, causal=w.causal, key_lens=tkl, mask=bias,
                                               out=out, lse=lse, stream=stream))
    # the same bias with every row's first 96 keys dropped (left padding):
    # each row's first key tile is masked entirely, or nearly
    bias_lp = bias.clone()
    bias_lp[:, :96] = -math.inf
    ms_lp, _ = timed(lambda: sdpa.forward_ex(tq, tk, tv, causal=w.causal, key_lens=tkl, mask=bias_lp,
                                             out=out, lse=lse, stream=stream))
    tf = lambda ms: w.flops / (ms * 1e-3) / 1e12
    print(f"[bench] forward_ex: interleaved {ms_il*1e3:.1f} us ({tf(ms_il):.1f} TFLOP/s), "
          f"with bias {ms_mask*1e3:.1f} us ({tf(ms_mask):.1f} TFLOP/s), left-padded bias "
          f"{ms_lp*1e3:.1f} us", file=sys.stderr, flush=True)
    del iq, ik, iv, iout, bias, bias_lp, out, lse
    return {"steps": steps,
            "interleaved": {"layout": "[B, L, H*d_k] for q, k, v and out", "us_per_call": ms_il * 1e3,
                            "value": tf(ms_il), "unit": "TFLOP/s"},
            "additive_bias": {"mask": "fp32 [Lq, Lk] shared by every (b, h), plus the workload's masks",
                              "us_per_call": ms_mask * 1e3, "value": tf(ms_mask), "unit": "TFLOP/s",
                              "mask_bytes": w.Lq * w.Lk * 4},
            "additive_bias_left_padded": {"mask": "the same bias with keys 0..95 at -inf in every row",
                                          "us_per_call": ms_lp * 1e3, "value": tf(ms_lp), "unit": "TFLOP/s",
                                          "time_vs_additive_bias": ms_lp / ms_mask}}


def decode_leg(torch, sdpa, inputs, name, args):
    """Time sdpa_decode and, on the same inputs, sdpa_forward."""
    import numpy as np
    w = inputs.WORKLOADS[name]
    print(f"[bench] decode leg: generating {w.name} (seed {w.seed})", file=sys.stderr, flush=True)
    q, k, v, kl = inputs.generate_workload(w)
    up = lambda x: torch.from_numpy(x).view(torch.bfloat16).cuda()
    tq, tk, tv = up(q), up(k), up(v)
    tkl = torch.from_numpy(kl).cuda() if kl is not None else None
    _, bytes_alg = algorithmic_work(w, kl)
    set_bytes = (tq.numel() + tk.numel() + tv.numel()) * 2
    nsets = 1 if set_bytes >= (1 << 30) else min(64, int(math.ceil((1 << 30) / set_bytes)))
    sets = [(tq, tk, tv)] + [(tq.clone(), tk.clone(), tv.clone()) for _ in range(nsets - 1)]
    out = torch.empty_like(tq)
    lse = torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device="cuda")
    need = sdpa.decode_workspace_size(tq, tk)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn, steps):
        # untimed calls for at least 100 ms: the clocks ramp up over tens of
        # milliseconds after the small main workload, and a few calls leave
        # the first timed leg up to 15% slow
        t_end = time.perf_counter() + 0.1
        i = 0
        while time.perf_counter() < t_end:
            for _ in range(10):
                fn(sets[i % nsets])
                i += 1
            torch.cuda.synchronize()
        # one event pair around the back-to-back calls (a call can take a
        # few microseconds, of the order of an event pair's own cost);
        # median of 3 batches
        res = []
        for _ in range(3):
            st = torch.cuda.Event(enable_timing=True)
            en = torch.cuda.Event(enable_timing=True)
            st.record(stream)
            for i in range(steps):
                fn(sets[i % nsets])
            en.record(stream)
            torch.cuda.synchronize()
            res.append(st.elapsed_time(en) / steps)
        return float(np.median(res))

    steps = 200 if w.B * w.H * w.Lk < (1 << 24) else 50
    dec = lambda a, st=stream: sdpa.decode(a[0], a[1], a[2], causal=w.causal, key_lens=tkl, out=out, lse=lse,
                                           workspace=ws, stream=st)
    fwd = lambda a, st=stream: sdpa.forward(a[0], a[1], a[2], causal=w.causal, key_lens=tkl, out=out, lse=lse,
                                            stream=st)
    dec_eager_ms = timed(dec, steps)
    # the GPU's time per call: the same calls replayed from a HIP graph
    dec_us, _ = graph_replay_us(torch, [lambda a=sets[i % nsets]: dec(a, None) for i in range(steps)], [out, lse])
    dec_ms = dec_us * 1e-3
    fwd_ms = None
    if not args.no_decode_forward:
        fwd_us, _ = graph_replay_us(torch, [lambda a=sets[i % nsets]: fwd(a, None) for i in range(steps)],
                                    [out, lse])
        fwd_ms = fwd_us * 1e-3
    gbs = bytes_alg / (dec_ms * 1e-3) / 1e9
    print(f"[bench] decode {w.name}: {dec_ms*1e3:.1f} us ({gbs:.0f} GB/s; eager launches {dec_eager_ms*1e3:.1f} us)"
          + (f"; forward on the same inputs {fwd_ms*1e3:.1f} us" if fwd_ms is not None else ""),
          file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = min(16, len(os.sched_getaffinity(0)))
        sdpa.decode(tq, tk, tv, causal=w.causal, key_lens=tkl, out=out, lse=lse, workspace=ws,
                    stream=stream)
        dec_out = out.float().cpu().numpy()
        t0 = time.perf_counter()
        ro, rl = oracle.sdpa(q, k, v, causal=w.causal, key_lens=kl, bf16=True, nthreads=threads)
        sec = time.perf_counter() - t0
        cpu = {"value": bytes_alg / sec / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"the whole {w.name} workload, fp64, {sec:.2f} s wall", "seconds": sec,
               "sample_max_abs_out_vs_gpu": float(np.max(np.abs(dec_out - ro)))}
    del sets, out, lse, ws
    res = {"workload": w.name, "B": w.B, "H": w.H, "Lq": w.Lq, "Lk": w.Lk, "d_k": w.d,
            "key_lens": None if kl is None else "uniform[%d,%d]" % w.key_lens,
            "input_sets": nsets, "steps": steps, "us_per_call": dec_ms * 1e3,
            "timing": "one HIP event pair around a HIP graph of the back-to-back calls, median of 5 replays",
            "us_per_call_eager": dec_eager_ms * 1e3,
            "workspace_bytes": need,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "algorithmic_bytes_per_call": bytes_alg,
                         "kernels": "the forward kernel when the slices fill the GPU (decode_d128), else decode_kernel (+ decode_combine when split)"},
            "forward_same_inputs_us": fwd_ms * 1e3 if fwd_ms is not None else None}
    if cpu is not None:
        res["cpu_baseline"] = cpu
    return res


def graph_replay_us(torch, calls, outputs, reps=5):
    """Per-call GPU time of `calls` (functions that each enqueue one library
    call on the current stream) captured into one HIP graph and replayed
    `reps` times; median over the replays.  A short call takes a few
    microseconds, about what the Python binding needs to enqueue one, so
    eager back-to-back calls measure the host's launch rate; the graph
    replays the same kernels without it.  `outputs` (tensors the calls
    write) are compared bit for bit with the eager results after the first
    and the last replay (the outputs of deterministic kernels on the same
    inputs)."""
    import numpy as np
    for c in calls:                       # eager reference (and warm-up)
        c()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    res = []
    for r in range(reps):
        for t in outputs:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) * 1e3 / len(calls))
        if r in (0, reps - 1):
            for t, rt in zip(outputs, ref):
                if not torch.equal(t.view(torch.uint8), rt.view(torch.uint8)):
                    raise RuntimeError("graph replay differs from the eager calls")
    del g
    return float(np.median(res)), res


SMALL_CONFIGS = ["toy_f32", "encoder_d64", "decoder_causal_d64", "cross_padded_d64"]


def config_leg(torch, sdpa, inputs, name, batch=200, batches=5):
    """One workload timed as batches of back-to-back sdpa_forward calls with
    rotated input/output sets (see the module docstring)."""
    import numpy as np
    w = inputs.WORKLOADS[name]
    print(f"[bench] config {w.name}: generating (seed {w.seed})", file=sys.stderr, flush=True)
    q, k, v, kl = inputs.generate_workload(w)

    def up(x):
        t = torch.from_numpy(x)
        return (t.view(torch.bfloat16) if w.dtype == "bf16" else t).cuda()

    base = (up(q), up(k), up(v))
    tkl = torch.from_numpy(kl).cuda() if kl is not None else None
    flops_alg, bytes_alg = algorithmic_work(w, kl)
    per_set = sum(t.numel() * t.element_size() for t in base) * 2 + w.B * w.H * w.Lq * 4
    nsets = min(64, max(8, int(math.ceil((300 << 20) / per_set))))
    sets = [tuple(t.clone() for t in base) + (torch.empty_like(base[0]),
                                               torch.empty((w.B, w.H, w.Lq), dtype=torch.float32,
                                                           device="cuda")) for _ in range(nsets)]
    stream = torch.cuda.current_stream()

    def call(a, stream=stream):
        sdpa.forward(a[0], a[1], a[2], causal=w.causal, key_lens=tkl, out=a[3], lse=a[4], stream=stream)

    t_end = time.perf_counter() + 0.2
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(50):
            call(sets[i % nsets])
            i += 1
        torch.cuda.synchronize()

    def timed(rotate):
        res = []
        for _ in range(batches):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for j in range(batch):
                call(sets[j % nsets] if rotate else sets[0])
            e1.record(stream)
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) * 1e3 / batch)
        return float(np.median(res)), res

    us_eager, eager_all = timed(True)
    us_eager_hot, _ = timed(False)
    # the same calls replayed from a HIP graph (the GPU's time per call)
    outs = [x for a in sets[:min(batch, nsets)] for x in a[3:5]]
    us, all_us = graph_replay_us(torch, [lambda a=sets[j % nsets]: call(a, None) for j in range(batch)], outs)
    us_hot, _ = graph_replay_us(torch, [lambda: call(sets[0], None) for _ in range(batch)], list(sets[0][3:5]))
    gbs = bytes_alg / (us * 1e-6) / 1e9
    out = {"workload": w.name, "B": w.B, "H": w.H, "Lq": w.Lq, "Lk": w.Lk, "d_k": w.d, "dtype": w.dtype,
           "causal": w.causal, "key_lens": None if kl is None else "uniform[%d,%d]" % w.key_lens,
           "seed": w.seed, "kernel": sdpa.kernel_name(base[0], base[1], w.causal, kl is not None),
           "timing": ("one HIP event pair around a HIP graph of the back-to-back calls (rotated input "
                      "sets), median of 5 replays; eager: the same calls launched from Python"),
           "us_per_call": us, "us_per_call_batches": all_us, "us_per_call_hot_cache": us_hot,
           "us_per_call_eager": us_eager, "us_per_call_eager_batches": eager_all,
           "us_per_call_eager_hot_cache": us_eager_hot,
           "calls_per_batch": batch, "input_sets": nsets,
           "value": w.flops / (us * 1e-6) / 1e12, "unit": "TFLOP/s",
           "algorithmic_flops_per_call": flops_alg, "algorithmic_bytes_per_call": bytes_alg}
    if w.dtype == "fp32":
        out["roofline"] = {"bound": "latency", "note": f"{bytes_alg:.0f} B and {flops_alg:.0f} flop per call: "
                           "the time is the launch; reported in us"}
    else:
        out["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": gbs / PEAK_HBM_GBS}
    print(f"[bench] config {w.name}: {us:.2f} us/call rotated (graph; eager {us_eager:.2f}), {us_hot:.2f} us hot, "
          f"{gbs:.0f} GB/s, kernel {out['kernel']}", file=sys.stderr, flush=True)
    del sets, base
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=60,
                    help="untimed steps first (about 0.1 s at the default workload: the clocks ramp up over tens of ms)")
    ap.add_argument("--workload", default="large_causal_d128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the CPU-oracle sample")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward leg")
    ap.add_argument("--decode-workload", default="decode_d128,decode_d64_single",
                    help="decode-shaped workloads of the decode leg, comma-separated ('none' skips it)")
    ap.add_argument("--no-forward-ex", action="store_true", help="skip the forward_ex leg")
    ap.add_argument("--no-decode-forward", action="store_true",
                    help="in the decode leg, skip timing sdpa_forward on the same inputs")
    ap.add_argument("--no-vendor-gemm", action="store_true",
                    help="skip the vendor GEMM context measurement")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (toy, encoder, decoder, cross-attention)")
    ap.add_argument("--all", action="store_true",
                    help="print one JSON line per workload (the main line first)")
    ap.add_argument("--clock-settle", type=float, default=0.25,
                    help="seconds of untimed calls before the warm-up steps (clock ramp)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the attention slices are independent, so N GPUs would each run "
              "this same kernel on their own share.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import transformer_scaled_dot_sdpa_amd as sdpa
    from transformer_scaled_dot_sdpa_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    w = inputs.WORKLOADS[args.workload]
    print(f"[bench] generating {w.name} (seed {w.seed})", file=sys.stderr, flush=True)
    q, k, v, kl = inputs.generate_workload(w)

    def up(x):
        t = torch.from_numpy(x)
        return (t.view(torch.bfloat16) if w.dtype == "bf16" else t).cuda()

    tq, tk, tv = up(q), up(k), up(v)
    tkl = torch.from_numpy(kl).cuda() if kl is not None else None
    flops_alg, bytes_alg = algorithmic_work(w, kl)
    # Small workloads fit in the 256 MB Infinity Cache: rotate several input
    # copies so every step reads HBM.
    set_bytes = (tq.numel() + tk.numel() + tv.numel()) * tq.element_size() * 2
    # (at most 64: a problem too small to need that many is bound by launch
    # latency, not by HBM)
    nsets = 1 if set_bytes >= (1 << 30) else min(64, int(math.ceil((1 << 30) / set_bytes)))
    sets = [(tq, tk, tv, torch.empty_like(tq),
             torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device="cuda"))]
    for _ in range(nsets - 1):
        sets.append((tq.clone(), tk.clone(), tv.clone(), torch.empty_like(tq),
                     torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device="cuda")))
    if args.copy_calibration_mib:
        copy_info = copy_calibration(args.copy_calibration_mib)
        print(f"[bench] copy calibration {copy_info}", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    kname = sdpa.kernel_name(tq, tk, w.causal, kl is not None)

    def step(i):
        a = sets[i % nsets]
        sdpa.forward(a[0], a[1], a[2], causal=w.causal, key_lens=tkl, out=a[3], lse=a[4],
                     stream=stream)

    settle_calls = 0
    t_end = time.perf_counter() + args.clock_settle
    while time.perf_counter() < t_end:
        step(settle_calls)
        settle_calls += 1
        torch.cuda.synchronize()
    print(f"[bench] clock settle {settle_calls} untimed calls; warmup {args.warmup} steps, kernel {kname}, "
          f"{nsets} input set(s)", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Kernel time on the launch stream.  A launch of the default workload
    # takes milliseconds, and HIP events around each launch measure it
    # directly.  A launch of the small workloads takes microseconds, of the
    # order of an event pair's own cost and of the binding's launch cost, so
    # those are timed as the K steps replayed from a HIP graph (the kernel
    # trace of the same command gives the per-dispatch figure to compare
    # with).
    batch_timing = w.flops < 1e11
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if batch_timing:
        starts[0].record(stream)
        for i in range(args.steps):
            step(i)
        ends[0].record(stream)
    else:
        for i in range(args.steps):
            starts[i].record(stream)
            step(i)
            ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    if batch_timing:
        # the GPU's time per step: the same K steps replayed from a HIP graph
        # (eager launches from Python would measure the host's launch rate)
        us, _ = graph_replay_us(torch, [lambda i=i: sdpa.forward(
            sets[i % nsets][0], sets[i % nsets][1], sets[i % nsets][2], causal=w.causal, key_lens=tkl,
            out=sets[i % nsets][3], lse=sets[i % nsets][4]) for i in range(args.steps)],
            [x for a in sets[:min(args.steps, nsets)] for x in a[3:5]])
        kernel_ms = [us * 1e-3]
    else:
        kernel_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    kernel_avg_ms = float(np.mean(kernel_ms))
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.4f} ms/step wall, kernel "
          f"avg {kernel_avg_ms:.4f} ms (min {min(kernel_ms):.4f}, max {max(kernel_ms):.4f})",
          file=sys.stderr, flush=True)

    value = w.flops / (ms_per_step * 1e-3) / 1e12
    ai = flops_alg / bytes_alg
    if ai >= RIDGE:
        achieved = flops_alg / (kernel_avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS}
    else:
        achieved = bytes_alg / (kernel_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS}
    roof["traffic"] = read_traffic(w.name)
    roof["algorithmic_flops_per_launch"] = flops_alg
    roof["algorithmic_bytes_per_launch"] = bytes_alg
    roof["kernel_avg_ms"] = kernel_avg_ms
    roof["timing"] = ("one HIP event pair around a HIP graph of the K steps, median of 5 replays" if batch_timing
                      else "HIP events around each timed launch")
    roof["kernel"] = kname

    result = {
        "metric": "attention fwd TFLOP/s (bf16, 1 GPU) and % of MI355X dense-bf16 MFMA peak",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": {"seconds": args.clock_settle, "untimed_calls": settle_calls},
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Lq": w.Lq, "Lk": w.Lk, "d_k": w.d,
                   "causal": w.causal, "key_lens": None if kl is None else "uniform[%d,%d]" % w.key_lens,
                   "input_scale": w.scale, "seed": w.seed, "input_sets": nsets},
        "roofline": roof,
    }
    configs = []
    if not args.no_configs:
        for name in SMALL_CONFIGS:
            if name != w.name:
                configs.append(config_leg(torch, sdpa, inputs, name))
        result["configs"] = {c["workload"]: {k: c[k] for k in ("us_per_call", "us_per_call_hot_cache",
                                                                "us_per_call_eager", "value", "unit", "roofline",
                                                                "kernel")}
                             for c in configs}
    if not args.no_backward and w.dtype == "bf16":
        result["backward"] = backward_leg(torch, sdpa, inputs, w, sets, tkl, stream, args,
                                          flops_alg)
    if not args.no_forward_ex and w.dtype == "bf16":
        result["forward_ex"] = forward_ex_leg(torch, sdpa, w, sets, tkl, stream, args)
    if args.decode_workload != "none":
        result["decode"] = {name: decode_leg(torch, sdpa, inputs, name, args)
                            for name in args.decode_workload.split(",")}
    if not args.no_vendor_gemm:
        g = vendor_gemm(torch)
        g["attention_value_over_gemm"] = value / g["value"]
        result["vendor_gemm"] = g
        print(f"[bench] vendor GEMM {g['value']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        a = sets[(args.steps - 1) % nsets]
        out_gpu = a[3].float().cpu().numpy()
        lse_gpu = a[4].cpu().numpy()
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, kl, out_gpu, lse_gpu, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    if args.all:
        for c in configs:
            line = {"metric": result["metric"], "value": c["value"], "unit": "TFLOP/s", "n_gpus": 1,
                    "steps": c["calls_per_batch"], "warmup": 0, "ms_per_step": c["us_per_call"] * 1e-3,
                    "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": c["dtype"],
                    "data": "synthetic",
                    "config": {k: c[k] for k in ("workload", "B", "H", "Lq", "Lk", "d_k", "causal", "key_lens",
                                                 "seed", "input_sets")},
                    "roofline": c["roofline"], "kernel": c["kernel"],
                    "us_per_call": c["us_per_call"], "us_per_call_hot_cache": c["us_per_call_hot_cache"],
                    "us_per_call_batches": c["us_per_call_batches"]}
            print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
