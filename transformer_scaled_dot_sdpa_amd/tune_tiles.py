"""Time every compiled bf16 tile configuration on a set of shapes and print
the markdown table behind the tile selector's thresholds.

    python -m transformer_scaled_dot_sdpa_amd.tune_tiles [--quick] > table.md

For each shape the inputs are drawn on the GPU (timing only; no parity is
checked here, the tests do that), every tile runs through
``sdpa_forward_ex``'s ``tile`` field, and the tiles are timed in turn as
batches of back-to-back calls between two HIP events (enough calls for about
20 ms), three rounds interleaved so that clock drift hits every tile alike;
the median per tile is reported, with the tile the selector picks
(``sdpa_kernel_name``) and its distance to the fastest.  Input sets are
rotated so that a shape's inputs exceed the 256 MiB Infinity Cache.
"""
from __future__ import annotations

import argparse
import sys
import time

TILES = {128: ["bf16_d128_bc64_w4", "bf16_d128_bc64_w4_pairs", "bf16_d128_bc64_w4_ks2", "bf16_d128_bc64_w8"],
         64: ["bf16_d64_bc64_w4", "bf16_d64_bc64_w4_pairs", "bf16_d64_bc64_w4_ks2", "bf16_d64_bc64_w8"]}

# (d_k, B, H, Lq, Lk, causal, key-length range or None)
SHAPES = [
    (64, 64, 8, 128, 128, False, None), (64, 32, 8, 256, 256, True, None), (64, 32, 8, 256, 512, False, (64, 512)),
    (64, 16, 8, 512, 512, False, None), (64, 16, 8, 1024, 1024, True, None), (64, 8, 8, 2048, 2048, True, None),
    (64, 64, 8, 512, 512, False, None), (64, 4, 8, 4096, 4096, True, None), (64, 128, 8, 256, 256, True, None),
    (64, 16, 8, 256, 1024, False, (64, 1024)), (64, 64, 8, 128, 256, False, (16, 256)),
    (64, 8, 8, 512, 2048, False, (128, 2048)), (64, 32, 8, 128, 512, False, (64, 512)),
    (64, 8, 8, 1024, 1024, True, None), (64, 16, 8, 2048, 2048, False, None), (64, 2, 8, 4096, 4096, False, None),
    (64, 16, 8, 512, 512, True, None), (64, 1, 8, 8192, 8192, True, None),
    (128, 4, 96, 4096, 4096, True, None), (128, 1, 32, 2048, 2048, True, None), (128, 2, 16, 1024, 1024, False, None),
    (128, 8, 16, 512, 512, True, None), (128, 1, 8, 4096, 4096, True, None), (128, 16, 32, 256, 256, False, None),
    (128, 4, 32, 1024, 1024, True, (256, 1024)), (128, 16, 16, 256, 1024, False, (128, 1024)),
    (128, 4, 32, 1024, 1024, False, (256, 1024)), (128, 4, 16, 512, 512, True, None),
    (128, 2, 32, 1024, 1024, True, None), (128, 1, 16, 2048, 2048, True, None), (128, 1, 64, 2048, 2048, True, None),
    (128, 1, 16, 4096, 4096, False, None), (128, 2, 8, 8192, 8192, True, None), (128, 16, 16, 512, 512, True, None),
    (128, 32, 8, 256, 256, True, None), (64, 2, 80, 256, 256, True, None), (64, 8, 40, 128, 300, False, (64, 300)),
    (128, 8, 40, 128, 512, False, (64, 512)), (128, 1, 32, 2048, 2048, True, None), (128, 4, 16, 2048, 2048, True, None),
    (64, 32, 16, 1024, 1024, True, None), (64, 64, 16, 512, 512, False, None), (64, 4, 32, 2048, 2048, False, None),
]
QUICK = [SHAPES[i] for i in (0, 1, 2, 18, 19, 22, 28)]


def time_shape(torch, sdpa, d, B, H, Lq, Lk, causal, kl, rounds=3):
    import numpy as np
    g = torch.Generator(device="cuda").manual_seed(1)
    q = torch.randn(B, H, Lq, d, device="cuda", generator=g).bfloat16()
    k = torch.randn(B, H, Lk, d, device="cuda", generator=g).bfloat16()
    v = torch.randn(B, H, Lk, d, device="cuda", generator=g).bfloat16()
    tkl = torch.randint(kl[0], kl[1] + 1, (B,), device="cuda", generator=g, dtype=torch.int32) if kl else None
    per_set = 2 * (q.numel() * 2 + k.numel() * 2)
    nsets = max(1, min(8, -(-(1 << 30) // per_set)))
    sets = [(q, k, v, torch.empty_like(q), torch.empty(B, H, Lq, device="cuda"))] + [
        (q.clone(), k.clone(), v.clone(), torch.empty_like(q), torch.empty(B, H, Lq, device="cuda"))
        for _ in range(nsets - 1)]
    s = torch.cuda.current_stream()

    def call(tile, i):
        a = sets[i % nsets]
        sdpa.forward_ex(a[0], a[1], a[2], causal=causal, key_lens=tkl, out=a[3], lse=a[4], stream=s, tile=tile)

    for tile in TILES[d]:
        call(tile, 0)
    torch.cuda.synchronize()
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < 0.2:
        for _ in range(10):
            call(TILES[d][0], i)
            i += 1
        torch.cuda.synchronize()
    per = (time.perf_counter() - t0) / i
    n = int(max(10, min(200, 0.02 / per)))
    meas = {t: [] for t in TILES[d]}
    for _ in range(rounds):
        for tile in TILES[d]:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for j in range(n):
                call(tile, j)
            e1.record(s)
            torch.cuda.synchronize()
            meas[tile].append(e0.elapsed_time(e1) / n * 1e3)
    chosen = sdpa.kernel_name(q, k, causal, kl is not None)
    del sets, q, k, v
    torch.cuda.empty_cache()
    return {t: float(np.median(m)) for t, m in meas.items()}, chosen


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--quick", action="store_true", help="seven shapes only")
    args = ap.parse_args()
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    torch.cuda.set_device(0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print("| d_k | B·H | Lq × Lk | causal | key lengths | items per CU | steps | "
          + " | ".join(t.split("_", 2)[2] for t in TILES[128]) + " | chosen, µs |")
    print("|---|---|---|---|---|---|---|" + "---|" * len(TILES[128]) + "---|")
    off = []
    for (d, B, H, Lq, Lk, causal, kl) in (QUICK if args.quick else SHAPES):
        res, chosen = time_shape(torch, sdpa, d, B, H, Lq, Lk, causal, kl)
        items = B * H * ((Lq + 127) // 128)
        steps = ((min(Lq, Lk) if causal else Lk) + 63) // 64
        best = min(res.values())
        rel = res[chosen] / best - 1
        cells = [f"{res[t]:.1f}" if t in res else "—" for t in
                 [t.replace("d128", f"d{d}") for t in TILES[128]]]
        mark = f" (best {best:.1f})" if rel >= 0.02 else ""
        off.append(rel)
        klt = f"{kl[0]}–{kl[1]}" if kl else "—"
        print(f"| {d} | {B}·{H} | {Lq} × {Lk} | {'yes' if causal else 'no'} | {klt} | {items / cus:.3g} | {steps} | "
              + " | ".join(cells) + f" | {chosen.split('_', 2)[2]} {res[chosen]:.1f}{mark} |", flush=True)
    within = sum(r < 0.02 for r in off)
    print(f"\nThe choice is within 2% of the fastest tile on {within} of {len(off)} shapes "
          f"(worst {100 * max(off):.1f}% off).", flush=True)


if __name__ == "__main__":
    sys.exit(main())
