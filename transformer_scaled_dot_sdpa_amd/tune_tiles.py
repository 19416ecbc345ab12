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

    python -m transformer_scaled_dot_sdpa_amd.tune_tiles --random 40 --seed 7

times shapes drawn at random instead (held out: none of them was used to set
the thresholds), to check that the selector generalises.
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


def random_shapes(n, seed, cus=256):
    """n shapes drawn from a seeded distribution over the selector's inputs:
    d_k 64 or 128, causal or not, key lengths in 40% of the non-causal
    draws, sequence lengths 100-8192 (cross-attention key ranges up to 4x
    the queries), and B·H such that the query blocks number between 1/4 and
    16 per compute unit (log-uniform).  Work is capped at about 2 TFLOP per
    call so that every shape times in well under a second."""
    import numpy as np
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        d = int(rng.choice([64, 128]))
        causal = bool(rng.random() < 0.5)
        Lq = int(round(float(np.exp(rng.uniform(np.log(100), np.log(8192))))))
        Lk = Lq if causal or rng.random() < 0.5 else int(min(8192, round(Lq * float(rng.uniform(0.5, 4.0)))))
        nqb = (Lq + 127) // 128
        items = float(np.exp(rng.uniform(np.log(cus / 4), np.log(16 * cus))))
        bh = max(1, int(round(items / nqb)))
        B = int(rng.choice([b for b in (1, 2, 4, 8, 16, 32) if b <= bh] or [1]))
        H = max(1, int(round(bh / B)))
        kl = None
        if not causal and rng.random() < 0.4 and B > 1:
            lo = int(rng.integers(1, max(2, Lk // 2)))
            kl = (lo, Lk)
        if 4.0 * B * H * Lq * Lk * d / (2 if causal else 1) > 2e12:
            continue
        out.append((d, B, H, Lq, Lk, causal, kl))
    return out


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
    ap.add_argument("--random", type=int, default=0, metavar="N", help="N random (held-out) shapes instead")
    ap.add_argument("--seed", type=int, default=7, help="seed of the random shapes")
    args = ap.parse_args()
    import torch
    import transformer_scaled_dot_sdpa_amd as sdpa
    torch.cuda.set_device(0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print("| d_k | B·H | Lq × Lk | causal | key lengths | items per CU | steps | "
          + " | ".join(t.split("_", 2)[2] for t in TILES[128]) + " | chosen, µs |")
    print("|---|---|---|---|---|---|---|" + "---|" * len(TILES[128]) + "---|")
    off = []
    shapes = random_shapes(args.random, args.seed, cus) if args.random else (QUICK if args.quick else SHAPES)
    for (d, B, H, Lq, Lk, causal, kl) in shapes:
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
    print(f"\nThe choice is within 2% of the fastest tile on {within} of {len(off)} shapes, "
          f"within 5% on {sum(r < 0.05 for r in off)} (worst {100 * max(off):.1f}% off, "
          f"mean {100 * sum(off) / len(off):.2f}%).", flush=True)


if __name__ == "__main__":
    sys.exit(main())
