#!/usr/bin/env python3
"""rocprofv3 harness: kernel time, matrix-core (MFMA) utilisation and HBM
traffic of the attention kernels, written as short summaries under
``profiles/``.

    python rocprof_harness.py [--workload NAME ...] [--leg forward|backward|decode|forward_ex]
                              [--passes trace,mfma,fetch,write] [--raw DIR] [--out DIR]

Runs where the GPU is.  Every pass is one ``rocprofv3`` run of ``bench.py``
(the program straight after ``--``, started as a child process of this
script, which itself never touches the GPU), with the bench legs that are
not being profiled switched off:

* ``trace``: ``--kernel-trace --stats``; per-kernel average duration over
  all dispatches and over the timed ones (the last ``--steps``), next to the
  HIP-event average that bench.py itself prints for the same command;
* ``mfma``: one counter pass, ``SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES
  SQ_INSTS_MFMA GRBM_GUI_ACTIVE``: the share of SIMD cycles with a busy
  matrix core, the shader clock the chip held (GRBM_GUI_ACTIVE per XCD over
  the traced duration), and the MFMA flops executed (32*32*16*2 per
  ``v_mfma_f32_32x32x16_bf16``) against the algorithmic flops;
* ``fetch`` / ``write``: ``FETCH_SIZE`` and ``WRITE_SIZE`` (KiB per dispatch)
  in separate passes (rocprofv3 does not split counters over passes).  The
  same runs copy 1 GiB device to device (``bench.py --copy-calibration-mib
  1024``); the counter's reading for the largest copy dispatches gives the
  scale factor to bytes (``calibration_factor``), so that HBM bytes per
  launch = counter KiB * 1024 * factor.

Raw rocprofv3 output (CSV files, tens of MB for a trace) goes to ``--raw``
(default: a fresh directory under the system temp directory) and is not
kept; only the summaries go to ``--out`` (default ``profiles/``).  The fp32
workloads get no MFMA pass (their kernel uses no matrix cores).  The forward
traffic summary carries ``kernel_source_sha256`` and
``traffic_bytes_per_launch`` lines, which bench.py reads for its roofline.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import shlex
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
MFMA_FLOPS = 32 * 32 * 16 * 2            # one v_mfma_f32_32x32x16_bf16
MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE"]
COPY_MIB = 1024
# kernel-name patterns of each leg
LEG_KERNELS = {"forward": r"fwd_bf16_kernel|fwd_f32", "forward_ex": r"fwd_bf16_kernel|fwd_f32",
               "backward": r"bwd_", "decode": r"decode_kernel|decode_combine|fwd_bf16_kernel"}


# ---------------------------------------------------------------- commands

def bench_args(workload: str, leg: str, steps: int, warmup: int, extra=()) -> list[str]:
    """bench.py arguments that run `leg` of `workload` and nothing else."""
    a = ["bench.py", "--steps", str(steps), "--warmup", str(warmup), "--no-cpu-baseline",
         "--no-vendor-gemm", "--no-configs"]
    if leg == "decode":
        # the decode leg runs after a minimal main leg on the smallest workload
        a += ["--workload", "toy_f32", "--decode-workload", workload, "--no-backward", "--no-forward-ex",
              "--no-decode-forward"]
    else:
        a += ["--workload", workload, "--decode-workload", "none"]
        if leg != "backward":
            a.append("--no-backward")
        if leg != "forward_ex":
            a.append("--no-forward-ex")
    return a + list(extra)


def pass_command(kind: str, workload: str, leg: str, raw: str, steps: int, warmup: int) -> tuple[list[str], str]:
    """(argv, output directory) of one rocprofv3 pass."""
    tag = f"{kind}_{leg}_{workload}"
    out = os.path.join(raw, tag)
    if kind == "trace":
        prof = ["--kernel-trace", "--stats"]
        b = bench_args(workload, leg, steps, warmup, ["--clock-settle", "0.1"])
    elif kind == "mfma":
        prof = ["--pmc", *MFMA_COUNTERS]
        b = bench_args(workload, leg, 3, 1, ["--clock-settle", "0.05"])
    elif kind in ("fetch", "write"):
        prof = ["--pmc", "FETCH_SIZE" if kind == "fetch" else "WRITE_SIZE"]
        b = bench_args(workload, leg, 3, 1, ["--clock-settle", "0.05", "--copy-calibration-mib", str(COPY_MIB)])
    else:
        raise ValueError(kind)
    argv = ["rocprofv3", *prof, "--output-format", "csv", "-d", out, "-o", "run", "--", "python3", *b]
    return argv, out


# ---------------------------------------------------------------- parsing

def read_csv(path: str) -> list[dict]:
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def find(dirpath: str, suffix: str) -> str | None:
    for base, _, files in os.walk(dirpath):
        for fn in sorted(files):
            if fn.endswith(suffix):
                return os.path.join(base, fn)
    return None


def kernel_stats(rows: list[dict], pattern: str) -> list[dict]:
    """Rows of *_kernel_stats.csv whose kernel name matches."""
    return [r for r in rows if re.search(pattern, r["Name"])]


def dispatch_durations(trace_rows: list[dict], pattern: str) -> dict[str, list[int]]:
    """Kernel name -> durations (ns) of its dispatches in dispatch order."""
    out: dict[str, list[tuple[int, int]]] = {}
    for r in trace_rows:
        if not re.search(pattern, r["Kernel_Name"]):
            continue
        d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        out.setdefault(r["Kernel_Name"], []).append((int(r["Dispatch_Id"]), d))
    return {k: [d for _, d in sorted(v)] for k, v in out.items()}


def counters_by_dispatch(rows: list[dict]) -> dict[int, dict]:
    """Dispatch id -> {"kernel": name, counter: value (summed over rows)}."""
    out: dict[int, dict] = {}
    for r in rows:
        did = int(r["Dispatch_Id"])
        e = out.setdefault(did, {"kernel": r["Kernel_Name"]})
        name = r["Counter_Name"]
        e[name] = e.get(name, 0.0) + float(r["Counter_Value"])
    return out


def calibration(disp: dict[int, dict], counter: str, nbytes: int) -> tuple[float, float]:
    """(factor, counter KiB) from the copy dispatches: the mean reading of the
    three largest copies; factor = bytes moved / (KiB read * 1024)."""
    vals = sorted((e[counter] for e in disp.values() if "copyBuffer" in e["kernel"] and counter in e),
                  reverse=True)[:3]
    if not vals:
        raise RuntimeError(f"no copy dispatch with {counter} in the run")
    kib = sum(vals) / len(vals)
    return nbytes / (kib * 1024.0), kib


def agent_info(dirpath: str) -> dict:
    p = find(dirpath, "_agent_info.csv")
    info = {"simds": 1024, "xcds": 8}
    if p:
        for r in read_csv(p):
            if r.get("Agent_Type") == "GPU":
                info = {"simds": int(r["Simd_Count"]), "xcds": int(r["Num_Xcc"]), "name": r.get("Name")}
    return info


def bench_json(stdout: str) -> dict | None:
    for line in stdout.splitlines()[::-1]:
        line = line.strip()
        if line.startswith("{") and '"metric"' in line:
            return json.loads(line)
    return None


# ---------------------------------------------------------------- running

def run_pass(argv: list[str], log: str, timeout: int) -> str:
    print(f"[harness] running: {' '.join(shlex.quote(a) for a in argv)}", flush=True)
    t0 = time.time()
    with open(log, "w") as f:
        r = subprocess.run(argv, cwd=ROOT, stdout=subprocess.PIPE, stderr=f, text=True, timeout=timeout)
    print(f"[harness] pass done in {time.time() - t0:.1f} s (rc {r.returncode})", flush=True)
    # rocprofv3 can end with a segmentation fault after the program finished
    # and its files are complete; the bench line printed is the check
    if bench_json(r.stdout) is None:
        tail = open(log, errors="replace").read().splitlines()[-30:]
        print("\n".join(["[harness] last lines of the pass's log:"] + tail), flush=True)
        raise RuntimeError(f"pass failed (rc {r.returncode}); log {log}")
    return r.stdout


_RAW_SHOWN = "$RAW"


def cmd_str(argv: list[str]) -> str:
    """The command as run, with the raw-output directory shown as $RAW (a
    temporary directory of the run)."""
    out = []
    for i, a in enumerate(argv):
        if i > 0 and argv[i - 1] == "-d":
            a = os.path.join(_RAW_SHOWN, os.path.basename(a))
        out.append(a if a.startswith("$RAW") else shlex.quote(a))
    return " ".join(out)


# Sources behind each leg's kernels.  The forward set is bench.py's own
# (bench.py trusts a forward traffic summary only while that hash matches);
# the decode leg may also run the forward kernel.
LEG_SOURCES = {
    "backward": ["transformer_scaled_dot_sdpa_amd/csrc/sdpa_bwd_bf16.hip",
                 "transformer_scaled_dot_sdpa_amd/csrc/sdpa_bwd_f32.hip",
                 "transformer_scaled_dot_sdpa_amd/csrc/bf16_common.h"],
    "decode": ["transformer_scaled_dot_sdpa_amd/csrc/sdpa_decode_bf16.hip"],
}


def kernel_source_hash(leg: str = "forward") -> str:
    """bench.py's hash of the forward kernel sources; for the backward and
    decode legs the hash of their own kernel sources (decode: followed by
    the forward sources, whose kernel it runs for many slices)."""
    sys.path.insert(0, ROOT)
    import bench
    if leg not in LEG_SOURCES:
        return bench.kernel_source_hash()
    h = hashlib.sha256()
    for rel in LEG_SOURCES[leg] + (bench.KERNEL_SOURCES if leg == "decode" else []):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------- summaries

def write_trace(out_dir, workload, leg, argv, raw, stdout, steps):
    stats = read_csv(find(raw, "_kernel_stats.csv"))
    trace = read_csv(find(raw, "_kernel_trace.csv"))
    pat = LEG_KERNELS[leg]
    js = bench_json(stdout)
    lines = [f"# Kernel time: {workload} ({leg})", "",
             "Command (from the repository root, on one MI355X; written by rocprof_harness.py):", "",
             "```", cmd_str(argv), "```", "", "`run_kernel_stats.csv`:", "",
             "| kernel | calls | avg ns | min ns | max ns | stddev |", "|---|---|---|---|---|---|"]
    for r in kernel_stats(stats, pat):
        lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                     f"{r['MaxNs']} | {float(r['StdDev']):.0f} |")
    durs = dispatch_durations(trace, pat)
    lines += ["", f"From `run_kernel_trace.csv`, the last {steps} dispatches of each kernel (the timed steps):", ""]
    summary = {}
    for name, d in durs.items():
        last = d[-steps:] if len(d) >= steps else d
        avg = sum(last) / len(last)
        summary[name] = avg
        lines.append(f"- `{name}`: average {avg:.0f} ns, min {min(last)} ns, max {max(last)} ns "
                     f"({len(last)} dispatches)")
    if js is not None:
        if leg == "forward":
            roof = js["roofline"]
            how = roof.get("timing", "HIP events around each timed launch")
            lines += ["", f"Same command, bench.py's own timing ({how}): "
                          f"{roof['kernel_avg_ms'] * 1e6:.0f} ns per launch -> {roof['achieved']:.1f} "
                          f"{roof['unit']} ({100 * roof['frac']:.1f}% of {roof['peak']:.0f}, {roof['bound']} bound)."]
        elif leg == "backward" and "backward" in js:
            lines += ["", f"Same command, HIP events inside bench.py: {js['backward']['ms_per_call'] * 1e6:.0f} ns "
                          f"per backward call ({js['backward']['roofline']['achieved']:.1f} TFLOP/s at 10*d_k "
                          "flops per valid pair)."]
        elif leg == "decode" and workload in js.get("decode", {}):
            d = js["decode"][workload]
            lines += ["", f"Same command, bench.py's own timing ({d.get('timing', 'HIP events')}, "
                          f"{d['steps']} calls): {d['us_per_call']:.1f} us per decode call "
                          f"({d['roofline']['achieved']:.0f} GB/s of algorithmic bytes)."]
        elif leg == "forward_ex" and "forward_ex" in js:
            f = js["forward_ex"]
            lines += ["", "Same command, HIP events inside bench.py: " + ", ".join(
                f"{k} {v['us_per_call']:.1f} us" for k, v in f.items() if isinstance(v, dict))]
    lines += ["", "bench.py's own figure comes from the same profiled run; the kernel trace adds work per "
                  "dispatch, which matters for calls of a few microseconds (there the unprofiled bench.py line is "
                  "the one to quote) and not for kernels of a millisecond.",
              "", f"kernel_source_sha256: {kernel_source_hash(leg)}", ""]
    name = {"forward": "kernel_stats", "backward": "backward_trace", "decode": "decode_trace",
            "forward_ex": "forward_ex"}[leg]
    path = os.path.join(out_dir, f"{workload}_{name}.md")
    open(path, "w").write("\n".join(lines))
    print(f"[harness] wrote {path}", flush=True)
    return summary, js


def write_mfma(out_dir, workload, leg, argv, raw, trace_avg_ns):
    disp = counters_by_dispatch(read_csv(find(raw, "_counter_collection.csv")))
    info = agent_info(raw)
    pat = LEG_KERNELS[leg]
    lines = [f"# MFMA utilisation: {workload} ({leg})", "",
             "One counter pass, from the repository root on one MI355X (written by rocprof_harness.py):", "",
             "```", cmd_str(argv), "```", "",
             f"GPU: {info['simds']} SIMDs in {info['xcds']} XCDs.  Per kernel, mean over its dispatches "
             "(GRBM_GUI_ACTIVE sums the XCDs):", "",
             "| kernel | dispatches | GRBM_GUI_ACTIVE | SQ_BUSY_CYCLES | SQ_INSTS_MFMA | SQ_VALU_MFMA_BUSY_CYCLES | "
             "MFMA busy | clock | MFMA flops executed |", "|---|---|---|---|---|---|---|---|---|"]
    by_kernel: dict[str, list[dict]] = {}
    for e in disp.values():
        if re.search(pat, e["kernel"]):
            by_kernel.setdefault(e["kernel"], []).append(e)
    result = {}
    for name, es in by_kernel.items():
        mean = {c: sum(e.get(c, 0.0) for e in es) / len(es) for c in MFMA_COUNTERS}
        cycles = mean["GRBM_GUI_ACTIVE"] / info["xcds"]
        busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (info["simds"] * cycles) if cycles else 0.0
        avg = trace_avg_ns.get(name) if trace_avg_ns else None
        # GRBM_GUI_ACTIVE also counts the counter pass's fixed busy cycles per
        # dispatch (tens of microseconds' worth), so the clock estimate only
        # holds for kernels far longer than that
        clock = f"{cycles / avg:.2f} GHz" if avg and avg > 200e3 else "n/a"
        flops = mean["SQ_INSTS_MFMA"] * MFMA_FLOPS
        result[name] = {"busy": busy, "cycles": cycles, "flops": flops}
        lines.append(f"| `{name}` | {len(es)} | {mean['GRBM_GUI_ACTIVE']:.4g} | {mean['SQ_BUSY_CYCLES']:.4g} | "
                     f"{mean['SQ_INSTS_MFMA']:.4g} | {mean['SQ_VALU_MFMA_BUSY_CYCLES']:.4g} | {100 * busy:.1f}% | "
                     f"{clock} | {flops:.4g} |")
    lines += ["", "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE per XCD).  The clock is "
                  "GRBM_GUI_ACTIVE per XCD over the kernel's average duration in the trace pass; 2.4 GHz is the "
                  "peak engine clock behind the 2.5 PFLOP/s figure, so busy x clock / 2.4 GHz approximates "
                  "the share of peak the kernel reaches (n/a for kernels under 200 us, where the counter "
                  "pass's own busy cycles dominate GRBM_GUI_ACTIVE).  Executed flops count every issued "
                  "32x32x16 bf16 MFMA (masked halves of boundary tiles included).", ""]
    path = os.path.join(out_dir, f"{workload}_{'mfma_util' if leg == 'forward' else leg + '_mfma_util'}.md")
    open(path, "w").write("\n".join(lines))
    print(f"[harness] wrote {path}", flush=True)
    return result


def write_traffic(out_dir, workload, leg, cmds, raws, algorithmic_bytes):
    pat = LEG_KERNELS[leg]
    rows = {}
    factors = {}
    for kind, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        disp = counters_by_dispatch(read_csv(find(raws[kind], "_counter_collection.csv")))
        factor, copy_kib = calibration(disp, counter, COPY_MIB << 20)
        factors[counter] = (factor, copy_kib)
        for e in disp.values():
            if re.search(pat, e["kernel"]) and counter in e:
                rows.setdefault(e["kernel"], {}).setdefault(counter, []).append(e[counter])
    lines = [f"# HBM traffic: {workload} ({leg})", "",
             "Two counter passes (one counter each), from the repository root on one MI355X "
             "(written by rocprof_harness.py):", "", "```", cmd_str(cmds["fetch"]), cmd_str(cmds["write"]), "```", "",
             f"Calibration: the same runs copy {COPY_MIB} MiB device to device (`__amd_rocclr_copyBuffer`); "
             "the mean reading of the three largest copy dispatches is " +
             ", ".join(f"{c} = {kib:.0f} KiB" for c, (_, kib) in factors.items()) +
             f" for {COPY_MIB << 10} KiB moved each way, so the counts are scaled by " +
             " and ".join(f"{f:.4f} ({c})" for c, (f, _) in factors.items()) + ".", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes / dispatch |",
             "|---|---|---|---|---|"]
    total = 0.0
    main_bytes = None
    for name, cs in rows.items():
        f = sum(cs.get("FETCH_SIZE", [0])) / max(1, len(cs.get("FETCH_SIZE", [])))
        w = sum(cs.get("WRITE_SIZE", [0])) / max(1, len(cs.get("WRITE_SIZE", [])))
        b = f * 1024 * factors["FETCH_SIZE"][0] + w * 1024 * factors["WRITE_SIZE"][0]
        n = max(len(cs.get("FETCH_SIZE", [])), len(cs.get("WRITE_SIZE", [])))
        lines.append(f"| `{name}` | {n} | {f:.0f} | {w:.0f} | {b:.4g} |")
        total += b
        main_bytes = b if main_bytes is None or b > main_bytes else main_bytes
    if algorithmic_bytes:
        lines += ["", f"Algorithmic bytes per call (Q, valid K/V rows, O once, lse once): {algorithmic_bytes:.4g}; "
                      f"measured / algorithmic: {total / algorithmic_bytes:.3f} (all kernels of the call)."]
    lines += ["", f"kernel_source_sha256: {kernel_source_hash(leg)}", f"traffic_bytes_per_launch: {total:.6g}", ""]
    path = os.path.join(out_dir, f"{workload}_{'hbm_traffic' if leg == 'forward' else leg + '_hbm_traffic'}.md")
    open(path, "w").write("\n".join(lines))
    print(f"[harness] wrote {path}", flush=True)
    return total


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", action="append", default=None)
    ap.add_argument("--leg", default="forward", choices=list(LEG_KERNELS))
    ap.add_argument("--passes", default="trace,mfma,fetch,write")
    ap.add_argument("--raw", default=None, help="directory for rocprofv3's raw output (default: a temp dir)")
    ap.add_argument("--out", default="profiles")
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--timeout", type=int, default=300, help="seconds per rocprofv3 pass")
    ap.add_argument("--dry-run", action="store_true", help="print the commands only")
    args = ap.parse_args()
    workloads = args.workload or ["large_causal_d128"]
    passes = args.passes.split(",")
    os.chdir(ROOT)
    if args.raw is None:
        args.raw = tempfile.mkdtemp(prefix="rocprof_harness_")
    os.makedirs(args.raw, exist_ok=True)
    os.makedirs(args.out, exist_ok=True)
    print(f"[harness] raw output under {args.raw}", flush=True)
    for wl in workloads:
        cmds, raws = {}, {}
        for kind in passes:
            cmds[kind], raws[kind] = pass_command(kind, wl, args.leg, args.raw, args.steps, args.warmup)
        if args.dry_run:
            for kind in passes:
                print(cmd_str(cmds[kind]))
            continue
        trace_avg, js = {}, None
        if "trace" in passes:
            out = run_pass(cmds["trace"], raws["trace"] + ".log", args.timeout)
            trace_avg, js = write_trace(args.out, wl, args.leg, cmds["trace"], raws["trace"], out, args.steps)
        fp32 = wl.startswith("toy")
        if "mfma" in passes and not fp32:
            run_pass(cmds["mfma"], raws["mfma"] + ".log", args.timeout)
            write_mfma(args.out, wl, args.leg, cmds["mfma"], raws["mfma"], trace_avg)
        if "fetch" in passes and "write" in passes:
            out = run_pass(cmds["fetch"], raws["fetch"] + ".log", args.timeout)
            run_pass(cmds["write"], raws["write"] + ".log", args.timeout)
            jsb = bench_json(out)
            alg = None
            if jsb is not None:
                if args.leg == "decode" and wl in jsb.get("decode", {}):
                    alg = jsb["decode"][wl]["roofline"]["algorithmic_bytes_per_call"]
                elif args.leg in ("forward", "forward_ex"):
                    alg = jsb["roofline"].get("algorithmic_bytes_per_launch")
            write_traffic(args.out, wl, args.leg, cmds, raws, alg)
    print("[harness] done", flush=True)


if __name__ == "__main__":
    main()
