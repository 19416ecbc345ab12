"""Build the HIP library ``lib/libsdpa_mi355x.so`` for gfx950 with hipcc.

Usage: ``python -m transformer_scaled_dot_sdpa_amd.build [--verbose]``.
Sources are compiled in parallel into ``_build/`` and linked in place, so the
shared library sits inside the package tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libsdpa_mi355x.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-result",
    # packed fp32 VALU instructions stay disabled in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# extra compiler flags (e.g. -D switches for tuning builds)
EXTRA = os.environ.get("SDPA_HIPCC_EXTRA", "").split()


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA, "-c", src, "-o", obj]
    if verbose and src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    return obj


# Global-memory instructions each forward kernel may contain: Q fragment
# loads (16 bytes per k-step pair), two key-length loads (the item's, and the
# ranking of batches by length), O stores (16 bytes per lane, whole rows
# staged through LDS: d_v / 16 per wavefront) and one lse store.  (K, V and
# an additive mask come in through buffer loads, which this does not count.)  Anything else -- a flat
# access, or more global accesses than these -- means an LDS access was
# compiled as a global one (an LDS address used as a global address faults
# the GPU), so the build refuses it.
_FWD_KERNEL = re.compile(r"^(_ZN4sdpa12_GLOBAL__N_115fwd_bf16_kernelILi(\d+)ELi(\d+)ELi\d+ELi\d+ELi\d+ELb([01])ELb([01])ELb([01])E\w*):",
                         re.M)


def audit_forward_isa(src: str | None = None) -> int:
    """Compile the forward kernels to gfx950 assembly and check every
    instance's global and flat memory instructions against the expected
    set; returns the number of kernels checked, raises on a mismatch."""
    src = src or os.path.join(CSRC, "sdpa_fwd_bf16.hip")
    os.makedirs(BUILD, exist_ok=True)
    asm = os.path.join(BUILD, "sdpa_fwd_bf16.audit.s")
    cmd = [HIPCC, *COMMON, *EXTRA, "--cuda-device-only", "-S", src, "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    text = open(asm).read()
    bad, n = [], 0
    for m in _FWD_KERNEL.finditer(text):
        name, d, dv, lens = m.group(1), int(m.group(2)), int(m.group(3)), m.group(5) == "1"
        body = text[m.end():text.index(".Lfunc_end", m.end())]
        ops = re.findall(r"^\s+((?:global|flat)_\w+)", body, re.M)
        expect = {"global_load_dwordx4": d // 16, "global_store_dwordx4": dv // 16, "global_store_dword": 1}
        if lens:
            expect["global_load_dword"] = 2
        got = {}
        for op in ops:
            got[op] = got.get(op, 0) + 1
        if got != expect:
            bad.append(f"{name}: {got} (expected {expect})")
        n += 1
    if n == 0:
        raise RuntimeError("no forward kernel found in the assembly")
    if bad:
        raise RuntimeError("forward kernels with unexpected global/flat memory instructions:\n" + "\n".join(bad))
    return n


def build(verbose: bool = False, out: str | None = None, build_dir: str | None = None) -> str:
    """Compile every source under ``csrc/`` and link the shared library
    (to ``out``, default ``lib/libsdpa_mi355x.so``)."""
    global BUILD
    if build_dir:
        BUILD = build_dir
    lib = out or LIB
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        audit = ex.submit(audit_forward_isa)
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
        audit.result()
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    # A kernel whose host stub was dropped links "successfully" but leaves
    # an undefined symbol behind; refuse such a library.
    nm = subprocess.run(["nm", "-C", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.strip() for l in nm.stdout.splitlines() if "sdpa::" in l]
    if missing:
        os.remove(tmp)
        raise RuntimeError("library has undefined kernel symbols:\n" + "\n".join(missing))
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if not a.startswith("--")]
    print(build(verbose="--verbose" in sys.argv, out=args[0] if args else None,
                build_dir=args[1] if len(args) > 1 else None))
