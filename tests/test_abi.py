"""The C ABI: the library loads and exports every symbol include/sdpa.h
declares (CPU), and argument validation returns the documented statuses
(CPU where no device is needed, GPU otherwise)."""
import ctypes
import os
import re

import pytest

from transformer_scaled_dot_sdpa_amd import binding as b

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "sdpa.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdpa_[a-z_]+)\s*\(", text)))


def test_header_declares_exactly_the_bound_symbols():
    assert declared_functions() == sorted(b.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = b.load_library()
    for name in declared_functions():
        assert getattr(lib, name) is not None, name
    # and the exported dynamic symbols really are C (unmangled) names
    out = os.popen(f"nm -D --defined-only {b.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_binding_sizes_match_header_defines():
    text = open(HEADER, encoding="utf-8").read()

    def define(name):
        m = re.search(rf"#define {name} \(\(size_t\)(\d+)(?: << (\d+))?\)", text)
        assert m, name
        return int(m.group(1)) << int(m.group(2) or 0)

    assert define("SDPA_DECODE_NOALLOC_SCRATCH_BYTES") == b.DECODE_NOALLOC_SCRATCH_BYTES


def test_status_strings():
    for code, name in [(0, "SUCCESS"), (1, "INVALID_VALUE"), (2, "NOT_SUPPORTED"),
                       (3, "HIP_ERROR"), (4, "ALLOC_FAILED")]:
        assert b.status_string(code) == f"SDPA_STATUS_{name}"
    assert b.status_string(99) == "SDPA_STATUS_UNKNOWN"


def test_null_handle_and_pointers_rejected_without_device():
    st = b.sdpa_forward(None, 16, 16, 16, 16, None, 1, 1, 1, 1, 64, 0, None, None)
    assert st == b.INVALID_VALUE
    lib = b.load_library()
    assert lib.sdpa_create(None, 1, 0) == b.INVALID_VALUE
    h = ctypes.c_void_p()
    assert lib.sdpa_create(ctypes.byref(h), 7, 0) == b.INVALID_VALUE
    assert lib.sdpa_destroy(None) == b.SUCCESS
    assert b.sdpa_kernel_name(None, 1, 1, 1, 1, 64, 0, 0) is None
    assert b.sdpa_backward(None, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16,
                           1, 1, 1, 1, 64, 0, None, None) == b.INVALID_VALUE


@pytest.mark.gpu
def test_validation_statuses_on_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    h = b.handle_for(b.DTYPE_BF16, 0)
    x = torch.zeros(2, 2, 64, 128, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros_like(x)
    o = torch.zeros_like(x)
    p = lambda t: t.data_ptr()
    fwd = lambda **kw: b.sdpa_forward(**{**dict(handle=h, q=p(x), k=p(y), v=p(y), out=p(o), lse=None,
                                                 B=2, H=2, Lq=64, Lk=64, d_k=128, causal=0,
                                                 key_lens=None, stream=None), **kw})
    assert fwd() == b.SUCCESS
    torch.cuda.synchronize()
    assert fwd(q=None) == b.INVALID_VALUE
    assert fwd(out=None) == b.INVALID_VALUE
    assert fwd(B=0) == b.INVALID_VALUE
    assert fwd(Lk=-1) == b.INVALID_VALUE
    assert fwd(causal=2) == b.INVALID_VALUE
    assert fwd(out=p(x)) == b.INVALID_VALUE               # out aliases q
    assert fwd(out=p(y) + 256) == b.INVALID_VALUE         # out overlaps k
    assert fwd(d_k=96) == b.NOT_SUPPORTED
    assert fwd(d_k=64, q=p(x) + 2) == b.NOT_SUPPORTED     # misaligned bf16
    assert fwd(B=1 << 30, H=1 << 30) == b.INVALID_VALUE   # element count overflow
    assert b.sdpa_kernel_name(h, 4, 96, 4096, 4096, 128, 1, 0).startswith("bf16_d128")
    hf = b.handle_for(b.DTYPE_FP32, 0)
    xf = torch.zeros(1, 1, 4, 300, device="cuda")
    of = torch.zeros_like(xf)
    assert b.sdpa_forward(hf, p(xf), p(xf), p(xf), p(of), None, 1, 1, 4, 4, 300, 0, None,
                          None) == b.NOT_SUPPORTED
    with pytest.raises(b.SdpaError):
        b.forward(x[..., :96].contiguous(), y[..., :96].contiguous(), y[..., :96].contiguous())


@pytest.mark.gpu
def test_backward_validation_statuses_on_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    h = b.handle_for(b.DTYPE_BF16, 0)
    B, H, L, d = 2, 2, 64, 128
    t = {n: torch.zeros(B, H, L, d, dtype=torch.bfloat16, device="cuda")
         for n in ("q", "k", "v", "out", "dout", "dq", "dk", "dv")}
    lse = torch.zeros(B, H, L, device="cuda")
    delta = torch.zeros_like(lse)
    p = lambda x: x.data_ptr()
    base = dict(handle=h, **{n: p(x) for n, x in t.items()}, lse=p(lse), delta=p(delta),
                B=B, H=H, Lq=L, Lk=L, d_k=d, causal=0, key_lens=None, stream=None)
    bwd = lambda **kw: b.sdpa_backward(**{**base, **kw})
    assert bwd() == b.SUCCESS
    torch.cuda.synchronize()
    for name in ("q", "out", "dout", "lse", "delta", "dq", "dk", "dv"):
        assert bwd(**{name: None}) == b.INVALID_VALUE, name
    assert bwd(Lq=0) == b.INVALID_VALUE
    assert bwd(causal=3) == b.INVALID_VALUE
    assert bwd(dq=p(t["q"])) == b.INVALID_VALUE            # dq aliases q
    assert bwd(dk=p(t["dv"]) + 512) == b.INVALID_VALUE     # dk overlaps dv
    assert bwd(delta=p(lse)) == b.INVALID_VALUE            # delta aliases lse
    assert bwd(d_k=96) == b.NOT_SUPPORTED
    assert bwd(d_k=64, dv=p(t["dv"]) + 2) == b.NOT_SUPPORTED   # misaligned bf16
    assert bwd(B=1 << 30, H=1 << 30) == b.INVALID_VALUE



@pytest.mark.gpu
def test_bf16_slices_of_4gib_rejected():
    """bf16 kernels address one (b, h) slice with 32-bit byte offsets: a key
    slice of 2^32 bytes or more is refused before any launch.  The tensors
    are real allocations of that size (k doubles as v), so no access could
    leave them either way."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    h = b.handle_for(b.DTYPE_BF16, 0)
    d, Lq, Lk = 128, 64, (1 << 24) + 64        # Lk * d * 2 = 2^32 + 16 KiB
    p = lambda t: t.data_ptr()
    small = lambda: torch.zeros(1, 1, Lq, d, dtype=torch.bfloat16, device="cuda")
    big = lambda: torch.empty(1, 1, Lk, d, dtype=torch.bfloat16, device="cuda")
    q, out, dout, dq = small(), small(), small(), small()
    kv = big()
    assert b.sdpa_forward(h, p(q), p(kv), p(kv), p(out), None, 1, 1, Lq, Lk, d, 0, None,
                          None) == b.NOT_SUPPORTED
    with pytest.raises(b.SdpaError):
        b.forward_ex(q, kv, kv)
    lse = torch.zeros(1, 1, Lq, device="cuda")
    delta = torch.zeros_like(lse)
    dk, dv = big(), big()
    assert b.sdpa_backward(h, p(q), p(kv), p(kv), p(out), p(dout), p(lse), p(delta), p(dq), p(dk),
                           p(dv), 1, 1, Lq, Lk, d, 0, None, None) == b.NOT_SUPPORTED
    torch.cuda.synchronize()


def test_missing_library_fails_loudly():
    """With the HIP library absent the binding raises; there is no fallback."""
    import subprocess
    import sys
    code = ("import transformer_scaled_dot_sdpa_amd.binding as b\n"
            "try:\n"
            "    b.load_library()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('loaded')\n")
    env = dict(os.environ, SDPA_MI355X_LIB="/nonexistent/libsdpa_mi355x.so")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], env=env, cwd=root, capture_output=True,
                         text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert "raised:" in out.stdout and "not found" in out.stdout, out.stdout


def test_product_package_does_not_import_the_oracle():
    """The oracle is test infrastructure: importing the package (and its
    binding) must not pull it in."""
    import subprocess
    import sys
    code = ("import sys\n"
            "import transformer_scaled_dot_sdpa_amd, transformer_scaled_dot_sdpa_amd.binding\n"
            "print(sorted(m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "[]", out.stdout
