"""fp64 CPU oracle for scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
this package imports nothing from the product path.

Two independent routes compute the same thing:

* :func:`sdpa` / :func:`sdpa_rows` call the plain C routines in
  ``sdpa_oracle.c`` (fp64, two passes per row, no tiling), built with gcc the
  first time they are needed;
* :mod:`oracle.brute` is a pure-Python per-query loop for tiny shapes.

Both follow "Aufmerksamkeit ist alles, was Sie brauchen", section 3.2.1,
eq. (1), and the proof section (証明) of the formula page
"トランスフォーマーの注意機構"; the header of ``sdpa_oracle.c`` gives the
step-by-step citations and the masking rules.

Parity status: ``sdpa``, ``sdpa_rows`` and ``brute.attention`` are all pinned
by ``tests/test_oracle_pins.py`` (values printed on the formula page,
closed-form limits and invariants, brute force on tiny shapes), and
``tests/test_oracle_mutants.py`` shows that plausible mistakes planted in a
copy of ``sdpa_oracle.c`` fail those pins.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "sdpa_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle_sdpa.so")

_DTYPE_F64, _DTYPE_F32, _DTYPE_BF16 = 0, 1, 2


def compile_source(src: str, out_path: str) -> str:
    """Compile one oracle C source into a shared library with gcc."""
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    tmp = out_path + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def build(force: bool = False) -> str:
    """Compile ``sdpa_oracle.c`` into ``_build/liboracle_sdpa.so``."""
    if (not force and os.path.exists(_LIB_PATH)
            and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(SOURCE)):
        return _LIB_PATH
    return compile_source(SOURCE, _LIB_PATH)


def _as_input(x, bf16: bool):
    """Return (contiguous array, dtype code).  bf16 data is passed as uint16 bits."""
    x = np.asarray(x)
    if bf16:
        if x.dtype != np.uint16:
            raise TypeError("bf16 inputs must be given as uint16 bit patterns")
        return np.ascontiguousarray(x), _DTYPE_BF16
    if x.dtype == np.float64:
        return np.ascontiguousarray(x), _DTYPE_F64
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), _DTYPE_F32
    raise TypeError(f"unsupported oracle input dtype {x.dtype}")


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, L, d_k]")
    B, H, Lq, d = q.shape
    if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    return B, H, Lq, k.shape[2], d


def _key_lens_arg(key_lens, B):
    if key_lens is None:
        return None, None
    kl = np.ascontiguousarray(np.asarray(key_lens, dtype=np.int32))
    if kl.shape != (B,):
        raise ValueError("key_lens must have shape [B]")
    return kl, kl.ctypes.data


class Oracle:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_sdpa.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64,
                                    i32, vp, dbl, vp, vp, i32]
        lib.oracle_sdpa.restype = i32
        lib.oracle_sdpa_rows.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64,
                                         i32, vp, dbl, vp, i64, vp, vp, i32]
        lib.oracle_sdpa_rows.restype = i32
        lib.oracle_sdpa_bwd.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, i64,
                                        i32, vp, dbl, vp, vp, vp, i32]
        lib.oracle_sdpa_bwd.restype = i32
        lib.oracle_sdpa_ex.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, i64,
                                       i32, vp, dbl, vp, vp, vp, i32]
        lib.oracle_sdpa_ex.restype = i32
        self._lib = lib
        self.path = lib_path

    def sdpa(self, q, k, v, causal: bool = False, key_lens=None,
             tau: float | None = None, bf16: bool = False, nthreads: int = 0):
        """All rows of softmax(q k^T / tau) v per (b, h), in fp64.

        q: [B, H, Lq, d]; k, v: [B, H, Lk, d]; float64, float32, or
        (``bf16=True``) uint16 bf16 bit patterns.  ``tau`` defaults to sqrt(d).
        Returns ``(out[B, H, Lq, d] float64, lse[B, H, Lq] float64)``.
        """
        q, dt = _as_input(q, bf16)
        k, dtk = _as_input(k, bf16)
        v, dtv = _as_input(v, bf16)
        if not (dt == dtk == dtv):
            raise TypeError("q, k, v must share one dtype")
        B, H, Lq, Lk, d = _check_shapes(q, k, v)
        _kl, kl_ptr = _key_lens_arg(key_lens, B)
        out = np.empty((B, H, Lq, d), dtype=np.float64)
        lse = np.empty((B, H, Lq), dtype=np.float64)
        rc = self._lib.oracle_sdpa(q.ctypes.data, k.ctypes.data, v.ctypes.data, dt,
                                   B, H, Lq, Lk, d, int(bool(causal)), kl_ptr,
                                   float(tau) if tau is not None else 0.0,
                                   out.ctypes.data, lse.ctypes.data, int(nthreads))
        if rc != 0:
            raise RuntimeError(f"oracle_sdpa failed with code {rc}")
        return out, lse

    def sdpa_rows(self, q, k, v, rows, causal: bool = False, key_lens=None,
                  tau: float | None = None, bf16: bool = False, nthreads: int = 0):
        """Selected rows only; ``rows`` are flat indices (b * H + h) * Lq + i.

        Returns ``(out[n, d] float64, lse[n] float64)`` in the order of ``rows``.
        """
        q, dt = _as_input(q, bf16)
        k, dtk = _as_input(k, bf16)
        v, dtv = _as_input(v, bf16)
        if not (dt == dtk == dtv):
            raise TypeError("q, k, v must share one dtype")
        B, H, Lq, Lk, d = _check_shapes(q, k, v)
        _kl, kl_ptr = _key_lens_arg(key_lens, B)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows.shape[0]
        out = np.empty((n, d), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        rc = self._lib.oracle_sdpa_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data, dt,
                                        B, H, Lq, Lk, d, int(bool(causal)), kl_ptr,
                                        float(tau) if tau is not None else 0.0,
                                        rows.ctypes.data if n else None, n,
                                        out.ctypes.data, lse.ctypes.data, int(nthreads))
        if rc != 0:
            raise RuntimeError(f"oracle_sdpa_rows failed with code {rc}")
        return out, lse


    def sdpa_bwd(self, q, k, v, dout, causal: bool = False, key_lens=None,
                 tau: float | None = None, bf16: bool = False, nthreads: int = 0):
        """Gradients of a loss L with dL/d(out) = ``dout`` ([B, H, Lq, d], same
        dtype as q): returns ``(dq, dk, dv)`` in fp64, shaped like q, k, v."""
        q, dt = _as_input(q, bf16)
        k, dtk = _as_input(k, bf16)
        v, dtv = _as_input(v, bf16)
        dout, dto = _as_input(dout, bf16)
        if not (dt == dtk == dtv == dto):
            raise TypeError("q, k, v, dout must share one dtype")
        B, H, Lq, Lk, d = _check_shapes(q, k, v)
        if dout.shape != q.shape:
            raise ValueError("dout must have the shape of q")
        _kl, kl_ptr = _key_lens_arg(key_lens, B)
        dq = np.empty((B, H, Lq, d), dtype=np.float64)
        dk = np.empty((B, H, Lk, d), dtype=np.float64)
        dv = np.empty((B, H, Lk, d), dtype=np.float64)
        rc = self._lib.oracle_sdpa_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                       dout.ctypes.data, dt, B, H, Lq, Lk, d,
                                       int(bool(causal)), kl_ptr,
                                       float(tau) if tau is not None else 0.0,
                                       dq.ctypes.data, dk.ctypes.data, dv.ctypes.data,
                                       int(nthreads))
        if rc != 0:
            raise RuntimeError(f"oracle_sdpa_bwd failed with code {rc}")
        return dq, dk, dv


    def sdpa_ex(self, q, k, v, causal: bool = False, key_lens=None, tau: float | None = None,
                mask=None, bf16: bool = False, nthreads: int = 0):
        """General form: v of its own width d_v, divisor ``tau`` (default
        sqrt(d_k)), optional additive ``mask`` broadcastable to [B, H, Lq, Lk]
        (any float dtype; -inf drops a key).  Returns ``(out[B, H, Lq, d_v],
        lse[B, H, Lq])`` in fp64."""
        q, dt = _as_input(q, bf16)
        k, dtk = _as_input(k, bf16)
        v, dtv = _as_input(v, bf16)
        if not (dt == dtk == dtv):
            raise TypeError("q, k, v must share one dtype")
        if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
            raise ValueError("q, k, v must be [B, H, L, width]")
        B, H, Lq, d = q.shape
        Lk, dv = k.shape[2], v.shape[3]
        if k.shape != (B, H, Lk, d) or v.shape[:3] != (B, H, Lk):
            raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
        _kl, kl_ptr = _key_lens_arg(key_lens, B)
        m_ptr = None
        if mask is not None:
            mask = np.ascontiguousarray(np.broadcast_to(np.asarray(mask, dtype=np.float64),
                                                        (B, H, Lq, Lk)))
            m_ptr = mask.ctypes.data
        out = np.empty((B, H, Lq, dv), dtype=np.float64)
        lse = np.empty((B, H, Lq), dtype=np.float64)
        rc = self._lib.oracle_sdpa_ex(q.ctypes.data, k.ctypes.data, v.ctypes.data, dt,
                                      B, H, Lq, Lk, d, dv, int(bool(causal)), kl_ptr,
                                      float(tau) if tau is not None else 0.0, m_ptr,
                                      out.ctypes.data, lse.ctypes.data, int(nthreads))
        if rc != 0:
            raise RuntimeError(f"oracle_sdpa_ex failed with code {rc}")
        return out, lse


_lock = threading.Lock()
_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from ``sdpa_oracle.c`` (compiled on first use)."""
    global _default
    with _lock:
        if _default is None:
            _default = Oracle(build())
    return _default


def sdpa(q, k, v, **kw):
    """:meth:`Oracle.sdpa` of the default oracle."""
    return default().sdpa(q, k, v, **kw)


def sdpa_rows(q, k, v, rows, **kw):
    """:meth:`Oracle.sdpa_rows` of the default oracle."""
    return default().sdpa_rows(q, k, v, rows, **kw)


def sdpa_ex(q, k, v, **kw):
    """:meth:`Oracle.sdpa_ex` of the default oracle."""
    return default().sdpa_ex(q, k, v, **kw)


def sdpa_bwd(q, k, v, dout, **kw):
    """:meth:`Oracle.sdpa_bwd` of the default oracle."""
    return default().sdpa_bwd(q, k, v, dout, **kw)
