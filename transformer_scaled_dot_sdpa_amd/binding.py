"""ctypes binding of the C ABI in ``include/sdpa.h``.

Argument marshalling only: tensors are checked and their device pointers and
the current HIP stream are passed to ``sdpa_forward`` / ``sdpa_backward``; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or a call fails, an exception is raised.

PyTorch provides device memory and streams and nothing else.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
# SDPA_MI355X_LIB may point at another build of the same library (tuning runs).
LIB_PATH = os.environ.get("SDPA_MI355X_LIB") or os.path.join(PKG, "lib", "libsdpa_mi355x.so")

SUCCESS, INVALID_VALUE, NOT_SUPPORTED, HIP_ERROR, ALLOC_FAILED = 0, 1, 2, 3, 4
DTYPE_FP32, DTYPE_BF16 = 0, 1

# Every symbol include/sdpa.h declares.
EXPORTED = ("sdpa_create", "sdpa_forward", "sdpa_forward_ex", "sdpa_backward", "sdpa_decode",
            "sdpa_decode_workspace_size", "sdpa_decode_noalloc", "sdpa_destroy", "sdpa_status_string",
            "sdpa_kernel_name")
# the fixed device array of sdpa_decode_noalloc (SDPA_DECODE_NOALLOC_SCRATCH_BYTES)
DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20


class Layout(ctypes.Structure):
    """``sdpa_layout_t``: element strides of batch, head and row."""
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("row", ctypes.c_int64)]


class ForwardDesc(ctypes.Structure):
    """``sdpa_forward_desc_t``."""
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("B", ctypes.c_int), ("H", ctypes.c_int), ("Lq", ctypes.c_int),
                ("Lk", ctypes.c_int), ("d_k", ctypes.c_int), ("d_v", ctypes.c_int),
                ("q_layout", Layout), ("k_layout", Layout), ("v_layout", Layout),
                ("out_layout", Layout), ("causal", ctypes.c_int),
                ("key_lens", ctypes.c_void_p), ("scale", ctypes.c_float),
                ("mask", ctypes.c_void_p), ("mask_layout", Layout), ("tile", ctypes.c_char_p)]


class SdpaError(RuntimeError):
    """A non-success status from the library."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


_lock = threading.Lock()
_lib = None
_handles: dict = {}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(
                    f"HIP library not found at {path}; build it with "
                    "`python -m transformer_scaled_dot_sdpa_amd.build`")
            # torch ships its own HIP runtime under the soname the library
            # links against.  Loaded first, that runtime also serves the
            # library; loaded second, it would come in as another copy of
            # the runtime beside the system one the library pulled in, and
            # the two would not share devices.
            try:
                import torch  # noqa: F401
            except ImportError:
                pass
            lib = ctypes.CDLL(path)
            vp, i32 = ctypes.c_void_p, ctypes.c_int
            lib.sdpa_create.argtypes = [ctypes.POINTER(vp), i32, i32]
            lib.sdpa_create.restype = i32
            lib.sdpa_forward.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                         i32, vp, vp]
            lib.sdpa_forward.restype = i32
            lib.sdpa_forward_ex.argtypes = [vp, ctypes.POINTER(ForwardDesc), vp]
            lib.sdpa_forward_ex.restype = i32
            lib.sdpa_backward.argtypes = [vp] * 11 + [i32] * 6 + [vp, vp]
            lib.sdpa_backward.restype = i32
            lib.sdpa_decode.argtypes = [vp] * 6 + [i32] * 6 + [vp, vp, ctypes.c_size_t, vp]
            lib.sdpa_decode.restype = i32
            lib.sdpa_decode_noalloc.argtypes = [vp] * 6 + [i32] * 6 + [vp, vp]
            lib.sdpa_decode_noalloc.restype = i32
            lib.sdpa_decode_workspace_size.argtypes = [vp] + [i32] * 5
            lib.sdpa_decode_workspace_size.restype = ctypes.c_size_t
            lib.sdpa_destroy.argtypes = [vp]
            lib.sdpa_destroy.restype = i32
            lib.sdpa_status_string.argtypes = [i32]
            lib.sdpa_status_string.restype = ctypes.c_char_p
            lib.sdpa_kernel_name.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32]
            lib.sdpa_kernel_name.restype = ctypes.c_char_p
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().sdpa_status_string(int(status)).decode()


def sdpa_create(dtype: int, device: int) -> int:
    """Raw ``sdpa_create``: returns the handle as an integer."""
    h = ctypes.c_void_p()
    st = load_library().sdpa_create(ctypes.byref(h), int(dtype), int(device))
    if st != SUCCESS:
        raise SdpaError(st, "sdpa_create")
    return h.value


def sdpa_destroy(handle: int) -> None:
    st = load_library().sdpa_destroy(handle)
    if st != SUCCESS:
        raise SdpaError(st, "sdpa_destroy")


def sdpa_forward(handle, q, k, v, out, lse, B, H, Lq, Lk, d_k, causal, key_lens, stream) -> int:
    """Raw ``sdpa_forward`` on integer pointers; returns the status code."""
    return load_library().sdpa_forward(handle, q, k, v, out, lse, int(B), int(H), int(Lq),
                                       int(Lk), int(d_k), int(causal), key_lens, stream)


def sdpa_backward(handle, q, k, v, out, dout, lse, delta, dq, dk, dv, B, H, Lq, Lk, d_k, causal,
                  key_lens, stream) -> int:
    """Raw ``sdpa_backward`` on integer pointers; returns the status code."""
    return load_library().sdpa_backward(handle, q, k, v, out, dout, lse, delta, dq, dk, dv,
                                        int(B), int(H), int(Lq), int(Lk), int(d_k), int(causal),
                                        key_lens, stream)


def sdpa_forward_ex(handle, desc: ForwardDesc, stream) -> int:
    """Raw ``sdpa_forward_ex``; returns the status code."""
    return load_library().sdpa_forward_ex(handle, ctypes.byref(desc), stream)


def sdpa_decode(handle, q, k, v, out, lse, B, H, Lq, Lk, d_k, causal, key_lens, workspace,
                workspace_bytes, stream) -> int:
    """Raw ``sdpa_decode`` on integer pointers; returns the status code."""
    return load_library().sdpa_decode(handle, q, k, v, out, lse, int(B), int(H), int(Lq), int(Lk),
                                      int(d_k), int(causal), key_lens, workspace,
                                      int(workspace_bytes), stream)


def sdpa_decode_noalloc(handle, q, k, v, out, lse, B, H, Lq, Lk, d_k, causal, key_lens, stream) -> int:
    """Raw ``sdpa_decode_noalloc`` on integer pointers; returns the status code."""
    return load_library().sdpa_decode_noalloc(handle, q, k, v, out, lse, int(B), int(H), int(Lq), int(Lk),
                                              int(d_k), int(causal), key_lens, stream)


def sdpa_decode_workspace_size(handle, B, H, Lq, Lk, d_k) -> int:
    return int(load_library().sdpa_decode_workspace_size(handle, int(B), int(H), int(Lq),
                                                         int(Lk), int(d_k)))


def sdpa_kernel_name(handle, B, H, Lq, Lk, d_k, causal, has_key_lens):
    r = load_library().sdpa_kernel_name(handle, int(B), int(H), int(Lq), int(Lk), int(d_k),
                                        int(causal), int(has_key_lens))
    return r.decode() if r is not None else None


def handle_for(dtype: int, device: int) -> int:
    """A cached handle per (dtype, device)."""
    key = (int(dtype), int(device))
    with _lock:
        h = _handles.get(key)
    if h is None:
        h = sdpa_create(dtype, device)
        with _lock:
            _handles[key] = h
    return h


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_FP32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def forward(q, k, v, causal: bool = False, key_lens=None, out=None, lse=None,
            need_lse: bool = True, stream=None):
    """softmax(q k^T / sqrt(d_k)) v for every (batch, head), on the GPU.

    q: [B, H, Lq, d_k]; k, v: [B, H, Lk, d_k]; contiguous CUDA/HIP tensors of
    one dtype (bfloat16 or float32) on one device.  ``key_lens``: int32 [B]
    on the same device, or None.  ``out`` / ``lse`` may be given
    preallocated.  Enqueued on ``stream`` (default: the current stream).
    Returns ``(out, lse)``; ``lse`` is None when ``need_lse`` is False and no
    ``lse`` tensor was given.
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, L, d_k], got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    B, H, Lq, d = q.shape
    if k.shape[:2] != (B, H) or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    Lk = k.shape[2]
    code = _dtype_code(q)
    dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must match q in shape, dtype and device, and be contiguous")
    if lse is None and need_lse:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, Lq) or lse.dtype != torch.float32
                            or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be float32 [B, H, Lq] on q's device")
    kl_ptr = None
    if key_lens is not None:
        if (key_lens.dtype != torch.int32 or key_lens.shape != (B,) or key_lens.device != q.device
                or not key_lens.is_contiguous()):
            raise ValueError("key_lens must be a contiguous int32 [B] tensor on q's device")
        kl_ptr = key_lens.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = sdpa_forward(handle_for(code, dev), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                      out.data_ptr(), lse.data_ptr() if lse is not None else None,
                      B, H, Lq, Lk, d, int(bool(causal)), kl_ptr, stream.cuda_stream)
    if st != SUCCESS:
        raise SdpaError(st, "sdpa_forward")
    return out, lse


def _layout_of(t, name):
    """Strides of a 4-d [B, H, L, width] tensor view (last dimension contiguous)."""
    if t.dim() != 4:
        raise ValueError(f"{name} must be a 4-d [B, H, L, width] view")
    sb, sh, sl, st = t.stride()
    if st != 1 and t.shape[3] > 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    return Layout(sb, sh, sl)


def forward_ex(q, k, v, causal: bool = False, key_lens=None, scale=None, mask=None, out=None,
               lse=None, need_lse: bool = True, stream=None, tile=None):
    """General forward: ``q``, ``k`` ([.., d_k]) and ``v`` ([.., d_v]) are
    [B, H, L, width] views with any strides whose last dimension is
    contiguous -- e.g. ``x.view(B, L, H, d).transpose(1, 2)`` for the
    head-interleaved [B, L, H*d] layout.  ``scale`` multiplies q.k (default
    1/sqrt(d_k)); ``mask`` is an additive float32 tensor broadcastable to
    [B, H, Lq, Lk] (last dimension contiguous; -inf drops a key).  ``out``
    may be a preallocated [B, H, Lq, d_v] view of any strides.  ``tile``
    names a compiled tile configuration (see :func:`kernel_name`) to run
    instead of the one chosen by shape.  Returns ``(out, lse)``."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q's dtype and device")
    B, H, Lq, dk = q.shape
    Lk, dv = k.shape[2], v.shape[3]
    if k.shape != (B, H, Lk, dk) or v.shape[:3] != (B, H, Lk):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    code = _dtype_code(q)
    dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
    if out is None:
        out = torch.empty((B, H, Lq, dv), dtype=q.dtype, device=q.device)
    elif out.shape != (B, H, Lq, dv) or out.dtype != q.dtype or out.device != q.device:
        raise ValueError("out must be a [B, H, Lq, d_v] view of q's dtype on q's device")
    if lse is None and need_lse:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, Lq) or lse.dtype != torch.float32
                            or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be float32 [B, H, Lq] on q's device")
    desc = ForwardDesc()
    desc.q, desc.k, desc.v, desc.out = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
    desc.lse = lse.data_ptr() if lse is not None else None
    desc.B, desc.H, desc.Lq, desc.Lk, desc.d_k, desc.d_v = B, H, Lq, Lk, dk, dv
    desc.q_layout = _layout_of(q, "q")
    desc.k_layout = _layout_of(k, "k")
    desc.v_layout = _layout_of(v, "v")
    desc.out_layout = _layout_of(out, "out")
    desc.causal = int(bool(causal))
    desc.key_lens = None
    if key_lens is not None:
        if (key_lens.dtype != torch.int32 or key_lens.shape != (B,) or key_lens.device != q.device
                or not key_lens.is_contiguous()):
            raise ValueError("key_lens must be a contiguous int32 [B] tensor on q's device")
        desc.key_lens = key_lens.data_ptr()
    desc.scale = float(scale) if scale is not None else 0.0
    desc.mask = None
    if mask is not None:
        if mask.dtype != torch.float32 or mask.device != q.device:
            raise ValueError("mask must be float32 on q's device")
        mv = mask.expand(B, H, Lq, Lk)
        ml = _layout_of(mv, "mask")
        if ml.row == 0:
            raise ValueError("mask rows must not be broadcast")
        desc.mask = mv.data_ptr()
        desc.mask_layout = ml
    desc.tile = tile.encode() if tile is not None else None
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = sdpa_forward_ex(handle_for(code, dev), desc, stream.cuda_stream)
    if st != SUCCESS:
        raise SdpaError(st, "sdpa_forward_ex")
    return out, lse


def backward(q, k, v, out, lse, dout, causal: bool = False, key_lens=None, dq=None, dk=None,
             dv=None, delta=None, stream=None):
    """Gradients (dq, dk, dv) of the forward that produced ``out`` and ``lse``.

    ``q, k, v, causal, key_lens`` as passed to :func:`forward`; ``out`` and
    ``lse`` its results; ``dout`` the gradient of the loss with respect to
    ``out`` (q's shape and dtype).  ``dq``/``dk``/``dv`` and the fp32
    [B, H, Lq] buffer ``delta`` (written with dout . out per row) may be
    given preallocated.  Returns ``(dq, dk, dv)``.
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, L, d_k] tensor")
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q's dtype and device")
    B, H, Lq, d = q.shape
    if k.shape[:2] != (B, H) or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must have q's shape")
    Lk = k.shape[2]
    code = _dtype_code(q)
    dev = q.device.index if q.device.index is not None else torch.cuda.current_device()

    def _vec(t, name):
        if (not isinstance(t, torch.Tensor) or t.shape != (B, H, Lq) or t.dtype != torch.float32
                or t.device != q.device or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 [B, H, Lq] tensor on q's device")
        return t

    _vec(lse, "lse")
    delta = _vec(delta, "delta") if delta is not None else torch.empty_like(lse)
    grads = []
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is None:
            t = torch.empty_like(ref)
        elif (t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device
              or not t.is_contiguous()):
            raise ValueError(f"{name} must match its input in shape, dtype and device")
        grads.append(t)
    dq, dk, dv = grads
    kl_ptr = None
    if key_lens is not None:
        if (key_lens.dtype != torch.int32 or key_lens.shape != (B,) or key_lens.device != q.device
                or not key_lens.is_contiguous()):
            raise ValueError("key_lens must be a contiguous int32 [B] tensor on q's device")
        kl_ptr = key_lens.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = sdpa_backward(handle_for(code, dev), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                       out.data_ptr(), dout.data_ptr(), lse.data_ptr(), delta.data_ptr(),
                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Lq, Lk, d,
                       int(bool(causal)), kl_ptr, stream.cuda_stream)
    if st != SUCCESS:
        raise SdpaError(st, "sdpa_backward")
    return dq, dk, dv


def decode(q, k, v, causal: bool = False, key_lens=None, out=None, lse=None,
           need_lse: bool = True, workspace=None, stream=None):
    """Decode-shaped forward (1 <= Lq <= 8 query rows, bf16, d_k 64 or 128):
    the same result as :func:`forward`, split over key chunks.  ``workspace``
    may be a preallocated uint8 CUDA tensor of at least
    ``decode_workspace_size(...)`` bytes; otherwise one is allocated here.
    Returns ``(out, lse)``."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, L, d_k] tensor")
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q's dtype and device")
    B, H, Lq, d = q.shape
    if k.shape[:2] != (B, H) or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    Lk = k.shape[2]
    code = _dtype_code(q)
    dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
    h = handle_for(code, dev)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must match q in shape, dtype and device, and be contiguous")
    if lse is None and need_lse:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, Lq) or lse.dtype != torch.float32
                            or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be float32 [B, H, Lq] on q's device")
    kl_ptr = None
    if key_lens is not None:
        if (key_lens.dtype != torch.int32 or key_lens.shape != (B,) or key_lens.device != q.device
                or not key_lens.is_contiguous()):
            raise ValueError("key_lens must be a contiguous int32 [B] tensor on q's device")
        kl_ptr = key_lens.data_ptr()
    need = sdpa_decode_workspace_size(h, B, H, Lq, Lk, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = sdpa_decode(h, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                     lse.data_ptr() if lse is not None else None, B, H, Lq, Lk, d,
                     int(bool(causal)), kl_ptr, ws_ptr, ws_bytes, stream.cuda_stream)
    if st != SUCCESS:
        raise SdpaError(st, "sdpa_decode")
    return out, lse


def decode_workspace_size(q, k) -> int:
    """Workspace bytes :func:`decode` needs for these tensors."""
    import torch
    B, H, Lq, d = q.shape
    dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
    return sdpa_decode_workspace_size(handle_for(_dtype_code(q), dev), B, H, Lq, k.shape[2], d)


def kernel_name(q, k, causal: bool = False, has_key_lens: bool = False):
    """Tile configuration the library would launch for these tensors."""
    import torch
    B, H, Lq, d = q.shape
    dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
    return sdpa_kernel_name(handle_for(_dtype_code(q), dev), B, H, Lq, k.shape[2], d,
                            int(bool(causal)), int(bool(has_key_lens)))
