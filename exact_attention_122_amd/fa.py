"""Thin Python binding of libfa.so (ctypes), same names as include/fa.h.

Only argument marshalling lives here: tensors become device pointers, the
current torch stream becomes the hipStream_t, and a non-OK status becomes a
RuntimeError carrying the library's detail message. Every step of the
attention computation runs in the library's HIP kernels; if the library is
missing this module raises instead of computing anything another way.
PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARGUMENT = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_HIP = 3
FA_BF16 = 0
FA_FP32 = 1
FA_FP16 = 2

EXPORTS = ("fa_version", "fa_status_string", "fa_last_error_detail", "fa_fwd",
           "fa_bwd_workspace_bytes", "fa_bwd", "fa_fwd_ex", "fa_bwd_ex_workspace_bytes",
           "fa_bwd_ex", "fa_bwd_noalloc")
# bytes of the device scratch fa_bwd_noalloc uses (FA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 16 << 20

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run `python -m exact_attention_122_amd.build` "
            "(or __graft_entry__.build()); there is no other implementation to fall back on")
    # torch ships its own HIP runtime. Loaded first, it is the one libfa.so
    # binds to; loaded after libfa.so, a second runtime would come in beside
    # the system one, and the library's launches would find no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_version.restype = i
    lib.fa_version.argtypes = []
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [i]
    lib.fa_last_error_detail.restype = ctypes.c_char_p
    lib.fa_last_error_detail.argtypes = []
    lib.fa_fwd.restype = i
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_bwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp, sz, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lp = ctypes.POINTER(ctypes.c_longlong)
    lib.fa_fwd_ex.restype = i
    lib.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, lp, lp, lp, lp, vp, lp, f, i, i, i, vp]
    lib.fa_bwd_ex_workspace_bytes.restype = sz
    lib.fa_bwd_ex_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_bwd_ex.restype = i
    lib.fa_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i,
                              lp, lp, lp, lp, lp, lp, lp, lp, vp, lp, f, i, i, i, vp, sz, vp]
    _lib = lib
    return lib


# ------------------------------------------------------------ raw C calls ---

def fa_version() -> int:
    return load_library().fa_version()


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(status).decode()


def fa_last_error_detail() -> str:
    return load_library().fa_last_error_detail().decode()


def _check(status: int, what: str):
    if status != FA_OK:
        raise RuntimeError(f"{what} failed: {fa_status_string(status)}: {fa_last_error_detail()}")


# --------------------------------------------------------- torch helpers ---

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_FP32
    if t.dtype == torch.float16:
        return FA_FP16
    raise RuntimeError(f"dtype {t.dtype} is not built (bfloat16, float16 or float32)")


def _shape(q):
    if q.dim() != 4:
        raise RuntimeError(f"expected [B, H, N, d] tensors, got shape {tuple(q.shape)}")
    return tuple(int(x) for x in q.shape)


def _same(ref, *ts):
    for t in ts:
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise RuntimeError("all [B, H, N, d] tensors must share shape, dtype and device")
        if not t.is_contiguous():
            raise RuntimeError("tensors must be contiguous [B, H, N, d]")
    if not ref.is_cuda:
        raise RuntimeError("tensors must live in GPU memory")


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded to float32 (the value the C call receives)."""
    return float(ctypes.c_float(1.0 / math.sqrt(d)).value)


def fa_fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """O, LSE = attention forward of [B, H, N, d] tensors (see include/fa.h)."""
    import torch
    _same(q, k, v)
    B, H, N, d = _shape(q)
    if scale is None:
        scale = default_scale(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _same(q, out)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise RuntimeError("lse must be a contiguous float32 [B, H, N] tensor")
    st = load_library().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                               _dtype_code(q), _stream(q))
    _check(st, "fa_fwd")
    return out, lse


def fa_bwd_workspace_bytes(B: int, H: int, N: int, d: int, dtype: int = FA_BF16) -> int:
    return int(load_library().fa_bwd_workspace_bytes(B, H, N, d, dtype))


def fa_bwd(q, k, v, o, do, lse, causal: bool = False, scale: float | None = None,
           dq=None, dk=None, dv=None, workspace=None):
    """dQ, dK, dV of sum(O * dO) for O = fa_fwd(q, k, v) (see include/fa.h)."""
    import torch
    _same(q, k, v, o, do)
    B, H, N, d = _shape(q)
    if scale is None:
        scale = default_scale(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _same(q, dq, dk, dv)
    code = _dtype_code(q)
    need = fa_bwd_workspace_bytes(B, H, N, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise RuntimeError("lse must be a contiguous float32 [B, H, N] tensor")
    st = load_library().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                               dv.data_ptr(), B, H, N, d, float(scale), int(bool(causal)), code,
                               workspace.data_ptr(), workspace.numel(), _stream(q))
    _check(st, "fa_bwd")
    return dq, dk, dv


def fa_bwd_noalloc(q, k, v, o, do, lse, causal: bool = False, scale: float | None = None,
                   dq=None, dk=None, dv=None):
    """fa_bwd without a workspace: the library's own per-GPU scratch holds the
    row statistics (see include/fa.h). Pass dq, dk, dv to allocate nothing."""
    import torch
    _same(q, k, v, o, do)
    B, H, N, d = _shape(q)
    if scale is None:
        scale = default_scale(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _same(q, dq, dk, dv)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise RuntimeError("lse must be a contiguous float32 [B, H, N] tensor")
    st = load_library().fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                       dv.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                                       _dtype_code(q), _stream(q))
    _check(st, "fa_bwd_noalloc")
    return dq, dk, dv


# ---------------------------------------------- general shapes and masks ---

def _band(causal: bool, window):
    """(window_left, window_right) for the C call; -1 = no bound."""
    left, right = (-1, -1) if window is None else (
        -1 if window[0] is None else int(window[0]), -1 if window[1] is None else int(window[1]))
    if causal:
        if right not in (-1, 0):
            raise RuntimeError("causal sets window_right = 0; window gives another right bound")
        right = 0
    return left, right


def _strides(t, name):
    """{batch, head, row} element strides of a [B, H, rows, d] view (d contiguous)."""
    if t.dim() != 4:
        raise RuntimeError(f"{name}: expected a [B, H, rows, d] tensor, got shape {tuple(t.shape)}")
    if t.stride(3) != 1 and t.shape[3] != 1:
        raise RuntimeError(f"{name}: the last dimension (d) must be contiguous")
    return (ctypes.c_longlong * 3)(t.stride(0), t.stride(1), t.stride(2))


def _bias_arg(bias, q, B, H, Nq, Nk):
    """(pointer, strides) of an optional float32 bias broadcastable to [B, H, Nq, Nk]."""
    import torch
    if bias is None:
        return None, None
    if bias.dtype != torch.float32 or bias.device != q.device:
        raise RuntimeError("bias must be a float32 tensor on Q's device")
    b = bias.expand(B, H, Nq, Nk)
    if Nk > 1 and b.stride(3) != 1:
        raise RuntimeError("bias: the key dimension must be contiguous")
    return b.data_ptr(), (ctypes.c_longlong * 3)(b.stride(0), b.stride(1), b.stride(2))


def _ex_operands(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise RuntimeError("expected [B, H, rows, d] tensors")
    B, H, Nq, d = (int(x) for x in q.shape)
    Nk = int(k.shape[2])
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d):
        raise RuntimeError("K and V must be [B, H, Nk, d] with Q's B, H and d")
    for t in (k, v):
        if t.dtype != q.dtype or t.device != q.device:
            raise RuntimeError("Q, K and V must share dtype and device")
    if not q.is_cuda:
        raise RuntimeError("tensors must live in GPU memory")
    return B, H, Nq, Nk, d


def fa_fwd_ex(q, k, v, causal: bool = False, window=None, scale: float | None = None,
              out=None, lse=None, bias=None):
    """O, LSE for Nq queries over Nk keys with a band mask and strided views.

    ``window`` = (left, right) bounds the visible keys around each query's
    aligned key i + Nk - Nq (None = unbounded); ``causal`` sets right = 0.
    ``bias`` (float32, broadcastable to [B, H, Nq, Nk]) is added to the scaled
    scores. Any [B, H, rows, d] views with d contiguous are accepted (see
    include/fa.h).
    """
    import torch
    B, H, Nq, Nk, d = _ex_operands(q, k, v)
    left, right = _band(causal, window)
    if scale is None:
        scale = default_scale(d)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (B, H, Nq, d) or out.dtype != q.dtype or out.device != q.device:
        raise RuntimeError("out must be [B, H, Nq, d] of Q's dtype and device")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq) or not lse.is_contiguous():
        raise RuntimeError("lse must be a contiguous float32 [B, H, Nq] tensor")
    bp, bs = _bias_arg(bias, q, B, H, Nq, Nk)
    st = load_library().fa_fwd_ex(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d,
        _strides(q, "Q"), _strides(k, "K"), _strides(v, "V"), _strides(out, "O"), bp, bs,
        float(scale), left, right, _dtype_code(q), _stream(q))
    _check(st, "fa_fwd_ex")
    return out, lse


def fa_bwd_ex_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int, dtype: int = FA_BF16) -> int:
    return int(load_library().fa_bwd_ex_workspace_bytes(B, H, Nq, Nk, d, dtype))


def fa_bwd_ex(q, k, v, o, do, lse, causal: bool = False, window=None, scale: float | None = None,
              dq=None, dk=None, dv=None, workspace=None, bias=None):
    """dQ, dK, dV for O, LSE = fa_fwd_ex(q, k, v, causal, window, scale, bias=bias)."""
    import torch
    B, H, Nq, Nk, d = _ex_operands(q, k, v)
    left, right = _band(causal, window)
    if scale is None:
        scale = default_scale(d)
    for t, shape, name in ((o, (B, H, Nq, d), "O"), (do, (B, H, Nq, d), "dO")):
        if tuple(t.shape) != shape or t.dtype != q.dtype or t.device != q.device:
            raise RuntimeError(f"{name} must be [B, H, Nq, d] of Q's dtype and device")
    dq = torch.empty((B, H, Nq, d), dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty((B, H, Nk, d), dtype=q.dtype, device=q.device) if dk is None else dk
    dv = torch.empty((B, H, Nk, d), dtype=q.dtype, device=q.device) if dv is None else dv
    for t, shape, name in ((dq, (B, H, Nq, d), "dQ"), (dk, (B, H, Nk, d), "dK"), (dv, (B, H, Nk, d), "dV")):
        if tuple(t.shape) != shape or t.dtype != q.dtype or t.device != q.device:
            raise RuntimeError(f"{name} has the wrong shape, dtype or device")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq) or not lse.is_contiguous():
        raise RuntimeError("lse must be a contiguous float32 [B, H, Nq] tensor")
    code = _dtype_code(q)
    need = fa_bwd_ex_workspace_bytes(B, H, Nq, Nk, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    bp, bs = _bias_arg(bias, q, B, H, Nq, Nk)
    st = load_library().fa_bwd_ex(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Nq, Nk, d,
        _strides(q, "Q"), _strides(k, "K"), _strides(v, "V"), _strides(o, "O"), _strides(do, "dO"),
        _strides(dq, "dQ"), _strides(dk, "dK"), _strides(dv, "dV"), bp, bs,
        float(scale), left, right, code, workspace.data_ptr(), workspace.numel(), _stream(q))
    _check(st, "fa_bwd_ex")
    return dq, dk, dv
