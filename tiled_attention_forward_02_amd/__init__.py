"""Python binding of libmi_attn: argument marshalling over the C ABI only.

Every step of the attention forward and backward runs in the HIP kernels
behind the C entry points of libmi_attn.so; this module checks tensors, allocates the
outputs with torch (device memory and streams are all torch provides here) and
passes raw pointers. There is no fallback: if the shared library is missing
the first call raises.
"""

from __future__ import annotations

import ctypes
import math
import os

__all__ = ["attn_fwd", "attn_fwd_cross", "attn_fwd_ex", "attn_bwd", "attn_bwd_noalloc",
           "attn_strerror",
           "attn_fwd_launch_shape", "lib_path", "load_library", "AttnError", "ATTN_BF16",
           "ATTN_F16"]

ATTN_BF16, ATTN_F16 = 0, 1  # attn_dtype values of the C ABI

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmi_attn.so")
_lib = None


class AttnError(RuntimeError):
    """A non-zero status returned by libmi_attn."""

    def __init__(self, status, message):
        super().__init__(f"libmi_attn call failed ({status}): {message}")
        self.status = status


def lib_path():
    return _LIB_PATH


def load_library():
    """Load libmi_attn.so (once). Raises ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with "
            "`python -m tiled_attention_forward_02_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp]
    lib.attn_fwd.restype = i32
    lib.attn_fwd_cross.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.attn_fwd_cross.restype = i32
    lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.attn_fwd_ex.restype = i32
    lib.attn_bwd.argtypes = [vp] * 10 + [i32] * 6 + [f32, i32, vp]
    lib.attn_bwd.restype = i32
    lib.attn_bwd_noalloc.argtypes = [vp] * 9 + [i32] * 6 + [f32, i32, vp]
    lib.attn_bwd_noalloc.restype = i32
    lib.attn_strerror.argtypes = [i32]
    lib.attn_strerror.restype = ctypes.c_char_p
    ip = ctypes.POINTER(i32)
    lib.attn_fwd_launch_shape.argtypes = [i32, i32, i32, i32, i32, ip, ip, ip, ip, ip]
    lib.attn_fwd_launch_shape.restype = i32
    _lib = lib
    return lib


def attn_strerror(status):
    return load_library().attn_strerror(int(status)).decode()


def attn_fwd_launch_shape(B, H, N, d, causal=False):
    """The launch attn_fwd makes for these sizes, as a dict (no launch)."""
    lib = load_library()
    out = [ctypes.c_int(0) for _ in range(5)]
    rc = lib.attn_fwd_launch_shape(B, H, N, d, int(bool(causal)),
                                   *[ctypes.byref(x) for x in out])
    if rc:
        raise AttnError(rc, attn_strerror(rc))
    return dict(zip(("grid", "block", "lds_bytes", "block_m", "block_n"),
                    (x.value for x in out)))


def _check_inputs(q, k, v, dtypes=None):
    import torch

    dtypes = (torch.bfloat16,) if dtypes is None else dtypes
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype not in dtypes:
            raise TypeError(f"{name} must be one of {dtypes}, got {t.dtype}")
        if t.dtype != q.dtype:
            raise TypeError("q, k, v must share one dtype")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a HIP device, got {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B, H, N, d]")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError(f"q, k, v must be [B, H, N, d] with k and v alike, got "
                         f"{tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError(f"q and k must share B, H and d, got {tuple(q.shape)}, {tuple(k.shape)}")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")


def _outputs(q, out, lse):
    import torch

    B, H, Nq, _ = q.shape
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype != q.dtype
          or out.device != q.device or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor shaped like q, of q's dtype")
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    elif (tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32
          or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor [B, H, Nq]")
    return out, lse


def _stream_handle(q, stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _default_scale(d):
    import torch

    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def attn_fwd(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """O, lse = attention forward of bf16 tensors q, k, v [B, H, N, d].

    scale defaults to float32(1/sqrt(d)). ``out`` ([B,H,N,d] bf16) and ``lse``
    ([B,H,N] float32) may be given to write into; otherwise they are allocated
    on q's device. The kernel is queued on ``stream`` (default: torch's current
    stream of q's device); nothing synchronises.
    """
    import torch

    lib = load_library()
    _check_inputs(q, k, v)
    if k.shape != q.shape:
        raise ValueError(f"q, k, v must share one [B, H, N, d] shape, got "
                         f"{tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    B, H, N, d = q.shape
    scale = _default_scale(d) if scale is None else scale
    out, lse = _outputs(q, out, lse)
    with torch.cuda.device(q.device):
        rc = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                          _stream_handle(q, stream))
    if rc:
        raise AttnError(rc, attn_strerror(rc))
    return out, lse


def attn_fwd_cross(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """O, lse = attention forward of q [B, H, Nq, d] against k, v [B, H, Nk, d].

    causal aligns the query and key axes at their ends (query i sees keys
    j <= i + Nk - Nq); a query that sees no key gets o = 0 and lse = -inf.
    Other arguments as for attn_fwd.
    """
    import torch

    lib = load_library()
    _check_inputs(q, k, v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    scale = _default_scale(d) if scale is None else scale
    out, lse = _outputs(q, out, lse)
    kp = k.data_ptr() if Nk else 0
    vp = v.data_ptr() if Nk else 0
    with torch.cuda.device(q.device):
        rc = lib.attn_fwd_cross(q.data_ptr(), kp, vp, out.data_ptr(), lse.data_ptr(),
                                B, H, Nq, Nk, d, float(scale), int(bool(causal)),
                                _stream_handle(q, stream))
    if rc:
        raise AttnError(rc, attn_strerror(rc))
    return out, lse


def attn_fwd_ex(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """attn_fwd_cross for bfloat16 or float16 tensors (q, k, v one dtype; o
    gets that dtype, lse float32)."""
    import torch

    lib = load_library()
    _check_inputs(q, k, v, dtypes=(torch.bfloat16, torch.float16))
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dtype = ATTN_BF16 if q.dtype == torch.bfloat16 else ATTN_F16
    scale = _default_scale(d) if scale is None else scale
    out, lse = _outputs(q, out, lse)
    kp = k.data_ptr() if Nk else 0
    vp = v.data_ptr() if Nk else 0
    with torch.cuda.device(q.device):
        rc = lib.attn_fwd_ex(q.data_ptr(), kp, vp, out.data_ptr(), lse.data_ptr(), B, H, Nq,
                             Nk, d, dtype, float(scale), int(bool(causal)),
                             _stream_handle(q, stream))
    if rc:
        raise AttnError(rc, attn_strerror(rc))
    return out, lse


def _like(t, ref, shape, dtype, name):
    """An output tensor: `t` checked, or a new one on ref's device."""
    import torch

    if t is None:
        return torch.empty(shape, dtype=dtype, device=ref.device)
    if (tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != ref.device
            or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor {tuple(shape)} on "
                         f"{ref.device}")
    return t


def _bwd_args(q, k, v, o, lse, do, scale, dq, dk, dv):
    """Checks and outputs shared by the two backward calls."""
    import torch

    _check_inputs(q, k, v, dtypes=(torch.bfloat16, torch.float16))
    B, H, Nq, d = q.shape
    for name, t in (("o", o), ("do", do)):
        if (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(q.shape)
                or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous tensor shaped like q, of q's dtype")
    if (not isinstance(lse, torch.Tensor) or tuple(lse.shape) != (B, H, Nq)
            or lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor [B, H, Nq]")
    dq = _like(dq, q, q.shape, q.dtype, "dq")
    dk = _like(dk, q, k.shape, q.dtype, "dk")
    dv = _like(dv, q, k.shape, q.dtype, "dv")
    dtype = ATTN_BF16 if q.dtype == torch.bfloat16 else ATTN_F16
    scale = _default_scale(d) if scale is None else scale
    return dq, dk, dv, dtype, float(scale)


def _ptr(t):
    return t.data_ptr() if t.numel() else 0


def attn_bwd(q, k, v, o, lse, do, scale=None, causal=False, dq=None, dk=None, dv=None,
             delta=None, stream=None):
    """dq, dk, dv = gradients of sum(do * o) where o, lse = attn_fwd_ex(q, k, v,
    scale, causal) are passed in (the forward's own outputs for these inputs).

    q, o, do [B, H, Nq, d] and k, v [B, H, Nk, d] share one element type
    (bf16 or fp16); lse is float32 [B, H, Nq]; d is 32, 64, 96, 128 or 256. ``delta``
    (float32 [B, H, Nq]) receives sum(do * o) per row and is allocated when
    not given; dq, dk, dv may be given to write into. Queued on ``stream``
    (default: torch's current stream of q's device); nothing synchronises.
    """
    import torch

    lib = load_library()
    dq, dk, dv, dtype, scale = _bwd_args(q, k, v, o, lse, do, scale, dq, dk, dv)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    delta = _like(delta, q, (B, H, Nq), torch.float32, "delta")
    with torch.cuda.device(q.device):
        rc = lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                          _ptr(dk), _ptr(dv), _ptr(delta), B, H, Nq, Nk, d, dtype, scale,
                          int(bool(causal)), _stream_handle(q, stream))
    if rc:
        raise AttnError(rc, attn_strerror(rc))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale=None, causal=False, stream=None):
    """attn_bwd into the given dq, dk, dv, with the row sums kept in the
    library's static device buffer: this call allocates no device memory
    (B*H*Nq up to 4194304 rows). Calls that overlap on one device race on that
    buffer. Queued on ``stream`` (default: torch's current stream of q's
    device); nothing synchronises.
    """
    import torch

    lib = load_library()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a preallocated torch.Tensor")
    dq, dk, dv, dtype, scale = _bwd_args(q, k, v, o, lse, do, scale, dq, dk, dv)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    with torch.cuda.device(q.device):
        rc = lib.attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                  _ptr(dq), _ptr(dk), _ptr(dv), B, H, Nq, Nk, d, dtype, scale,
                                  int(bool(causal)), _stream_handle(q, stream))
    if rc:
        raise AttnError(rc, attn_strerror(rc))
    return dq, dk, dv
