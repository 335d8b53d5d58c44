"""Python binding of libct.so: the transposed-convolution / pooling hot path
on AMD Instinct MI355X (gfx950).

Every function here only marshals arguments into the C ABI of ``include/ct.h``
(same names, same argument order); all arithmetic runs in the HIP kernels.
PyTorch is used for device memory and streams only: tensors must be CUDA
(HIP) tensors, contiguous, of the dtype the entry point expects; work is
enqueued on the current torch stream of the tensor's device (or ``stream``).

There is no CPU fallback: importing this package without a built
``libct.so`` raises ImportError, and a call the library rejects raises
``CtError`` carrying the library's status and reason.

Operations (POPCORNBENCH pages, one problem each):
  [p50] "Kimi-K2.6 l2_p50" -- fused ConvTranspose3d -> scale -> AvgPool3d ->
        bias -> scale (``ct_convT3d_scale_pool_bias``)
        and the unfused first layer alone (``ct_convT3d``)
  [p46] "Kimi-K2.6 l1_p46" -- AvgPool3d(k3, s2, p1), divisor 27
        (``ct_avgpool3d``)
  [p74] "Kimi-K2.6 l1_p74" -- dilated ConvTranspose1d (``ct_convT1d``)
"""
from __future__ import annotations

import ctypes
import functools
import os

# torch is imported before libct.so is loaded so that libct.so's libamdhip64.so.7
# dependency binds to the HIP runtime torch already loaded: one process must
# hold a single HIP/ROCr runtime, or device memory and streams from torch are
# invalid handles to the library (it then sees no device at all).
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libct.so")

CT_OK, CT_EINVAL, CT_EUNSUPPORTED, CT_EHIP = 0, 1, 2, 3
CT_F32, CT_BF16 = 0, 1

_i64, _int, _ptr, _f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run transposed_conv_pooling_amd.build.build() "
            "(hipcc --offload-arch=gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.ct_convT_out_len.restype = _i64
    lib.ct_convT_out_len.argtypes = [_i64] * 6
    lib.ct_pool_out_len.restype = _i64
    lib.ct_pool_out_len.argtypes = [_i64] * 4
    lib.ct_convT3d_scale_pool_bias.restype = _int
    lib.ct_convT3d_scale_pool_bias.argtypes = (
        [_ptr, _int, _ptr, _int, _ptr, _ptr, _f32, _f32] + [_i64] * 6 + [_int] * 6 + [_ptr, _ptr])
    lib.ct_convT3d.restype = _int
    lib.ct_convT3d.argtypes = [_ptr, _int, _ptr, _int, _ptr] + [_i64] * 6 + [_int] * 4 + [_ptr, _ptr]
    lib.ct_avgpool3d.restype = _int
    lib.ct_avgpool3d.argtypes = [_ptr] + [_i64] * 5 + [_int] * 4 + [_ptr, _ptr]
    lib.ct_avgpool3d_bf16.restype = _int
    lib.ct_avgpool3d_bf16.argtypes = [_ptr] + [_i64] * 5 + [_int] * 4 + [_ptr, _ptr]
    lib.ct_convT1d.restype = _int
    lib.ct_convT1d.argtypes = [_ptr, _int, _ptr, _int, _ptr] + [_i64] * 4 + [_int] * 5 + [_ptr, _ptr]
    lib.ct_status_str.restype = ctypes.c_char_p
    lib.ct_status_str.argtypes = [_int]
    lib.ct_last_error.restype = ctypes.c_char_p
    lib.ct_last_error.argtypes = []
    lib.ct_version.restype = ctypes.c_char_p
    lib.ct_version.argtypes = []
    return lib


lib = _load()

# The CPython forwarding module built beside libct.so (same entry points, same
# argument order); the ctypes functions above serve where it is not built.
try:
    from . import _ctcall as _call
except ImportError:          # pragma: no cover - only a partial build lacks it
    _call = None


class CtError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{ct_status_str(status)}: {message}")
        self.status = status


def ct_status_str(status: int) -> str:
    return lib.ct_status_str(status).decode()


def ct_last_error() -> str:
    return lib.ct_last_error().decode()


def ct_version() -> str:
    return lib.ct_version().decode()


# The size helpers are pure functions of their integer arguments: each distinct
# geometry asks the library once (a ctypes call costs microseconds, which is
# most of a small workload's time per call).
@functools.lru_cache(maxsize=4096)
def ct_convT_out_len(n_in: int, k: int, stride: int = 1, pad: int = 0, out_pad: int = 0,
                     dilation: int = 1) -> int:
    return int(lib.ct_convT_out_len(n_in, k, stride, pad, out_pad, dilation))


@functools.lru_cache(maxsize=4096)
def ct_pool_out_len(n_in: int, k: int, stride: int = 0, pad: int = 0) -> int:
    return int(lib.ct_pool_out_len(n_in, k, stride, pad))


@functools.lru_cache(maxsize=4096)
def _fused_dims(D, H, W, k, stride, pad, out_pad, pool_k, pool_s):
    """Pooled output sizes of the fused chain per spatial axis (0 where empty)."""
    ps = pool_s if pool_s else pool_k
    dims = []
    for n in (D, H, W):
        o = ct_convT_out_len(n, k, stride, pad, out_pad, 1)
        dims.append(ct_pool_out_len(o, pool_k, ps, 0) if o > 0 else 0)
    return tuple(dims)


def _check(status: int):
    if status != CT_OK:
        raise CtError(status, ct_last_error())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return CT_F32
    if t.dtype == torch.bfloat16:
        return CT_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev_ptr(t, name, required=True):
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


# the current stream's raw handle without building a Stream object, where this
# torch build has the accessor
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(t, stream):
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(t.get_device())
        stream = torch.cuda.current_stream(t.device)
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def ct_convT3d_scale_pool_bias(x, w, conv_bias=None, bias=None, scale1: float = 1.0,
                               scale2: float = 1.0, stride: int = 2, pad: int = 1,
                               out_pad: int = 0, pool_k: int = 2, pool_s: int = 0,
                               out=None, stream=None):
    """out = ((AvgPool3d(ConvTranspose3d(x, w) + conv_bias) * scale1) + bias) * scale2.

    x [N,Cin,D,H,W] and w [Cin,Cout,k,k,k] both float32 or both bfloat16;
    conv_bias / bias float32 [Cout] (or [Cout,1,1,1]) or None; output float32.
    """
    torch = _torch()
    N, Cin, D, H, W = x.shape
    Cin2, Cout, k = w.shape[0], w.shape[1], w.shape[2]
    if Cin2 != Cin or tuple(w.shape[2:]) != (k, k, k):
        raise ValueError(f"weight shape {tuple(w.shape)} does not match input {tuple(x.shape)}")
    dims = _fused_dims(D, H, W, k, stride, pad, out_pad, pool_k, pool_s)
    if out is None:
        out = torch.empty((N, Cout, *[max(d, 0) for d in dims]), dtype=torch.float32,
                          device=x.device)
    elif tuple(out.shape) != (N, Cout, *dims) or out.dtype != torch.float32:
        raise ValueError(f"out must be float32 {(N, Cout, *dims)}")
    for name, b in (("conv_bias", conv_bias), ("bias", bias)):
        if b is not None and (b.dtype != torch.float32 or b.numel() != Cout):
            raise ValueError(f"{name} must be float32 with {Cout} elements")
    args = (_dev_ptr(x, "x"), _dtype_code(x), _dev_ptr(w, "w"), _dtype_code(w),
            _dev_ptr(conv_bias, "conv_bias", False) or 0, _dev_ptr(bias, "bias", False) or 0,
            float(scale1), float(scale2), N, Cin, D, H, W, Cout, k, stride, pad, out_pad,
            pool_k, pool_s, _dev_ptr(out, "out"), _stream_handle(x, stream))
    st = _call.fused(*args) if _call else lib.ct_convT3d_scale_pool_bias(*args)
    _check(st)
    return out


def ct_convT3d(x, w, bias=None, stride: int = 2, pad: int = 1, out_pad: int = 0, out=None,
               stream=None):
    """ConvTranspose3d; x [N,Cin,D,H,W], w [Cin,Cout,k,k,k] (both float32 or both
    bfloat16), bias float32 [Cout] or None -> float32 [N,Cout,Do,Ho,Wo]."""
    torch = _torch()
    N, Cin, D, H, W = x.shape
    Cin2, Cout, k = w.shape[0], w.shape[1], w.shape[2]
    if Cin2 != Cin or tuple(w.shape[2:]) != (k, k, k):
        raise ValueError(f"weight shape {tuple(w.shape)} does not match input {tuple(x.shape)}")
    dims = [ct_convT_out_len(n, k, stride, pad, out_pad, 1) for n in (D, H, W)]
    if out is None:
        out = torch.empty((N, Cout, *[max(d, 0) for d in dims]), dtype=torch.float32,
                          device=x.device)
    elif tuple(out.shape) != (N, Cout, *dims) or out.dtype != torch.float32:
        raise ValueError(f"out must be float32 {(N, Cout, *dims)}")
    if bias is not None and (bias.dtype != torch.float32 or bias.numel() != Cout):
        raise ValueError(f"bias must be float32 with {Cout} elements")
    args = (_dev_ptr(x, "x"), _dtype_code(x), _dev_ptr(w, "w"), _dtype_code(w),
            _dev_ptr(bias, "bias", False) or 0, N, Cin, D, H, W, Cout, k, stride, pad, out_pad,
            _dev_ptr(out, "out"), _stream_handle(x, stream))
    st = _call.convT3d(*args) if _call else lib.ct_convT3d(*args)
    _check(st)
    return out


def ct_avgpool3d(x, k: int = 3, stride: int = 2, pad: int = 1, count_include_pad: bool = True,
                 out=None, stream=None):
    """AvgPool3d over zero padding; x [N,C,D,H,W] float32 -> float32, or
    bfloat16 -> bfloat16 (fp32 sums, each mean rounded to the nearest bf16)."""
    torch = _torch()
    N, C, D, H, W = x.shape
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    dt = x.dtype
    dims = [ct_pool_out_len(n, k, stride, pad) for n in (D, H, W)]
    if out is None:
        out = torch.empty((N, C, *[max(d, 0) for d in dims]), dtype=dt, device=x.device)
    elif tuple(out.shape) != (N, C, *dims) or out.dtype != dt:
        raise ValueError(f"out must be {dt} {(N, C, *dims)}")
    args = (_dev_ptr(x, "x"), N, C, D, H, W, k, stride, pad, 1 if count_include_pad else 0,
            _dev_ptr(out, "out"), _stream_handle(x, stream))
    if _call:
        st = _call.avgpool3d(dt != torch.float32, *args)
    else:
        st = (lib.ct_avgpool3d if dt == torch.float32 else lib.ct_avgpool3d_bf16)(*args)
    _check(st)
    return out


def ct_convT1d(x, w, bias=None, stride: int = 1, pad: int = 0, dilation: int = 1,
               out_pad: int = 0, out=None, stream=None):
    """Transposed 1D convolution; x [N,Cin,L], w [Cin,Cout,K] (both float32 or both
    bfloat16), bias float32 [Cout] or None -> float32 [N,Cout,L_out]."""
    torch = _torch()
    N, Cin, L = x.shape
    Cin2, Cout, K = w.shape
    if Cin2 != Cin:
        raise ValueError(f"weight shape {tuple(w.shape)} does not match input {tuple(x.shape)}")
    Lo = ct_convT_out_len(L, K, stride, pad, out_pad, dilation)
    if out is None:
        out = torch.empty((N, Cout, max(Lo, 0)), dtype=torch.float32, device=x.device)
    elif tuple(out.shape) != (N, Cout, Lo) or out.dtype != torch.float32:
        raise ValueError(f"out must be float32 {(N, Cout, Lo)}")
    if bias is not None and (bias.dtype != torch.float32 or bias.numel() != Cout):
        raise ValueError(f"bias must be float32 with {Cout} elements")
    args = (_dev_ptr(x, "x"), _dtype_code(x), _dev_ptr(w, "w"), _dtype_code(w),
            _dev_ptr(bias, "bias", False) or 0, N, Cin, L, Cout, K, stride, pad, dilation,
            out_pad, _dev_ptr(out, "out"), _stream_handle(x, stream))
    st = _call.convT1d(*args) if _call else lib.ct_convT1d(*args)
    _check(st)
    return out


__all__ = [
    "CtError", "CT_OK", "CT_EINVAL", "CT_EUNSUPPORTED", "CT_EHIP", "CT_F32", "CT_BF16",
    "ct_convT3d_scale_pool_bias", "ct_convT3d", "ct_avgpool3d", "ct_convT1d", "ct_convT_out_len",
    "ct_pool_out_len", "ct_status_str", "ct_last_error", "ct_version", "lib", "LIB_PATH",
]
