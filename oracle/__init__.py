"""CPU oracle for the transposed-convolution / pooling path (fp64).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``transposed_conv_pooling_amd``) never imports it, and this package imports
nothing from there.

The arithmetic lives in ``oracle.c`` (plain C, fp64, literal scatter-form
transposed convolutions and literal pooling loops); this module only marshals
numpy arrays into it.  Every function takes an optional ``lib`` (a library
loaded with ``load_library``) so the test suite can run its pins against
deliberately broken builds of the same source.  Inputs are taken as float32 (the values the GPU sees)
and outputs are float64.

Sources are web pages on the POPCORNBENCH site, one problem each:

* [p50] "Kimi-K2.6 l2_p50" -- fused ConvTranspose3d -> scale -> AvgPool3d ->
  bias -> scale.
* [p46] "Kimi-K2.6 l1_p46" -- AvgPool3d(k3, s2, p1).
* [p74] "Kimi-K2.6 l1_p74" -- dilated ConvTranspose1d.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))

_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p


def load_library(path: str) -> ctypes.CDLL:
    """Load an oracle shared library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    lib.oracle_convT_out_len.restype = _i64
    lib.oracle_convT_out_len.argtypes = [_i64] * 6
    lib.oracle_pool_out_len.restype = _i64
    lib.oracle_pool_out_len.argtypes = [_i64] * 4
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_convT3d.restype = ctypes.c_int
    lib.oracle_convT3d.argtypes = [_ptr, _ptr, _ptr] + [_i64] * 10 + [_ptr]
    lib.oracle_convT3d_scale_pool_bias.restype = ctypes.c_int
    lib.oracle_convT3d_scale_pool_bias.argtypes = (
        [_ptr, _ptr, _ptr, _ptr, ctypes.c_double, ctypes.c_double]
        + [_i64] * 12 + [_ptr])
    lib.oracle_avgpool3d.restype = ctypes.c_int
    lib.oracle_avgpool3d.argtypes = [_ptr] + [_i64] * 7 + [ctypes.c_int, _ptr]
    lib.oracle_convT1d.restype = ctypes.c_int
    lib.oracle_convT1d.argtypes = [_ptr, _ptr, _ptr] + [_i64] * 9 + [_ptr]
    return lib


_DEFAULT_LIB = None


def _lib():
    global _DEFAULT_LIB
    if _DEFAULT_LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            _build.build()
        _DEFAULT_LIB = load_library(path)
    return _DEFAULT_LIB


def _f32(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc == -1:
        raise ValueError(f"{what}: invalid geometry (non-positive size or empty output)")
    if rc != 0:
        raise MemoryError(f"{what}: scratch allocation failed")


def num_threads(lib=None) -> int:
    """OpenMP threads the oracle runs on."""
    return int((lib or _lib()).oracle_num_threads())


def convT_out_len(n_in, k, stride=1, pad=0, out_pad=0, dilation=1, lib=None) -> int:
    """(in-1)*stride - 2*pad + dilation*(k-1) + out_pad + 1 ([p50], [p74])."""
    return int((lib or _lib()).oracle_convT_out_len(n_in, k, stride, pad, out_pad, dilation))


def pool_out_len(n_in, k, stride, pad=0, lib=None) -> int:
    """floor((in + 2*pad - k)/stride) + 1, ceil_mode off ([p50], [p46])."""
    return int((lib or _lib()).oracle_pool_out_len(n_in, k, stride, pad))


def convT3d(x, w, conv_bias=None, stride=1, pad=0, out_pad=0, lib=None):
    """Scatter-form ConvTranspose3d, fp64.  x [N,Cin,D,H,W], w [Cin,Cout,k,k,k]."""
    x, w, cb = _f32(x), _f32(w), _f32(conv_bias)
    N, Cin, D, H, W = x.shape
    Cin2, Cout, k, k2, k3 = w.shape
    assert Cin2 == Cin and k == k2 == k3
    Do, Ho, Wo = (convT_out_len(n, k, stride, pad, out_pad, lib=lib) for n in (D, H, W))
    y = np.empty((N, Cout, max(Do, 0), max(Ho, 0), max(Wo, 0)), dtype=np.float64)
    rc = (lib or _lib()).oracle_convT3d(_p(x), _p(w), _p(cb), N, Cin, D, H, W, Cout, k,
                               stride, pad, out_pad, _p(y))
    _check(rc, "convT3d")
    return y


def convT3d_scale_pool_bias(x, w, conv_bias, bias, scale1, scale2, stride=2,
                            pad=1, out_pad=0, pool_k=2, pool_s=None, lib=None):
    """The [p50] chain: convT3d (+conv_bias) -> *scale1 -> AvgPool3d -> +bias -> *scale2."""
    x, w, cb, b = _f32(x), _f32(w), _f32(conv_bias), _f32(bias)
    if pool_s is None:
        pool_s = pool_k
    N, Cin, D, H, W = x.shape
    Cin2, Cout, k, k2, k3 = w.shape
    assert Cin2 == Cin and k == k2 == k3
    dims = []
    for n in (D, H, W):
        o = convT_out_len(n, k, stride, pad, out_pad, lib=lib)
        dims.append(pool_out_len(o, pool_k, pool_s, 0, lib=lib) if o > 0 else 0)
    out = np.empty((N, Cout) + tuple(max(d, 0) for d in dims), dtype=np.float64)
    rc = (lib or _lib()).oracle_convT3d_scale_pool_bias(
        _p(x), _p(w), _p(cb), _p(b), float(scale1), float(scale2),
        N, Cin, D, H, W, Cout, k, stride, pad, out_pad, pool_k, pool_s, _p(out))
    _check(rc, "convT3d_scale_pool_bias")
    return out


def avgpool3d(x, k=3, stride=None, pad=0, count_include_pad=True, lib=None):
    """AvgPool3d over zero padding ([p46]).  x [..., D, H, W] (leading dims are slices)."""
    x = _f32(x)
    if stride is None:
        stride = k
    *lead, D, H, W = x.shape
    NC = int(np.prod(lead)) if lead else 1
    dims = [pool_out_len(n, k, stride, pad, lib=lib) for n in (D, H, W)]
    out = np.empty(tuple(lead) + tuple(max(d, 0) for d in dims), dtype=np.float64)
    rc = (lib or _lib()).oracle_avgpool3d(_p(x), NC, D, H, W, k, stride, pad,
                                 1 if count_include_pad else 0, _p(out))
    _check(rc, "avgpool3d")
    return out


def convT1d(x, w, bias=None, stride=1, pad=0, dilation=1, out_pad=0, lib=None):
    """Scatter-form ConvTranspose1d ([p74]).  x [N,Cin,L], w [Cin,Cout,K]."""
    x, w, b = _f32(x), _f32(w), _f32(bias)
    N, Cin, L = x.shape
    Cin2, Cout, K = w.shape
    assert Cin2 == Cin
    Lo = convT_out_len(L, K, stride, pad, out_pad, dilation, lib=lib)
    y = np.empty((N, Cout, max(Lo, 0)), dtype=np.float64)
    rc = (lib or _lib()).oracle_convT1d(_p(x), _p(w), _p(b), N, Cin, L, Cout, K, stride,
                               pad, dilation, out_pad, _p(y))
    _check(rc, "convT1d")
    return y
