"""Seeded synthetic inputs shared by the GPU tests, the CPU oracle and the bench.

This package holds no convolution or pooling arithmetic.  It maps
(seed, stream, element index) to numbers with Philox4x32-10 (Salmon et al.,
SC'11) in ``synth.c``, so any element range of any tensor can be regenerated
independently (the oracle can rebuild one (n, c) slice of a multi-GB input
without the rest).  See ``synth.c`` for the exact mapping.

``WORKLOADS`` lists the five workloads with their shapes and value
distributions; ``make_inputs`` draws them.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "synth.c")
    out = os.path.join(_HERE, "libsynth.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        u64, u32, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p
        lib.synth_philox4x32_10.argtypes = [vp, vp, vp]
        lib.synth_philox4x32_10.restype = None
        lib.synth_uniform_f32.argtypes = [u64, u32, u64, u64, ctypes.c_double,
                                          ctypes.c_double, vp]
        lib.synth_uniform_f32.restype = None
        lib.synth_normal_f32.argtypes = [u64, u32, u64, u64, vp]
        lib.synth_normal_f32.restype = None
        lib.synth_f32_to_bf16.argtypes = [vp, u64, vp]
        lib.synth_f32_to_bf16.restype = None
        _LIB = lib
    return _LIB


def philox4x32_10(ctr, key):
    """One Philox4x32-10 block: four uint32 counter words, two uint32 key words."""
    c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(v) & 0xFFFFFFFF for v in key])
    o = (ctypes.c_uint32 * 4)()
    _lib().synth_philox4x32_10(ctypes.addressof(c), ctypes.addressof(k), ctypes.addressof(o))
    return [int(v) for v in o]


def normal(seed: int, stream: int, shape, first: int = 0, out=None) -> np.ndarray:
    """N(0,1) float32 elements [first, first + prod(shape)) of (seed, stream)."""
    n = int(np.prod(shape))
    a = out if out is not None else np.empty(shape, dtype=np.float32)
    assert a.dtype == np.float32 and a.flags.c_contiguous and a.size == n
    _lib().synth_normal_f32(seed, stream, first, n, a.ctypes.data)
    return a


def uniform(seed: int, stream: int, shape, lo: float, hi: float, first: int = 0) -> np.ndarray:
    """U[lo, hi) float32 elements [first, first + prod(shape)) of (seed, stream)."""
    n = int(np.prod(shape))
    a = np.empty(shape, dtype=np.float32)
    _lib().synth_uniform_f32(seed, stream, first, n, float(lo), float(hi), a.ctypes.data)
    return a


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of a float32 array, round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    o = np.empty(a.shape, dtype=np.uint16)
    _lib().synth_f32_to_bf16(a.ctypes.data, a.size, o.ctypes.data)
    return o


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bf16 bit patterns."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Workloads.  Shapes follow the three problem statements on the pages; the
# value distributions are N(0,1) activations and biases and U(+-1/sqrt(fan))
# weights (fan = Cin * k^3 for the 3D chain, Cin * K for the 1D conv).
# Streams: 0 = x, 1 = weight, 2 = bias, 3 = conv bias.
# --------------------------------------------------------------------------
STREAM_X, STREAM_W, STREAM_BIAS, STREAM_CONV_BIAS = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    op: str                      # "fused3d" | "avgpool3d" | "convT1d"
    x_shape: tuple
    w_shape: tuple = ()
    w_bound: float = 0.0
    dtype: str = "f32"           # x / w storage: "f32" or "bf16"
    seed: int = 0
    params: dict = field(default_factory=dict)

    @property
    def description(self) -> str:
        return f"{self.name}: {self.op} x{list(self.x_shape)} {self.dtype}"


def _seed(i: int) -> int:
    return 0x5EED0000 + i


WORKLOADS = {
    # ConvTranspose3d(3->16,k3,s2,p1) -> x0.5 -> AvgPool3d(2) -> +bias -> x1.0
    "c1": Workload("c1", "fused3d", (2, 3, 8, 16, 16), (3, 16, 3, 3, 3),
                   1.0 / math.sqrt(81.0), "f32", _seed(1),
                   dict(scale1=0.5, scale2=1.0)),
    "c2": Workload("c2", "fused3d", (128, 3, 16, 32, 32), (3, 16, 3, 3, 3),
                   1.0 / math.sqrt(81.0), "f32", _seed(2),
                   dict(scale1=0.5, scale2=1.0)),
    # AvgPool3d(k3, s2, p1), count_include_pad
    "c3": Workload("c3", "avgpool3d", (16, 32, 128, 128, 256), seed=_seed(3),
                   params=dict(k=3, stride=2, pad=1)),
    # ConvTranspose1d(32->64, k5, s1, p0, dilation 3), no bias
    "c4": Workload("c4", "convT1d", (32, 32, 131072), (32, 64, 5),
                   1.0 / math.sqrt(160.0), "f32", _seed(4),
                   dict(stride=1, pad=0, dilation=3)),
    # ConvTranspose3d(32->64,...) chain with bf16 x and w
    "c5": Workload("c5", "fused3d", (16, 32, 16, 32, 32), (32, 64, 3, 3, 3),
                   1.0 / math.sqrt(864.0), "bf16", _seed(5),
                   dict(scale1=0.5, scale2=1.0)),
}


def make_inputs(wl: Workload, conv_bias: bool = False, x_dist: str = "normal",
                seed_offset: int = 0) -> dict:
    """Draw a workload's tensors as numpy arrays.

    Returns float32 arrays, and for bf16 workloads also ``x_bits`` / ``w_bits``
    (uint16) whose exact float32 values are ``x`` / ``w``.  ``x_dist`` may be
    "uniform01" for all-positive U[0,1) activations (the page's torch.rand).
    """
    seed = wl.seed + seed_offset
    out = {}
    if x_dist == "normal":
        x = normal(seed, STREAM_X, wl.x_shape)
    elif x_dist == "uniform01":
        x = uniform(seed, STREAM_X, wl.x_shape, 0.0, 1.0)
    else:
        raise ValueError(x_dist)
    if wl.op == "avgpool3d":
        out["x"] = x
        return out
    w = uniform(seed, STREAM_W, wl.w_shape, -wl.w_bound, wl.w_bound)
    if wl.dtype == "bf16":
        out["x_bits"] = to_bf16_bits(x)
        out["w_bits"] = to_bf16_bits(w)
        x = bf16_bits_to_f32(out["x_bits"]).reshape(wl.x_shape)
        w = bf16_bits_to_f32(out["w_bits"]).reshape(wl.w_shape)
    out["x"], out["w"] = x, w
    cout = wl.w_shape[1]
    if wl.op == "fused3d":
        out["bias"] = normal(seed, STREAM_BIAS, (cout,))
        if conv_bias:
            out["conv_bias"] = normal(seed, STREAM_CONV_BIAS, (cout,))
    elif wl.op == "convT1d" and conv_bias:
        out["bias"] = normal(seed, STREAM_BIAS, (cout,))
    return out
