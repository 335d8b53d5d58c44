"""The C ABI without a GPU: libct.so loads, exports every function include/ct.h
declares, its pure host helpers follow the pages' size formulas, and every
malformed request is rejected by host-side validation (before any HIP call).

Every request below is invalid on purpose and is rejected before launch; none
would reach the GPU even on a GPU machine (the fake device addresses are
never dereferenced)."""
import ctypes
import os
import re

import pytest

import transposed_conv_pooling_amd as ct

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ct.h")

FAKE = 0x10000      # a 256-byte aligned address that is never dereferenced
FAKE2 = 0x40000000  # far from FAKE: no overlap between buffers


def declared_functions():
    src = open(HEADER).read()
    return re.findall(r"CT_API\s+[\w\s\*]+?\b(ct_\w+)\s*\(", src)


def test_header_declares_the_entry_points():
    names = set(declared_functions())
    for n in ["ct_convT3d_scale_pool_bias", "ct_convT3d", "ct_avgpool3d", "ct_convT1d",
              "ct_convT_out_len", "ct_pool_out_len", "ct_status_str", "ct_last_error",
              "ct_version"]:
        assert n in names


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(ct.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in ct.h but not exported"


def test_version_and_status_strings():
    assert "gfx950" in ct.ct_version()
    assert ct.ct_status_str(0) == "CT_OK"
    assert ct.ct_status_str(1) == "CT_EINVAL"
    assert ct.ct_status_str(2) == "CT_EUNSUPPORTED"
    assert ct.ct_status_str(3) == "CT_EHIP"
    assert ct.ct_status_str(99) == "CT_UNKNOWN_STATUS"


def test_size_helpers_match_the_pages():
    assert ct.ct_convT_out_len(16, 3, 2, 1, 0, 1) == 31
    assert ct.ct_convT_out_len(32, 3, 2, 1, 0, 1) == 63
    assert ct.ct_pool_out_len(31, 2, 2, 0) == 15
    assert ct.ct_pool_out_len(63, 2, 0, 0) == 31        # stride 0 -> k
    assert ct.ct_pool_out_len(128, 3, 2, 1) == 64
    assert ct.ct_pool_out_len(256, 3, 2, 1) == 128
    assert ct.ct_convT_out_len(131072, 5, 1, 0, 0, 3) == 131084
    # the pooled size of the k3 s2 p1 + 2-pool chain is in - 1 for any size
    for n in range(2, 40):
        assert ct.ct_pool_out_len(ct.ct_convT_out_len(n, 3, 2, 1, 0, 1), 2, 2, 0) == n - 1
    # floor mode with a negative numerator
    assert ct.ct_pool_out_len(1, 3, 2, 0) == 0


def test_size_helpers_report_lengths_past_int64():
    i64max = 2**63 - 1
    # (in - 1) * stride alone is past int64; exact 128-bit evaluation gives -1
    assert ct.ct_convT_out_len(2**62, 3, 2**30, 0, 0, 1) == -1
    assert ct.ct_convT_out_len(2, 2**40, 1, 0, 0, 2**40) == -1
    # the largest representable length still comes back exactly
    assert ct.ct_convT_out_len(i64max, 1, 1, 0, 0, 1) == i64max
    assert ct.ct_convT_out_len(2**62, 1, 2, 0, 0, 1) == 2**63 - 1
    assert ct.ct_convT_out_len(2**62 + 1, 1, 2, 0, 0, 1) == -1
    # in + 2 * pad is past int64, the quotient is not
    assert ct.ct_pool_out_len(i64max, 4, 4, 2**30) == (i64max + 2**31 - 4) // 4 + 1
    assert ct.ct_pool_out_len(i64max, 1, 1, 2**30) == -1
    assert ct.ct_pool_out_len(-i64max - 1, 1, 1, 0) == -i64max - 1
    assert ct.ct_pool_out_len(-i64max - 1, 2, 1, 0) == -1


def fused(**kw):
    a = dict(x=FAKE, xd=ct.CT_F32, w=FAKE2, wd=ct.CT_F32, cb=None, b=None, s1=0.5, s2=1.0,
             N=2, Cin=3, D=8, H=16, W=16, Cout=16, k=3, stride=2, pad=1, out_pad=0,
             pool_k=2, pool_s=2, out=FAKE2 * 2, stream=None)
    a.update(kw)
    return ct.lib.ct_convT3d_scale_pool_bias(
        a["x"], a["xd"], a["w"], a["wd"], a["cb"], a["b"], a["s1"], a["s2"], a["N"], a["Cin"],
        a["D"], a["H"], a["W"], a["Cout"], a["k"], a["stride"], a["pad"], a["out_pad"],
        a["pool_k"], a["pool_s"], a["out"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), ct.CT_EINVAL),
    (dict(w=None), ct.CT_EINVAL),
    (dict(out=None), ct.CT_EINVAL),
    (dict(xd=7), ct.CT_EINVAL),
    (dict(N=0), ct.CT_EINVAL),
    (dict(Cin=-1), ct.CT_EINVAL),
    (dict(D=1), ct.CT_EINVAL),              # pooled depth 0: empty output
    (dict(W=1), ct.CT_EINVAL),
    (dict(stride=0), ct.CT_EINVAL),
    (dict(out_pad=2), ct.CT_EINVAL),                # out_pad must be < stride
    (dict(stride=1, out_pad=1), ct.CT_EINVAL),
    (dict(pad=-1), ct.CT_EINVAL),
    (dict(k=0), ct.CT_EINVAL),
    (dict(pool_k=0), ct.CT_EINVAL),
    (dict(pool_s=-1), ct.CT_EINVAL),
    (dict(pool_k=16, D=8), ct.CT_EINVAL),           # pool window longer than depth 15
    (dict(pad=9, D=8, k=3), ct.CT_EINVAL),          # conv output empty
    (dict(xd=ct.CT_BF16), ct.CT_EUNSUPPORTED),      # mixed dtypes
    (dict(x=FAKE + 2), ct.CT_EINVAL),               # fp32 x misaligned
    (dict(out=FAKE2 * 2 + 1), ct.CT_EINVAL),
    (dict(b=FAKE + 1), ct.CT_EINVAL),
    (dict(out=FAKE + 64), ct.CT_EINVAL),            # out overlaps x
    (dict(out=FAKE2 + 4), ct.CT_EINVAL),            # out overlaps w
    (dict(xd=ct.CT_BF16, wd=ct.CT_BF16, x=FAKE + 1), ct.CT_EINVAL),
    (dict(W=1 << 31), ct.CT_EUNSUPPORTED),          # beyond the kernels' index range
    (dict(Cout=(1 << 30) + 1), ct.CT_EUNSUPPORTED),
    (dict(k=1025, pad=600, D=600, H=600, W=600, N=1, Cin=1, Cout=1, out=1 << 44),
     ct.CT_EUNSUPPORTED),
    (dict(pool_k=1025, pool_s=1, D=600, H=600, W=600, out=1 << 44), ct.CT_EUNSUPPORTED),
    (dict(N=1 << 60), ct.CT_EINVAL),                # byte size overflows int64
])
def test_fused_rejects(kw, status):
    assert fused(**kw) == status
    assert ct.ct_last_error() != ""


def pool(fn="ct_avgpool3d", **kw):
    a = dict(x=FAKE, N=16, C=32, D=128, H=128, W=256, k=3, stride=2, pad=1, cip=1,
             out=FAKE2 * 8, stream=None)
    a.update(kw)
    return getattr(ct.lib, fn)(a["x"], a["N"], a["C"], a["D"], a["H"], a["W"], a["k"],
                               a["stride"], a["pad"], a["cip"], a["out"], a["stream"])


POOL_REJECTS = [
    (dict(x=None), ct.CT_EINVAL),
    (dict(out=None), ct.CT_EINVAL),
    (dict(C=0), ct.CT_EINVAL),
    (dict(pad=2), ct.CT_EINVAL),                    # pad > k/2
    (dict(cip=2), ct.CT_EINVAL),
    (dict(k=5, pad=0, D=3, H=3, W=3), ct.CT_EINVAL),  # no window fits
    (dict(k=0), ct.CT_EINVAL),
    (dict(stride=-1), ct.CT_EINVAL),
    (dict(k=2, pad=0, N=1, C=1, D=2, H=2, W=(1 << 30) + 2, out=1 << 44),
     ct.CT_EUNSUPPORTED),                           # general kernel's index range
    (dict(k=1025, pad=0, N=1, C=1, D=2000, H=2000, W=2000, out=1 << 44), ct.CT_EUNSUPPORTED),
    (dict(x=FAKE + 1), ct.CT_EINVAL),               # misaligned for 4- and 2-byte elements
    (dict(out=FAKE + 4096), ct.CT_EINVAL),          # overlaps x
]


@pytest.mark.parametrize("kw,status", POOL_REJECTS)
def test_pool_rejects(kw, status):
    assert pool(**kw) == status


@pytest.mark.parametrize("kw,status", POOL_REJECTS)
def test_pool_bf16_rejects(kw, status):
    assert pool("ct_avgpool3d_bf16", **kw) == status
    assert ct.ct_last_error().startswith("avgpool3d_bf16")


def conv1d(**kw):
    a = dict(x=FAKE, xd=ct.CT_F32, w=FAKE2, wd=ct.CT_F32, b=None, N=32, Cin=32, L=131072,
             Cout=64, K=5, stride=1, pad=0, dil=3, out_pad=0, out=FAKE2 * 8, stream=None)
    a.update(kw)
    return ct.lib.ct_convT1d(a["x"], a["xd"], a["w"], a["wd"], a["b"], a["N"], a["Cin"], a["L"],
                             a["Cout"], a["K"], a["stride"], a["pad"], a["dil"], a["out_pad"],
                             a["out"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), ct.CT_EINVAL),
    (dict(w=None), ct.CT_EINVAL),
    (dict(L=0), ct.CT_EINVAL),
    (dict(K=0), ct.CT_EINVAL),
    (dict(dil=0), ct.CT_EINVAL),
    (dict(pad=5, L=2, K=2, dil=1), ct.CT_EINVAL),   # empty output
    (dict(stride=0), ct.CT_EINVAL),
    (dict(pad=-1), ct.CT_EINVAL),
    (dict(out_pad=3), ct.CT_EINVAL),                # out_pad must be < max(stride, dilation)
    (dict(out_pad=4, stride=4, dil=1), ct.CT_EINVAL),
    (dict(xd=ct.CT_BF16), ct.CT_EUNSUPPORTED),      # mixed dtypes
    (dict(L=(1 << 30) + 1, stride=2, N=1, Cin=1, out=1 << 44),
     ct.CT_EUNSUPPORTED),                           # general kernel's index range
    (dict(dil=1 << 29, K=5), ct.CT_EUNSUPPORTED),
    (dict(x=FAKE + 2), ct.CT_EINVAL),
    (dict(xd=ct.CT_BF16, wd=ct.CT_BF16, x=FAKE + 1), ct.CT_EINVAL),
    (dict(out=FAKE2 + 8), ct.CT_EINVAL),            # overlaps w
])
def test_conv1d_rejects(kw, status):
    assert conv1d(**kw) == status


def convT3d(**kw):
    a = dict(x=FAKE, xd=ct.CT_F32, w=FAKE2, wd=ct.CT_F32, b=None, N=2, Cin=3, D=8, H=16, W=16,
             Cout=16, k=3, stride=2, pad=1, out_pad=0, out=FAKE2 * 2, stream=None)
    a.update(kw)
    return ct.lib.ct_convT3d(a["x"], a["xd"], a["w"], a["wd"], a["b"], a["N"], a["Cin"], a["D"],
                             a["H"], a["W"], a["Cout"], a["k"], a["stride"], a["pad"],
                             a["out_pad"], a["out"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), ct.CT_EINVAL),
    (dict(out=None), ct.CT_EINVAL),
    (dict(wd=9), ct.CT_EINVAL),
    (dict(H=0), ct.CT_EINVAL),
    (dict(stride=0), ct.CT_EINVAL),
    (dict(out_pad=2), ct.CT_EINVAL),
    (dict(pad=3, k=3, D=1), ct.CT_EINVAL),          # conv output empty
    (dict(b=FAKE + 2), ct.CT_EINVAL),
    (dict(out=FAKE + 128), ct.CT_EINVAL),           # overlaps x
    (dict(wd=ct.CT_BF16), ct.CT_EUNSUPPORTED),      # mixed dtypes
    (dict(D=1 << 31), ct.CT_EUNSUPPORTED),
])
def test_convT3d_rejects(kw, status):
    assert convT3d(**kw) == status
    assert ct.ct_last_error().startswith("convT3d")


def test_python_binding_requires_gpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 4, 4)
    with pytest.raises(ValueError):
        ct.ct_avgpool3d(x, out=torch.zeros(1, 1, 2, 2, 2))


def test_forwarding_module_reaches_the_library():
    """The CPython module _ctcall forwards each compute call to the same C
    entry point (argument order of ct.h): null buffers come back as CT_EINVAL
    with the entry point's own message."""
    call = ct._call
    assert call is not None, "transposed_conv_pooling_amd._ctcall is not built"
    cases = [
        (call.fused, (0, ct.CT_F32, FAKE, ct.CT_F32, 0, 0, 0.5, 1.0, 2, 3, 8, 16, 16, 16,
                      3, 2, 1, 0, 2, 0, FAKE2, 0), "convT3d_scale_pool_bias"),
        (call.convT3d, (FAKE, ct.CT_F32, 0, ct.CT_F32, 0, 1, 1, 1, 1, 1, 1, 3, 2, 1, 0, FAKE2, 0),
         "convT3d"),
        (call.avgpool3d, (False, FAKE, 1, 1, 2, 2, 4, 3, 2, 1, 1, 0, 0), "avgpool3d"),
        (call.avgpool3d, (True, 0, 1, 1, 2, 2, 4, 3, 2, 1, 1, FAKE2, 0), "avgpool3d_bf16"),
        (call.convT1d, (FAKE, ct.CT_F32, FAKE2, ct.CT_F32, 0, 1, 1, 8, 1, 3, 1, 0, 1, 0, 0, 0),
         "convT1d"),
    ]
    for fn, args, name in cases:
        assert fn(*args) == ct.CT_EINVAL, name
        assert ct.ct_last_error().startswith(name + ":"), (name, ct.ct_last_error())
