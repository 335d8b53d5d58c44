"""NaN and infinity propagation on every operation, against the fp64 oracle.

A non-finite input must reach exactly the outputs whose definition contains
it ([p46]'s window sum, [p74]'s gather sum, [p50]'s chain), and every other
output must stay finite and within the usual tolerance.

Where an output holds a single non-finite term (the pool window sums, and the
1D conv, whose output o takes at most one product from a given input element),
the NaN / +-Inf pattern is unique and must match exactly.  The fused chain sums
the pre-pool values Inf * w over taps of both signs (the oracle gets NaN or
+-Inf depending on the weights), while the kernels first group the weights
(Inf * Weff); the two orders are equal only for finite values, so for an
infinite input only the set of non-finite outputs is compared.  A NaN input
gives NaN under any order and is compared exactly.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (assert_close_nonfinite, bf16_round, bf16_tensor_to_f32, log, nan_like,
                      opt, to_dev)

torch = pytest.importorskip("torch")
import transposed_conv_pooling_amd as ct  # noqa: E402

pytestmark = pytest.mark.gpu

F32_TOL = (1e-4, 1e-5)
BF16_TOL = (1e-4, 2e-2)
POOL_BF16_TOL = (1e-5, 2.0 ** -8)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def plant(x, spots):
    x = x.copy()
    for idx, v in spots:
        x[idx] = v
    return x


POOL_SPOTS = [((0, 1, 4, 7, 10), np.nan), ((1, 0, 2, 3, 33), np.inf),
              ((1, 1, 8, 19, 63), -np.inf), ((0, 0, 0, 0, 0), np.inf)]


@pytest.mark.parametrize("include_pad", [True, False], ids=["pad27", "validtaps"])
@pytest.mark.parametrize("shift", [0, 1], ids=["vector", "element"])
def test_pool_f32_nonfinite(dev, include_pad, shift):
    shape = (2, 2, 9, 20, 64)
    log(f"pool f32 nonfinite include_pad={include_pad} shift={shift}")
    x = plant(synth.normal(41, 0, shape), POOL_SPOTS)
    buf = torch.zeros(x.size + shift, dtype=torch.float32, device=dev)
    buf[shift:] = torch.from_numpy(x.reshape(-1)).to(dev)
    out = nan_like((2, 2, 5, 10, 32), dev)
    ct.ct_avgpool3d(buf[shift:].view(shape), 3, 2, 1, include_pad, out=out)
    torch.cuda.synchronize()
    ref = oracle.avgpool3d(x, 3, 2, 1, include_pad)
    assert (~np.isfinite(ref)).sum() >= 4
    assert_close_nonfinite(out.cpu().numpy(), ref, F32_TOL, "pool f32")


@pytest.mark.parametrize("shift", [0, 1], ids=["vector", "element"])
def test_pool_bf16_nonfinite(dev, shift):
    shape = (2, 2, 9, 20, 64)
    log(f"pool bf16 nonfinite shift={shift}")
    x = plant(bf16_round(synth.normal(42, 0, shape)), POOL_SPOTS)
    bits = torch.from_numpy(synth.to_bf16_bits(x).reshape(-1).view(np.int16))
    buf = torch.zeros(bits.numel() + shift, dtype=torch.int16, device=dev)
    buf[shift:] = bits.to(dev)
    out = nan_like((2, 2, 5, 10, 32), dev, torch.bfloat16)
    ct.ct_avgpool3d(buf[shift:].view(torch.bfloat16).view(shape), 3, 2, 1, True, out=out)
    torch.cuda.synchronize()
    ref = oracle.avgpool3d(x, 3, 2, 1, True)
    assert_close_nonfinite(bf16_tensor_to_f32(out), ref, POOL_BF16_TOL, "pool bf16")


CONV1D_SPOTS = [((0, 3, 100), np.nan), ((1, 7, 650), np.inf), ((0, 31, 0), -np.inf),
                ((1, 0, 699), np.inf)]


@pytest.mark.parametrize("geom", [(1, 0, 0), (2, 1, 1)], ids=["stride1", "stride2"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv1d_nonfinite(dev, dtype, geom):
    stride, pad, op = geom
    N, Cin, Cout, L, K, d = 2, 32, 64, 704, 5, 3    # L % 8 == 0: the matrix-core kernels
    log(f"conv1d nonfinite {dtype} stride={stride}")
    x = synth.normal(43, 0, (N, Cin, L))
    w = synth.uniform(43, 1, (Cin, Cout, K), -0.08, 0.08)
    if dtype == "bf16":
        x, w = bf16_round(x), bf16_round(w)
    x = plant(x, CONV1D_SPOTS)
    b = synth.normal(43, 2, (Cout,))
    Lo = (L - 1) * stride - 2 * pad + d * (K - 1) + op + 1
    out = nan_like((N, Cout, Lo), dev)
    ct.ct_convT1d(to_dev(x, dev, dtype), to_dev(w, dev, dtype), opt(b, dev), stride, pad, d, op,
                  out=out)
    torch.cuda.synchronize()
    ref = oracle.convT1d(x, w, b, stride, pad, d, op)
    assert (~np.isfinite(ref)).sum() >= 4 * Cout
    assert_close_nonfinite(out.cpu().numpy(), ref, F32_TOL, f"conv1d {dtype}")


@pytest.mark.parametrize("spot", ["nan", "inf"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_nonfinite(dev, dtype, spot):
    N, Cin, Cout, D, H, W = (2, 32, 64, 4, 9, 32) if dtype == "bf16" else (2, 3, 16, 4, 9, 32)
    log(f"fused nonfinite {dtype} {spot}")
    x = synth.normal(44, 0, (N, Cin, D, H, W))
    bnd = 1.0 / np.sqrt(Cin * 27)
    w = synth.uniform(44, 1, (Cin, Cout, 3, 3, 3), -bnd, bnd)
    if dtype == "bf16":
        x, w = bf16_round(x), bf16_round(w)
    v = np.nan if spot == "nan" else np.inf
    x = plant(x, [((0, 1, 2, 4, 17), v), ((1, Cin - 1, 0, 0, 0), -v), ((1, 0, 3, 8, 31), v)])
    b = synth.normal(44, 2, (Cout,))
    out = nan_like((N, Cout, D - 1, H - 1, W - 1), dev)
    ct.ct_convT3d_scale_pool_bias(to_dev(x, dev, dtype), to_dev(w, dev, dtype), None, opt(b, dev),
                                  0.5, 1.0, out=out)
    torch.cuda.synchronize()
    ref = oracle.convT3d_scale_pool_bias(x, w, None, b, 0.5, 1.0)
    # each planted input reaches every channel of the 1..8 pooled voxels whose taps hold it
    assert (~np.isfinite(ref)).sum() == Cout * (8 + 1 + 1)
    assert_close_nonfinite(out.cpu().numpy(), ref, F32_TOL if dtype == "f32" else BF16_TOL,
                           f"fused {dtype}", exact_nonfinite=(spot == "nan"))
