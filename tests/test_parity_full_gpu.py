"""Every element of each full-size workload against the fp64 oracle, in the
launch configuration the bench times.

Outputs are NaN-prefilled, copied to the host once, and compared slice by
slice (pool) or batch item by batch item (convolutions) with the oracle run on
the same slices, so host memory stays bounded.  Tolerances as elsewhere:
fp32 inputs |g - r| <= 1e-4 + 1e-5 |r|; bf16 inputs 1e-4 + 2e-2 |r| (plus the
tight 1e-4 + 1e-4 |r| bound the hi/lo filter split keeps); bf16 pooling data
1e-5 + 2^-8 |r|.

Workloads ([p50] fused chain, [p46] AvgPool3d, [p74] ConvTranspose1d):
  fused fp32   [128,3,16,32,32] -> [128,16,15,31,31]   (test_parity_gpu.py)
  pool         [16,32,128,128,256] -> [16,32,64,64,128], fp32 and bf16 data,
               count_include_pad True and False
  conv1d       [32,32,131072] -> [32,64,131084], fp32 and bf16 inputs; stride 2,
               pad 1, output_padding 1 with a bias -> [32,64,262154]
  fused bf16   [16,32,16,32,32] -> [16,64,15,31,31]
  fused f32    [128,3,16,32,32] with a conv bias and output_padding 1
               -> [128,16,16,32,32]
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, bf16_round, bf16_tensor_to_f32, log, nan_like, opt, to_dev

torch = pytest.importorskip("torch")
import transposed_conv_pooling_amd as ct  # noqa: E402

pytestmark = pytest.mark.gpu

F32_TOL = (1e-4, 1e-5)
BF16_TOL = (1e-4, 2e-2)
TIGHT_TOL = (1e-4, 1e-4)
POOL_BF16_TOL = (1e-5, 2.0 ** -8)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def pool_x():
    """The [16,32,128,128,256] pooling input (2^31 fp32 values), drawn once."""
    wl = synth.WORKLOADS["c3"]
    log(wl.description + ": drawing 8.6 GB")
    return synth.normal(wl.seed, synth.STREAM_X, wl.x_shape)


def compare_pool(got, xs, include_pad, tol, what, chunk=64):
    """got: host [512, 64, 64, 128]; xs(i, j) -> input slices i..j as fp32."""
    for i in range(0, got.shape[0], chunk):
        ref = oracle.avgpool3d(xs(i, i + chunk), 3, 2, 1, include_pad)
        assert_close(got[i:i + chunk], ref, tol, f"{what} slices {i}..{i + chunk - 1}")


@pytest.mark.parametrize("include_pad", [True, False], ids=["pad27", "validtaps"])
def test_pool_f32_full_every_slice(dev, pool_x, include_pad):
    log(f"pool fp32 full, count_include_pad={include_pad}")
    xg = torch.from_numpy(pool_x).to(dev)
    out = nan_like((16, 32, 64, 64, 128), dev)
    ct.ct_avgpool3d(xg, 3, 2, 1, include_pad, out=out)
    torch.cuda.synchronize()
    del xg
    got = out.cpu().numpy().reshape(512, 64, 64, 128)
    del out
    xr = pool_x.reshape(512, 128, 128, 256)
    compare_pool(got, lambda i, j: xr[i:j], include_pad, F32_TOL, "pool fp32")


def test_pool_bf16_full_every_slice(dev, pool_x):
    log("pool bf16 full")
    bits = synth.to_bf16_bits(pool_x).reshape(512, 128, 128, 256)
    xg = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16).view(16, 32, 128, 128, 256)
    out = nan_like((16, 32, 64, 64, 128), dev, torch.bfloat16)
    ct.ct_avgpool3d(xg, 3, 2, 1, True, out=out)
    torch.cuda.synchronize()
    del xg
    got = bf16_tensor_to_f32(out).reshape(512, 64, 64, 128)
    del out

    def xs(i, j):
        b = bits[i:j]
        return synth.bf16_bits_to_f32(b).reshape(b.shape)
    compare_pool(got, xs, True, POOL_BF16_TOL, "pool bf16")


def compare_items(got, ref_fn, n_items, chunk, tols, what):
    for i in range(0, n_items, chunk):
        ref = ref_fn(i, min(i + chunk, n_items))
        for tol in tols:
            assert_close(got[i:i + chunk], ref, tol, f"{what} items {i}..{i + chunk - 1}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv1d_full_every_item(dev, dtype):
    wl = synth.WORKLOADS["c4"]
    log(f"{wl.description} ({dtype} inputs)")
    t = synth.make_inputs(wl)
    x, w = t["x"], t["w"]
    if dtype == "bf16":
        x = synth.bf16_bits_to_f32(synth.to_bf16_bits(x)).reshape(x.shape)
        w = synth.bf16_bits_to_f32(synth.to_bf16_bits(w)).reshape(w.shape)
    out = nan_like((32, 64, 131084), dev)
    ct.ct_convT1d(to_dev(x, dev, dtype), to_dev(w, dev, dtype), None, 1, 0, 3, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    del out
    # bf16 products are exact in the fp32 accumulator: the fp32 bound applies
    compare_items(got, lambda i, j: oracle.convT1d(x[i:j], w, None, 1, 0, 3), 32, 8,
                  [F32_TOL], f"conv1d {dtype}")


def test_conv1d_stride2_full_every_item(dev):
    """stride 2, pad 1, output_padding 1, dilation 3, with a bias."""
    wl = synth.WORKLOADS["c4"]
    t = synth.make_inputs(wl, conv_bias=True)
    log(wl.description + ", stride 2, pad 1, output_padding 1, bias")
    out = nan_like((32, 64, 262154), dev)
    ct.ct_convT1d(to_dev(t["x"], dev), to_dev(t["w"], dev), opt(t["bias"], dev), 2, 1, 3, 1,
                  out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    del out
    compare_items(got, lambda i, j: oracle.convT1d(t["x"][i:j], t["w"], t["bias"], 2, 1, 3, 1),
                  32, 4, [F32_TOL], "conv1d stride 2")


def test_fused_bf16_full_every_item(dev):
    wl = synth.WORKLOADS["c5"]
    log(wl.description)
    t = synth.make_inputs(wl)
    xg = torch.from_numpy(t["x_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    wg = torch.from_numpy(t["w_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    out = nan_like((16, 64, 15, 31, 31), dev)
    ct.ct_convT3d_scale_pool_bias(xg, wg, None, opt(t["bias"], dev), 0.5, 1.0, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    compare_items(got, lambda i, j: oracle.convT3d_scale_pool_bias(
        t["x"][i:j], t["w"], None, t["bias"], 0.5, 1.0), 16, 16, [BF16_TOL, TIGHT_TOL], "c5")


def test_fused_outpad1_full_every_item(dev):
    """[128,3,16,32,32] with a conv bias and output_padding=1 -> [128,16,16,32,32]."""
    wl = synth.WORKLOADS["c2"]
    t = synth.make_inputs(wl, conv_bias=True)
    log(wl.description + ", conv bias, output_padding=1")
    out = nan_like((128, 16, 16, 32, 32), dev)
    ct.ct_convT3d_scale_pool_bias(to_dev(t["x"], dev), to_dev(t["w"], dev),
                                  opt(t["conv_bias"], dev), opt(t["bias"], dev), 0.5, 1.0,
                                  2, 1, 1, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    compare_items(got, lambda i, j: oracle.convT3d_scale_pool_bias(
        t["x"][i:j], t["w"], t["conv_bias"], t["bias"], 0.5, 1.0, 2, 1, 1), 128, 32,
        [F32_TOL], "fused output_padding=1")


def test_fused_bf16_direct_full_every_item(dev):
    """The bf16 chain at the wide workload's size where the bf16 kernel does not
    apply (W = 31, output_padding = 1 and a conv bias): the direct kernel with
    the taps widened to fp32, every element against the oracle."""
    N, Cin, Cout, D, H, W = 16, 32, 64, 16, 32, 31
    log(f"fused bf16 direct [{N},{Cin},{D},{H},{W}] -> Cout {Cout}, output_padding 1, conv bias")
    x = bf16_round(synth.normal(0x5EED0015, 0, (N, Cin, D, H, W)))
    bound = 1.0 / np.sqrt(Cin * 27)
    w = bf16_round(synth.uniform(0x5EED0015, 1, (Cin, Cout, 3, 3, 3), -bound, bound))
    b = synth.normal(0x5EED0015, 2, (Cout,))
    cb = synth.normal(0x5EED0015, 3, (Cout,))
    out = nan_like((N, Cout, D, H, W), dev)
    ct.ct_convT3d_scale_pool_bias(to_dev(x, dev, "bf16"), to_dev(w, dev, "bf16"), opt(cb, dev),
                                  opt(b, dev), 0.5, 1.0, 2, 1, 1, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    compare_items(got, lambda i, j: oracle.convT3d_scale_pool_bias(
        x[i:j], w, cb, b, 0.5, 1.0, 2, 1, 1), N, 16, [BF16_TOL, TIGHT_TOL], "bf16 direct")
