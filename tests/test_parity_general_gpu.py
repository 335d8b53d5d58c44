"""Parity of the general-geometry paths (everything outside the pages' own
k3 s2 p1 / 2-pool, k3 s2 p1 / divisor-27 and stride-1 fp32 cases) with the
fp64 CPU oracle, through the C ABI.

Same tolerances as the specialised paths: fp32 inputs atol 1e-4, rtol 1e-5;
bf16 inputs atol 1e-4, rtol 2e-2, with the oracle fed the identical
bf16-rounded values.  Outputs are NaN-prefilled so an unwritten element fails.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import transposed_conv_pooling_amd as ct  # noqa: E402

pytestmark = pytest.mark.gpu

F32_TOL = (1e-4, 1e-5)
BF16_TOL = (1e-4, 2e-2)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def assert_close(got, ref, tol, what=""):
    atol, rtol = tol
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    ok = err <= atol + rtol * np.abs(ref)
    if not ok.all():
        idx = np.argwhere(~ok)
        i0 = tuple(idx[0])
        raise AssertionError(
            f"{what}: {len(idx)} of {ok.size} elements out of tolerance; first at {i0}: "
            f"gpu={got[i0]!r} oracle={ref[i0]!r}; max err {np.nanmax(err):.3g}")


def log(msg):
    print(msg, flush=True)


def bf16_round(a):
    return synth.bf16_bits_to_f32(synth.to_bf16_bits(a)).reshape(a.shape)


def to_dev(a, dev, dtype):
    if dtype == "bf16":
        return torch.from_numpy(synth.to_bf16_bits(a).reshape(a.shape).view(np.int16)).to(
            dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def opt(a, dev):
    return None if a is None else torch.from_numpy(a).to(dev)


# ------------------------------------------------ fused, general geometry ----
FUSED_GENERAL = [
    # N, Cin, Cout, D, H, W, k, stride, pad, out_pad, pool_k, pool_s, dtype
    (2, 3, 16, 5, 7, 9, 3, 2, 1, 1, 2, 2, "f32"),     # output_padding 1
    (2, 3, 16, 5, 7, 9, 3, 2, 1, 1, 2, 2, "bf16"),  # bf16 with output padding: the direct kernel
    (1, 4, 6, 4, 5, 6, 4, 2, 1, 0, 2, 2, "f32"),      # even kernel
    (1, 3, 5, 4, 6, 7, 3, 1, 0, 0, 3, 2, "f32"),      # stride 1, 3-pool with stride 2
    (2, 2, 3, 3, 4, 5, 5, 3, 2, 2, 2, 1, "f32"),      # overlapping pool windows
    (1, 5, 7, 3, 3, 4, 2, 2, 0, 0, 2, 2, "f32"),      # non-overlapping taps
    (1, 2, 3, 4, 5, 6, 1, 1, 0, 0, 1, 1, "f32"),      # 1x1x1 conv, identity pool
    (1, 3, 4, 3, 4, 5, 3, 2, 1, 0, 3, 3, "bf16"),
    (1, 130, 4, 3, 3, 5, 3, 2, 1, 0, 2, 2, "f32"),    # page geometry, Cin beyond the MFMA path
    (1, 40, 8, 3, 4, 8, 3, 2, 1, 0, 2, 2, "bf16"),    # page geometry, bf16 Cin > 32: direct kernel
    (2, 3, 16, 4, 5, 13, 3, 2, 1, 0, 2, 2, "bf16"),   # page geometry, bf16 W % 8 != 0: direct kernel
    (2, 3, 16, 9, 17, 33, 3, 2, 1, 1, 2, 2, "f32"),   # output_padding 1, scalar slab rows (W % 4 != 0)
    (1, 40, 40, 3, 3, 4, 3, 2, 1, 1, 2, 2, "f32"),    # output_padding 1, Cin > 4: the direct kernel
    (1, 130, 4, 3, 3, 5, 3, 2, 1, 1, 2, 2, "f32"),    # Cin > 128: the effective-filter gather
    (1, 130, 40, 3, 3, 5, 3, 2, 1, 0, 2, 2, "f32"),   # Cin*Cout > 1024 as well: the plain gather
    # output_padding 1 on the fp32 slab kernel (Cin <= 4): far-edge taps read 0,
    # float4 rows (W % 4 == 0) and scalar rows, several tasks per workgroup
    (2, 3, 16, 6, 10, 16, 3, 2, 1, 1, 2, 2, "f32"),
    (1, 4, 20, 3, 9, 8, 3, 2, 1, 1, 2, 2, "f32"),     # ragged Cout
    (3, 1, 16, 4, 33, 32, 3, 2, 1, 1, 2, 2, "f32"),
    (1, 2, 5, 2, 2, 4, 3, 2, 1, 1, 2, 2, "f32"),      # one input plane pair
    (5, 3, 16, 7, 20, 23, 3, 2, 1, 1, 2, 2, "f32"),   # scalar rows, ragged W
    (2, 3, 16, 1, 1, 1, 3, 2, 1, 1, 2, 2, "f32"),     # a single input voxel
    # Cin 3, W 32 with output padding 1: the compiled-in geometry (7 rows per task)
    (2, 3, 16, 4, 9, 32, 3, 2, 1, 1, 2, 2, "f32"),
    (3, 3, 16, 5, 20, 32, 3, 2, 1, 1, 2, 2, "f32"),
    (1, 3, 24, 3, 7, 32, 3, 2, 1, 1, 2, 2, "f32"),
]


@pytest.mark.parametrize("case", FUSED_GENERAL, ids=lambda c: "x".join(map(str, c)))
def test_fused_general(dev, case):
    N, Cin, Cout, D, H, W, k, s, p, op, pk, ps, dt = case
    log(f"fused general {case}")
    seed = 5000 + sum(c for c in case if isinstance(c, int))
    x = synth.normal(seed, 0, (N, Cin, D, H, W))
    bound = 1.0 / np.sqrt(Cin * k ** 3)
    w = synth.uniform(seed, 1, (Cin, Cout, k, k, k), -bound, bound)
    if dt == "bf16":
        x, w = bf16_round(x), bf16_round(w)
    b = synth.normal(seed, 2, (Cout,))
    cb = synth.normal(seed, 3, (Cout,))
    ref = oracle.convT3d_scale_pool_bias(x, w, cb, b, 0.5, 1.25, stride=s, pad=p, out_pad=op,
                                         pool_k=pk, pool_s=ps)
    out = torch.full(ref.shape, float("nan"), dtype=torch.float32, device=dev)
    ct.ct_convT3d_scale_pool_bias(to_dev(x, dev, dt), to_dev(w, dev, dt), opt(cb, dev),
                                  opt(b, dev), 0.5, 1.25, stride=s, pad=p, out_pad=op,
                                  pool_k=pk, pool_s=ps, out=out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, F32_TOL if dt == "f32" else BF16_TOL, str(case))


def test_fused_bf16_misaligned_x_takes_direct_path(dev):
    shape = (1, 8, 3, 4, 16)
    x = bf16_round(synth.normal(71, 0, shape))
    w = bf16_round(synth.uniform(71, 1, (8, 16, 3, 3, 3), -0.1, 0.1))
    b = synth.normal(71, 2, (16,))
    buf = torch.empty(x.size + 1, dtype=torch.bfloat16, device=dev)
    buf[1:] = to_dev(x.reshape(-1), dev, "bf16")
    xg = buf[1:].view(shape)                        # 2-byte but not 16-byte aligned
    out = torch.full((1, 16, 2, 3, 15), float("nan"), dtype=torch.float32, device=dev)
    ct.ct_convT3d_scale_pool_bias(xg, to_dev(w, dev, "bf16"), None, opt(b, dev), 0.5, 1.0,
                                  out=out)
    torch.cuda.synchronize()
    ref = oracle.convT3d_scale_pool_bias(x, w, None, b, 0.5, 1.0)
    assert_close(out.cpu().numpy(), ref, BF16_TOL, "bf16 misaligned")


def test_fused_bf16_misaligned_w_takes_chunked_weights(dev):
    # 32 input channels, 64 output channels, weights 2-byte but not 16-byte
    # aligned: the filter is formed from the raw weights staged in LDS in
    # 16-channel chunks instead of the whole-line weight reads
    shape = (2, 32, 3, 5, 32)
    x = bf16_round(synth.normal(73, 0, shape))
    w = bf16_round(synth.uniform(73, 1, (32, 64, 3, 3, 3), -0.03, 0.03))
    b = synth.normal(73, 2, (64,))
    buf = torch.empty(w.size + 1, dtype=torch.bfloat16, device=dev)
    buf[1:] = to_dev(w.reshape(-1), dev, "bf16")
    wg = buf[1:].view(w.shape)
    out = torch.full((2, 64, 2, 4, 31), float("nan"), dtype=torch.float32, device=dev)
    ct.ct_convT3d_scale_pool_bias(to_dev(x, dev, "bf16"), wg, None, opt(b, dev), 0.5, 1.0,
                                  out=out)
    torch.cuda.synchronize()
    ref = oracle.convT3d_scale_pool_bias(x, w, None, b, 0.5, 1.0)
    assert_close(out.cpu().numpy(), ref, BF16_TOL, "bf16 misaligned w")


# ------------------------------------------------- standalone ConvTranspose3d ----
CONVT3D = [
    # N, Cin, Cout, D, H, W, k, stride, pad, out_pad, bias, dtype
    (2, 3, 16, 8, 16, 16, 3, 2, 1, 0, False, "f32"),  # the page's first layer at the small size
    (1, 3, 5, 4, 5, 6, 3, 2, 1, 1, True, "f32"),
    (1, 2, 3, 3, 4, 5, 4, 3, 1, 2, True, "f32"),
    (1, 4, 4, 3, 3, 3, 2, 1, 0, 0, False, "f32"),
    (2, 5, 6, 4, 4, 6, 3, 2, 1, 0, True, "bf16"),
    # the k3 s2 p1 parity kernel (Cin <= 8), both output paddings, edges
    (2, 3, 16, 5, 7, 9, 3, 2, 1, 1, True, "f32"),
    (1, 8, 5, 3, 4, 70, 3, 2, 1, 0, False, "f32"),
    (1, 1, 1, 1, 1, 1, 3, 2, 1, 0, False, "f32"),
    (1, 2, 3, 1, 2, 1, 3, 2, 1, 1, True, "f32"),
    (2, 7, 4, 3, 5, 6, 3, 2, 1, 1, True, "bf16"),
    (1, 9, 4, 3, 3, 4, 3, 2, 1, 0, True, "f32"),      # Cin 9: general kernel
]


@pytest.mark.parametrize("case", CONVT3D, ids=lambda c: "x".join(map(str, c)))
def test_convT3d(dev, case):
    N, Cin, Cout, D, H, W, k, s, p, op, with_bias, dt = case
    log(f"convT3d {case}")
    seed = 6000 + sum(c for c in case if isinstance(c, int))
    x = synth.normal(seed, 0, (N, Cin, D, H, W))
    bound = 1.0 / np.sqrt(Cin * k ** 3)
    w = synth.uniform(seed, 1, (Cin, Cout, k, k, k), -bound, bound)
    if dt == "bf16":
        x, w = bf16_round(x), bf16_round(w)
    b = synth.normal(seed, 2, (Cout,)) if with_bias else None
    ref = oracle.convT3d(x, w, b, stride=s, pad=p, out_pad=op)
    out = torch.full(ref.shape, float("nan"), dtype=torch.float32, device=dev)
    ct.ct_convT3d(to_dev(x, dev, dt), to_dev(w, dev, dt), opt(b, dev), stride=s, pad=p,
                  out_pad=op, out=out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, F32_TOL if dt == "f32" else BF16_TOL, str(case))


def test_unfused_chain_c2_matches_fused(dev):
    """The pages' unfused baseline at full size: ConvTranspose3d materialises
    [128,16,31,63,63] (1.0 GB), then a 2-pool; the scaled, biased result equals
    the fused kernel's.  Batch items 0 and 127 of the pre-pool tensor are also
    recomputed by the oracle."""
    wl = synth.WORKLOADS["c2"]
    log(wl.description)
    t = synth.make_inputs(wl)
    xg, wg = torch.from_numpy(t["x"]).to(dev), torch.from_numpy(t["w"]).to(dev)
    bg = torch.from_numpy(t["bias"]).to(dev)
    y = torch.full((128, 16, 31, 63, 63), float("nan"), dtype=torch.float32, device=dev)
    ct.ct_convT3d(xg, wg, None, out=y)
    pooled = torch.full((128, 16, 15, 31, 31), float("nan"), dtype=torch.float32, device=dev)
    ct.ct_avgpool3d(y, 2, 2, 0, True, out=pooled)
    fused = ct.ct_convT3d_scale_pool_bias(xg, wg, None, bg, 0.5, 1.0)
    torch.cuda.synchronize()
    for n in (0, 127):
        ref = oracle.convT3d(t["x"][n:n + 1], t["w"], None, stride=2, pad=1)
        assert_close(y[n:n + 1].cpu().numpy(), ref, F32_TOL, f"c2 convT3d n={n}")
    unfused = (pooled * 0.5 + bg.view(1, 16, 1, 1, 1)) * 1.0
    assert_close(unfused.cpu().numpy(), fused.cpu().numpy().astype(np.float64), F32_TOL,
                 "unfused vs fused")


# ------------------------------------------------- pool, general geometry ----
POOL_GENERAL = [
    # shape, k, stride, pad, count_include_pad
    ((2, 3, 9, 10, 13), 3, 2, 1, False),    # the page's window, valid-tap divisor
    ((1, 2, 8, 9, 10), 2, 2, 0, True),      # the fused chain's pool, standalone
    ((1, 2, 7, 6, 11), 3, 1, 1, True),
    ((1, 1, 11, 12, 13), 5, 3, 2, False),
    ((1, 1, 11, 12, 13), 5, 3, 2, True),
    ((2, 1, 9, 8, 7), 4, 0, 2, False),      # stride 0 -> k
    ((1, 1, 3, 4, 5), 1, 1, 0, True),       # identity
    ((1, 1, 1, 1, 1), 1, 2, 0, False),
    ((1, 2, 2, 3, 300), 2, 1, 1, False),
    # the page's window with the valid-tap divisor on the streaming kernels
    ((2, 5, 9, 10, 16), 3, 2, 1, False),     # small-plane kernel
    ((1, 2, 5, 6, 260), 3, 2, 1, False),
    ((40, 8, 12, 10, 16), 3, 2, 1, False),   # 320 slices, several per workgroup
    ((1, 1, 1, 1, 4), 3, 2, 1, False),       # length-1 axes: one valid tap
    ((1, 1, 2, 131, 8), 3, 2, 1, False),
    ((2, 3, 7, 9, 31), 3, 2, 1, False),      # small-plane kernel, element loads
    ((2, 5, 9, 70, 64), 3, 2, 1, False),     # vector kernel, one column chunk
    ((1, 2, 5, 18, 260), 3, 2, 1, False),    # vector kernel, two column chunks
    ((40, 8, 12, 34, 128), 3, 2, 1, False),  # 320 slices in plane ranges (bf16 staggered starts)
    ((1, 1, 2, 131, 40), 3, 2, 1, False),    # two row groups
    ((1, 2, 3, 70, 63), 3, 2, 1, False),     # element kernel
    ((1, 2, 3, 30, 1024), 3, 2, 1, False),   # vector kernel, 4 column groups
]


@pytest.mark.parametrize("case", POOL_GENERAL, ids=lambda c: "x".join(map(str, c[0])) +
                         f"_k{c[1]}s{c[2]}p{c[3]}c{int(c[4])}")
def test_pool_general(dev, case):
    shape, k, s, p, cip = case
    log(f"pool general {case}")
    x = synth.normal(7000 + sum(shape) + k, 0, shape)
    ref = oracle.avgpool3d(x, k, s if s else k, p, cip)
    out = torch.full(ref.shape, float("nan"), dtype=torch.float32, device=dev)
    ct.ct_avgpool3d(torch.from_numpy(x).to(dev), k, s, p, cip, out=out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, F32_TOL, str(case))


@pytest.mark.parametrize("case", POOL_GENERAL, ids=lambda c: "x".join(map(str, c[0])) +
                         f"_k{c[1]}s{c[2]}p{c[3]}c{int(c[4])}")
def test_pool_general_bf16(dev, case):
    """bf16 data on the general kernel: fp32 sums, each mean rounded to the
    nearest bf16 (within one bf16 step of the fp64 oracle on the same values)."""
    shape, k, s, p, cip = case
    log(f"pool general bf16 {case}")
    x = bf16_round(synth.normal(7500 + sum(shape) + k, 0, shape))
    ref = oracle.avgpool3d(x, k, s if s else k, p, cip)
    out = torch.full(ref.shape, float("nan"), dtype=torch.bfloat16, device=dev)
    ct.ct_avgpool3d(to_dev(x, dev, "bf16"), k, s, p, cip, out=out)
    torch.cuda.synchronize()
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    got = synth.bf16_bits_to_f32(o).reshape(o.shape)
    assert_close(got, ref, (1e-5, 2.0 ** -8), str(case))


def test_pool_valid_tap_divisor_border_values(dev):
    """count_include_pad off: an all-ones input averages to exactly 1 everywhere."""
    x = torch.ones((1, 1, 6, 7, 9), dtype=torch.float32, device=dev)
    out = ct.ct_avgpool3d(x, 3, 2, 1, False)
    torch.cuda.synchronize()
    assert bool((out == 1.0).all())


# ---------------------------------------------- convT1d, general geometry ----
CONV1D_GENERAL = [
    # N, Cin, Cout, L, K, stride, pad, dilation, out_pad, bias, dtype
    (2, 32, 64, 300, 5, 1, 0, 3, 0, False, "bf16"),  # the page's geometry in bf16
    (1, 4, 6, 37, 4, 2, 1, 1, 1, True, "f32"),
    (2, 3, 5, 29, 5, 3, 2, 2, 1, True, "f32"),
    (1, 5, 3, 40, 3, 1, 2, 3, 2, False, "f32"),      # out_pad < dilation
    (1, 2, 2, 1, 1, 1, 0, 1, 0, True, "f32"),
    (1, 8, 9, 50, 6, 4, 3, 2, 3, True, "bf16"),
    (1, 300, 8, 20, 3, 1, 0, 1, 0, False, "f32"),    # weights beyond the LDS tile
    # the residue-ordered gather (stride <= 8, L_out >= 64*stride)
    (2, 6, 7, 200, 5, 2, 1, 3, 1, True, "f32"),      # the stride-2 shape of the general bench op
    (1, 5, 3, 300, 4, 3, 2, 2, 2, False, "f32"),
    (2, 3, 4, 150, 3, 8, 0, 1, 7, True, "bf16"),     # largest stride it takes
    (1, 33, 65, 520, 5, 2, 1, 3, 1, True, "f32"),    # a partial group of four channels
    (1, 4, 3, 100, 2, 1, 5, 1, 0, False, "f32"),     # pad 5: early taps fall before the input
    # the bf16 matrix-core kernel (Cin 32, K 5, dilation 3, L % 8 == 0)
    (2, 32, 64, 296, 5, 1, 0, 3, 0, False, "bf16"),
    (1, 32, 70, 520, 5, 1, 0, 3, 0, True, "bf16"),    # two output-channel groups, ragged
    (1, 32, 16, 8, 5, 1, 0, 3, 0, True, "bf16"),      # shortest input
    (3, 32, 64, 1024, 5, 1, 0, 3, 0, True, "bf16"),   # several tiles per item
    (8, 32, 64, 40000, 5, 1, 0, 3, 0, True, "bf16"),  # more tiles than workgroups, ranges across items
    # stride 2 on the fp32 matrix cores: two stride-1 gathers (residues of
    # o + pad), pads of both parities, output padding up to 2, ragged tails
    (1, 32, 64, 4, 5, 2, 0, 3, 0, False, "f32"),      # shortest input
    (2, 32, 64, 64, 5, 2, 1, 3, 1, True, "f32"),
    (1, 32, 64, 100, 5, 2, 2, 3, 2, True, "f32"),
    (1, 32, 70, 520, 5, 2, 3, 3, 0, True, "f32"),     # two output-channel groups, ragged
    (1, 32, 16, 260, 5, 2, 5, 3, 1, False, "f32"),    # pad past the first tile's halo
    (1, 32, 64, 8, 5, 2, 9, 3, 2, True, "f32"),       # pad larger than the input
    (3, 32, 64, 1028, 5, 2, 1, 3, 1, True, "f32"),    # tiles straddling batch items
    (8, 32, 64, 20004, 5, 2, 1, 3, 1, True, "f32"),   # more tiles than waves: halos carried
    (8, 32, 64, 20004, 5, 2, 0, 3, 0, True, "f32"),   # even pad over many tiles
    (4, 32, 64, 20000, 5, 2, 2, 3, 1, False, "f32"),
    (4, 32, 64, 20000, 5, 2, 3, 3, 0, True, "f32"),   # odd output length: 4-byte aligned pairs
    (3, 32, 40, 4000, 5, 2, 4, 3, 2, True, "f32"),    # odd output length, even pad
    # stride 3 on the same kernel: three residue classes of o + pad (at
    # dilation 3 every tap falls in class 0; classes 1 and 2 are the bias),
    # 12-byte stores of three outputs, pads of every residue mod 3
    (1, 32, 64, 4, 5, 3, 0, 3, 0, False, "f32"),      # shortest input
    (2, 32, 64, 64, 5, 3, 1, 3, 1, True, "f32"),
    (1, 32, 64, 100, 5, 3, 2, 3, 2, True, "f32"),
    (1, 32, 70, 520, 5, 3, 3, 3, 0, True, "f32"),     # two output-channel groups, ragged
    (1, 32, 16, 260, 5, 3, 7, 3, 1, False, "f32"),    # pad past the first tile's halo
    (1, 32, 64, 8, 5, 3, 13, 3, 2, True, "f32"),      # pad larger than the input
    (3, 32, 64, 1028, 5, 3, 1, 3, 1, True, "f32"),    # tiles straddling batch items
    (8, 32, 64, 20004, 5, 3, 4, 3, 2, True, "f32"),   # more tiles than waves: halos carried
    (4, 32, 64, 20000, 5, 3, 0, 3, 0, True, "f32"),
    # stride 4: four classes (taps {0, 4}, {3}, {2}, {1}), 16-byte stores
    (1, 32, 64, 4, 5, 4, 0, 3, 0, False, "f32"),      # shortest input
    (2, 32, 64, 64, 5, 4, 1, 3, 1, True, "f32"),
    (1, 32, 70, 520, 5, 4, 3, 3, 2, True, "f32"),     # two output-channel groups, ragged
    (1, 32, 64, 8, 5, 4, 17, 3, 3, True, "f32"),      # pad larger than the input
    (3, 32, 64, 1028, 5, 4, 2, 3, 1, True, "f32"),    # tiles straddling batch items
    (8, 32, 64, 20004, 5, 4, 5, 3, 0, True, "f32"),   # more tiles than waves: halos carried
    # strides 5 to 8: 32-q tiles, a 16-byte store and one of 4 to 16 bytes
    # per lane and block; at 6 and above some classes have no tap (bias only)
    (1, 32, 64, 4, 5, 5, 0, 3, 0, False, "f32"),      # shortest input
    (2, 32, 70, 520, 5, 5, 3, 3, 4, True, "f32"),     # two output-channel groups, ragged
    (3, 32, 64, 1028, 5, 5, 7, 3, 2, True, "f32"),    # tiles straddling batch items
    (1, 32, 64, 8, 5, 6, 23, 3, 5, True, "f32"),      # pad larger than the input
    (2, 32, 64, 300, 5, 6, 1, 3, 1, False, "f32"),
    (4, 32, 64, 20000, 5, 6, 4, 3, 3, True, "f32"),   # more tiles than waves: halos carried
    (1, 32, 16, 260, 5, 7, 9, 3, 6, True, "f32"),
    (3, 32, 70, 1028, 5, 7, 2, 3, 0, True, "f32"),
    (1, 32, 64, 4, 5, 8, 0, 3, 7, False, "f32"),      # shortest input, largest output padding
    (2, 32, 64, 520, 5, 8, 5, 3, 1, True, "f32"),
    (8, 32, 64, 20004, 5, 8, 12, 3, 2, True, "f32"),  # more tiles than waves: halos carried
    # stride 1 with a pad or output padding on the fp32 matrix cores (the
    # unpadded kernel over a shifted output window; output length % 4 == 0):
    # pads of every residue mod 4, "same" padding, pad past the halo
    (2, 32, 64, 300, 5, 1, 2, 3, 0, True, "f32"),
    (1, 32, 70, 520, 5, 1, 1, 3, 2, True, "f32"),     # odd pad, two channel groups, ragged
    (2, 32, 64, 296, 5, 1, 6, 3, 0, False, "f32"),    # "same": output length = input length
    (1, 32, 16, 260, 5, 1, 3, 3, 2, True, "f32"),
    (1, 32, 64, 8, 5, 1, 5, 3, 2, True, "f32"),       # pad larger than half the input
    (3, 32, 64, 1028, 5, 1, 4, 3, 0, True, "f32"),    # tiles straddling batch items
    (8, 32, 64, 20004, 5, 1, 7, 3, 2, True, "f32"),   # more tiles than waves: halos carried
    # output length % 4 != 0: rows start at 4-byte boundaries, the row end's
    # partial vector stored element by element
    (1, 32, 64, 100, 5, 1, 1, 3, 0, True, "f32"),
    (2, 32, 70, 1000, 5, 1, 1, 3, 0, True, "f32"),    # two channel groups, several tiles
    (1, 32, 16, 260, 5, 1, 3, 3, 1, False, "f32"),
    (3, 32, 64, 1028, 5, 1, 0, 3, 1, True, "f32"),    # output padding alone, tiles across items
    (8, 32, 64, 20004, 5, 1, 0, 3, 2, True, "f32"),   # more tiles than waves
    (1, 32, 64, 8, 5, 1, 1, 3, 0, True, "f32"),       # one tile
    # stride 1 with a pad or output padding on the bf16 matrix cores (the
    # strip shifted by the pad rounded up to 8 positions): pads of several
    # residues mod 8, output lengths with and without 16-byte row starts
    (2, 32, 64, 296, 5, 1, 2, 3, 0, True, "bf16"),
    (1, 32, 70, 520, 5, 1, 1, 3, 2, True, "bf16"),    # two channel groups, ragged
    (2, 32, 64, 296, 5, 1, 6, 3, 0, False, "bf16"),   # "same": output length = input length
    (1, 32, 16, 264, 5, 1, 3, 3, 1, True, "bf16"),    # output length % 4 != 0: ragged rows
    (2, 32, 70, 2000, 5, 1, 1, 3, 0, True, "bf16"),   # ragged rows, two channel groups
    (8, 32, 64, 40000, 5, 1, 0, 3, 1, True, "bf16"),  # ragged rows, more tiles than workgroups
    (2, 32, 64, 512, 5, 1, 8, 3, 1, True, "bf16"),    # pad a multiple of 8
    (1, 32, 64, 2000, 5, 1, 15, 3, 0, True, "bf16"),  # pad past the halo
    (1, 32, 64, 8, 5, 1, 9, 3, 2, True, "bf16"),      # pad larger than the input
    (1, 32, 64, 16, 5, 1, 7, 3, 0, True, "bf16"),
    (1, 32, 64, 1000, 5, 1, 0, 3, 2, True, "bf16"),   # output padding alone
    (3, 32, 64, 1024, 5, 1, 4, 3, 0, True, "bf16"),   # tiles straddling batch items
    (8, 32, 64, 40000, 5, 1, 5, 3, 2, True, "bf16"),  # more tiles than workgroups
]


@pytest.mark.parametrize("case", CONV1D_GENERAL, ids=lambda c: "x".join(map(str, c)))
def test_conv1d_general(dev, case):
    N, Cin, Cout, L, K, s, p, d, op, with_bias, dt = case
    log(f"convT1d general {case}")
    seed = 8000 + N + Cin + Cout + L + K
    x = synth.normal(seed, 0, (N, Cin, L))
    bnd = 1.0 / np.sqrt(Cin * K)
    w = synth.uniform(seed, 1, (Cin, Cout, K), -bnd, bnd)
    if dt == "bf16":
        x, w = bf16_round(x), bf16_round(w)
    b = synth.normal(seed, 2, (Cout,)) if with_bias else None
    ref = oracle.convT1d(x, w, b, s, p, d, op)
    out = torch.full(ref.shape, float("nan"), dtype=torch.float32, device=dev)
    ct.ct_convT1d(to_dev(x, dev, dt), to_dev(w, dev, dt), opt(b, dev), s, p, d, op, out=out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, F32_TOL if dt == "f32" else BF16_TOL, str(case))


def test_conv1d_bf16_misaligned_x_takes_general_path(dev):
    x = bf16_round(synth.normal(91, 0, (1, 32, 64)))
    w = bf16_round(synth.uniform(91, 1, (32, 8, 5), -0.1, 0.1))
    buf = torch.empty(x.size + 1, dtype=torch.bfloat16, device=dev)
    buf[1:] = to_dev(x.reshape(-1), dev, "bf16")
    out = torch.full((1, 8, 76), float("nan"), dtype=torch.float32, device=dev)
    ct.ct_convT1d(buf[1:].view(1, 32, 64), to_dev(w, dev, "bf16"), None, 1, 0, 3, out=out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), oracle.convT1d(x, w, None, 1, 0, 3), F32_TOL, "misaligned")


@pytest.mark.parametrize("dt,pad,op", [("f32", 0, 0), ("f32", 1, 0), ("bf16", 0, 0), ("bf16", 2, 1)])
def test_conv1d_out_misaligned(dev, dt, pad, op):
    """An output that starts 4 bytes past a 16-byte boundary: the matrix-core
    kernels store its rows with 4-byte aligned vectors (and the row ends'
    partial vectors element by element); every element matches the oracle and
    the floats around the output stay untouched."""
    N, Cin, Cout, L = 2, 32, 40, 1032
    log(f"conv1d misaligned out {dt} pad {pad} op {op}")
    x = synth.normal(92, 0, (N, Cin, L))
    w = synth.uniform(92, 1, (Cin, Cout, 5), -0.08, 0.08)
    if dt == "bf16":
        x, w = bf16_round(x), bf16_round(w)
    b = synth.normal(92, 2, (Cout,))
    ref = oracle.convT1d(x, w, b, 1, pad, 3, op)
    n = ref.size
    buf = torch.full((n + 8,), float("nan"), dtype=torch.float32, device=dev)
    buf[0], buf[n + 1] = -7.0, -9.0
    out = buf[1:n + 1].view(ref.shape)
    ct.ct_convT1d(to_dev(x, dev, dt), to_dev(w, dev, dt), opt(b, dev), 1, pad, 3, op, out=out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, F32_TOL if dt == "f32" else BF16_TOL, "misaligned out")
    assert float(buf[0]) == -7.0 and float(buf[n + 1]) == -9.0
