"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Tolerances (elementwise, |gpu - oracle| <= atol + rtol * |oracle|):
  fp32 inputs:  atol 1e-4, rtol 1e-5
  bf16 inputs:  atol 1e-4, rtol 2e-2 (the oracle consumes the same
                bf16-rounded values, widened exactly)
Outputs are pre-filled with NaN so an element the kernel never writes fails.
Small cases span several tiles plus ragged tails.  The fused fp32 workload
is checked here at full size on every element; the other full-size workloads
are in test_parity_full_gpu.py.
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
    ok = err <= atol + rtol * np.abs(ref)          # NaN -> not ok
    if not ok.all():
        idx = np.argwhere(~ok)
        i0 = tuple(idx[0])
        raise AssertionError(
            f"{what}: {len(idx)} of {ok.size} elements out of tolerance; first at {i0}: "
            f"gpu={got[i0]!r} oracle={ref[i0]!r}; max err {np.nanmax(err):.3g}")


def nan_like(shape, dev):
    return torch.full(shape, float("nan"), dtype=torch.float32, device=dev)


def log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------ fused fp32 ----
def run_fused(dev, x, w, cb, b, s1, s2, dtype="f32"):
    N, Cin, D, H, W = x.shape
    Cout = w.shape[1]
    if dtype == "bf16":
        xg = torch.from_numpy(synth.to_bf16_bits(x).view(np.int16)).to(dev).view(torch.bfloat16)
        wg = torch.from_numpy(synth.to_bf16_bits(w).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        xg, wg = torch.from_numpy(x).to(dev), torch.from_numpy(w).to(dev)
    cbg = None if cb is None else torch.from_numpy(cb).to(dev)
    bg = None if b is None else torch.from_numpy(b).to(dev)
    out = nan_like((N, Cout, D - 1, H - 1, W - 1), dev)
    ct.ct_convT3d_scale_pool_bias(xg, wg, cbg, bg, s1, s2, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


FUSED_SMALL = [
    # N, Cin, Cout, D, H, W
    (1, 1, 1, 2, 2, 2),
    (2, 3, 16, 8, 16, 16),
    (2, 3, 16, 5, 7, 40),
    (1, 4, 20, 3, 9, 17),
    (3, 2, 33, 4, 4, 4),
    (1, 5, 7, 6, 5, 18),
    (1, 32, 64, 3, 5, 33),
    (1, 7, 3, 2, 3, 49),
    # several tasks per workgroup: staged rows carried across row chunks,
    # planes and batch items, ragged last chunks, W % 4 != 0, ragged Cout
    (5, 3, 16, 7, 20, 24),
    (3, 4, 40, 5, 19, 13),
    (9, 1, 16, 4, 33, 32),
    (2, 2, 17, 3, 70, 9),
    # Cin 3, W 32: the instantiation with the page's geometry compiled in (8
    # pooled rows per task): one exact chunk, a ragged last chunk, ragged Cout
    # (two channel blocks), and streams carried across batch items
    (2, 3, 16, 5, 9, 32),
    (3, 3, 16, 4, 20, 32),
    (1, 3, 20, 3, 33, 32),
    (16, 3, 16, 4, 17, 32),
]


@pytest.mark.parametrize("shape", FUSED_SMALL, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_cb", [False, True], ids=["nocb", "cb"])
def test_fused_f32_small(dev, shape, with_cb):
    N, Cin, Cout, D, H, W = shape
    log(f"fused f32 {shape} cb={with_cb}")
    seed = 1000 + sum(shape)
    x = synth.normal(seed, 0, (N, Cin, D, H, W))
    bound = 1.0 / np.sqrt(Cin * 27)
    w = synth.uniform(seed, 1, (Cin, Cout, 3, 3, 3), -bound, bound)
    b = synth.normal(seed, 2, (Cout,))
    cb = synth.normal(seed, 3, (Cout,)) if with_cb else None
    got = run_fused(dev, x, w, cb, b, 0.5, 1.0)
    ref = oracle.convT3d_scale_pool_bias(x, w, cb, b, 0.5, 1.0)
    assert_close(got, ref, F32_TOL, f"fused {shape}")


# fp32 calls below 48 blocks of 16 outputs x 16 channels per CU (12,288
# blocks on the 256 CUs of an MI355X) run on the direct kernel, so most shapes
# above exercise that one.  The slab pipeline gets the same shapes (Cin <= 4)
# with the batch scaled past that size: staged rows carried across row chunks,
# planes and batch items, ragged last chunks, scalar rows (W % 4 != 0) and
# ragged channel blocks.
SLAB_BLOCKS = 48 * 256


def slab_shape(shape):
    N, Cin, Cout, D, H, W = shape
    per_item = (D - 1) * (H - 1) * ((W - 1 + 15) // 16) * ((Cout + 15) // 16)
    return (max(N, -(-SLAB_BLOCKS // per_item)),) + tuple(shape[1:])


FUSED_SLAB = [slab_shape(s) for s in FUSED_SMALL if s[1] <= 4]


@pytest.mark.parametrize("shape", FUSED_SLAB, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_cb", [False, True], ids=["nocb", "cb"])
def test_fused_f32_slab(dev, shape, with_cb):
    test_fused_f32_small(dev, shape, with_cb)


def test_fused_f32_other_scales_no_bias(dev):
    x = synth.uniform(77, 0, (2, 3, 6, 9, 21), 0.0, 1.0)      # the page's torch.rand inputs
    w = synth.uniform(77, 1, (3, 5, 3, 3, 3), -0.2, 0.2)
    got = run_fused(dev, x, w, None, None, -1.7, 0.3)
    ref = oracle.convT3d_scale_pool_bias(x, w, None, None, -1.7, 0.3)
    assert_close(got, ref, F32_TOL, "fused scales")


def test_fused_f32_c1_workload(dev):
    wl = synth.WORKLOADS["c1"]
    t = synth.make_inputs(wl, conv_bias=True)
    log(wl.description)
    for cb in (None, t["conv_bias"]):
        got = run_fused(dev, t["x"], t["w"], cb, t["bias"], 0.5, 1.0)
        ref = oracle.convT3d_scale_pool_bias(t["x"], t["w"], cb, t["bias"], 0.5, 1.0)
        assert got.shape == (2, 16, 7, 15, 15)
        assert_close(got, ref, F32_TOL, "c1")


def test_fused_f32_c2_full(dev):
    """Full-size [128,3,16,32,32] -> [128,16,15,31,31], every element."""
    wl = synth.WORKLOADS["c2"]
    log(wl.description)
    t = synth.make_inputs(wl)
    got = run_fused(dev, t["x"], t["w"], None, t["bias"], 0.5, 1.0)
    ref = oracle.convT3d_scale_pool_bias(t["x"], t["w"], None, t["bias"], 0.5, 1.0)
    assert got.shape == (128, 16, 15, 31, 31)
    assert_close(got, ref, F32_TOL, "c2")


def test_fused_f32_nan_propagates_locally(dev):
    """A NaN input reaches exactly the pooled voxels whose 2x2x2 taps contain it."""
    x = synth.normal(5, 0, (1, 2, 5, 6, 7))
    x[0, 1, 2, 3, 4] = np.nan
    w = synth.uniform(5, 1, (2, 3, 3, 3, 3), -0.2, 0.2)
    got = run_fused(dev, x, w, None, None, 0.5, 1.0)
    nan = np.isnan(got)
    exp = np.zeros_like(nan)
    exp[0, :, 1:3, 2:4, 3:5] = True
    assert np.array_equal(nan, exp)


# ------------------------------------------------------------ fused bf16 ----
FUSED_BF16 = [
    # N, Cin, Cout, D, H, W   (W a multiple of 8, Cin <= 32)
    (1, 8, 16, 2, 2, 8),
    (2, 32, 64, 3, 5, 32),
    (1, 5, 20, 4, 6, 16),      # Cin8 = 8
    (1, 17, 70, 3, 4, 24),     # Cin8 = 24, two channel groups, ragged Cout
    (2, 12, 64, 5, 3, 40),     # Cin8 = 16, three voxel blocks per row
    (1, 32, 8, 2, 9, 64),
    # several tiles per workgroup: staged rows carried across row chunks,
    # planes and batch items, ragged last chunks, a ragged second channel group
    (10, 8, 64, 9, 23, 24),
    (20, 8, 96, 4, 10, 40),
    (12, 32, 64, 6, 18, 16),
    # one 64-channel group, weights read straight into registers: input
    # channels padded to 32, 8 (one couple per thread) and 24 (some threads
    # with a second couple)
    (3, 25, 64, 3, 4, 32),
    (2, 3, 64, 2, 3, 8),
    (2, 20, 64, 3, 6, 16),
    # direct weights, but the slab is larger than the raw-weight region, so
    # the first slab is staged after the fragments are loaded
    (1, 32, 64, 2, 3, 128),
    # 25..32 input channels, Cout a multiple of 64: weights read as whole
    # lines in two 16-channel halves; two and three 64-channel groups, input
    # channels padded from 27 and 29
    (2, 32, 128, 3, 5, 32),
    (2, 27, 192, 2, 4, 24),
    (3, 29, 64, 4, 11, 32),
]


def bf16_round(a):
    return synth.bf16_bits_to_f32(synth.to_bf16_bits(a)).reshape(a.shape)


@pytest.mark.parametrize("shape", FUSED_BF16, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_cb", [False, True], ids=["nocb", "cb"])
def test_fused_bf16_small(dev, shape, with_cb):
    N, Cin, Cout, D, H, W = shape
    log(f"fused bf16 {shape} cb={with_cb}")
    seed = 4000 + sum(shape)
    x = bf16_round(synth.normal(seed, 0, (N, Cin, D, H, W)))
    bound = 1.0 / np.sqrt(Cin * 27)
    w = bf16_round(synth.uniform(seed, 1, (Cin, Cout, 3, 3, 3), -bound, bound))
    b = synth.normal(seed, 2, (Cout,))
    cb = synth.normal(seed, 3, (Cout,)) if with_cb else None
    got = run_fused(dev, x, w, cb, b, 0.5, 1.0, dtype="bf16")
    ref = oracle.convT3d_scale_pool_bias(x, w, cb, b, 0.5, 1.0)
    assert_close(got, ref, BF16_TOL, f"fused bf16 {shape}")
    # the hi/lo filter split keeps the result far inside the bf16 tolerance
    assert_close(got, ref, (1e-4, 1e-4), f"fused bf16 {shape} (tight)")


# ------------------------------------------------------------ avgpool3d ----
POOL_SMALL = [
    # planes of at most 4096 elements: the small-plane kernel (several
    # slices per workgroup, 4-element loads when W % 4 == 0, else 1)
    (1, 1, 1, 1, 1),
    (1, 1, 2, 2, 2),
    (2, 3, 9, 10, 13),
    (1, 2, 5, 6, 256),
    (1, 1, 3, 4, 260),
    (1, 1, 4, 5, 514),        # element loads, the widest row that fits
    (1, 2, 33, 35, 64),       # several plane chunks
    (2, 1, 7, 3, 1),
    (1, 1, 3, 131, 8),
    (4, 25, 40, 6, 8),        # 100 slices: several plane chunks of more than one plane
    (3, 1, 1, 4, 4),          # a single input plane
    (8, 40, 40, 10, 16),      # 320 slices, 10 per workgroup
    (64, 16, 8, 16, 16),      # 1024 slices of 16 x 16 planes
    (3, 5, 9, 64, 64),        # one slice per workgroup (4096-element planes)
    # larger planes: the vector kernel (W % 4 == 0) or the element kernel
    (1, 1, 3, 20, 260),       # two column chunks, vector path
    (1, 1, 4, 9, 514),        # two column chunks, element path
    (1, 2, 33, 135, 64),      # several plane chunks and row groups
    (1, 1, 3, 131, 40),       # two row groups: the row above a group comes from memory
    (1, 1, 2, 140, 264),      # two row groups and two column chunks
    (1, 1, 5, 258, 520),      # three row groups, three column chunks, ragged last of each
    (8, 40, 20, 34, 128),     # 320 slices in ranges of 10 planes: every start offset of a bf16 range
    # fewer than 128 rows, several column chunks: the vector kernel's waves
    # split into 2, 4 or 8 column groups (some past W)
    (2, 3, 5, 60, 600),       # 2 groups, 3 chunks: one group of the second workgroup idle
    (1, 2, 3, 30, 1024),      # 4 groups
    (1, 1, 3, 12, 2100),      # 8 groups, 9 chunks
]


@pytest.mark.parametrize("shape", POOL_SMALL, ids=lambda s: "x".join(map(str, s)))
def test_pool_small(dev, shape):
    log(f"pool {shape}")
    x = synth.normal(2000 + sum(shape), 0, shape)
    xg = torch.from_numpy(x).to(dev)
    dims = [(n - 1) // 2 + 1 for n in shape[2:]]
    out = nan_like(shape[:2] + tuple(dims), dev)
    ct.ct_avgpool3d(xg, 3, 2, 1, True, out=out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), oracle.avgpool3d(x, 3, 2, 1, True), F32_TOL, f"pool {shape}")


@pytest.mark.parametrize("shape", [(2, 2, 6, 7, 64), (2, 2, 6, 70, 64)],
                         ids=["small-plane element loads", "element kernel"])
def test_pool_misaligned_input_takes_element_loads(dev, shape):
    x = synth.normal(31, 0, shape)
    buf = torch.empty(x.size + 1, dtype=torch.float32, device=dev)
    buf[1:] = torch.from_numpy(x.reshape(-1)).to(dev)
    xg = buf[1:].view(shape)                        # 4-byte but not 16-byte aligned
    out = nan_like(shape[:2] + tuple((n - 1) // 2 + 1 for n in shape[2:]), dev)
    ct.ct_avgpool3d(xg, 3, 2, 1, True, out=out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), oracle.avgpool3d(x, 3, 2, 1, True), F32_TOL, "misaligned")


def test_pool_constant_input_border_values(dev):
    """All-ones input: 8/27 at corners, 12/27 on edges, 18/27 on faces, 1 inside."""
    x = torch.ones((1, 2, 16, 16, 32), dtype=torch.float32, device=dev)
    out = ct.ct_avgpool3d(x, 3, 2, 1, True)
    torch.cuda.synchronize()
    o = out.cpu().numpy()[0, 0]
    assert abs(o[0, 0, 0] - 8 / 27) < 1e-6 and abs(o[0, 0, 5] - 12 / 27) < 1e-6
    assert abs(o[0, 3, 5] - 18 / 27) < 1e-6 and abs(o[3, 3, 5] - 1.0) < 1e-6
    assert abs(o[-1, -1, -1] - 1.0) < 1e-6


# bf16 pooling: fp32 sums of exactly widened taps, each mean rounded to the
# nearest bf16.  The rounding is at most half a bf16 step (2^-9 relative) and
# the fp32 sum/divide adds ~1e-6 absolute at these magnitudes, so one step
# (2^-8 relative) plus 1e-5 absolute bounds the difference from the fp64
# oracle on the same bf16 values (well inside the rel 2e-2 bf16 bound).
POOL_BF16_TOL = (1e-5, 2.0 ** -8)


def pool_bf16(dev, x, shift=0):
    """Pool the bf16 values x (fp32 array) on the GPU; returns fp32.  shift > 0
    places x that many elements into its buffer (misaligned starts)."""
    bits = torch.from_numpy(synth.to_bf16_bits(x).reshape(-1).view(np.int16))
    buf = torch.zeros(bits.numel() + shift, dtype=torch.int16, device=dev)
    buf[shift:] = bits.to(dev)
    xg = buf[shift:].view(torch.bfloat16).view(x.shape)
    dims = [(n - 1) // 2 + 1 for n in x.shape[2:]]
    out = torch.full(x.shape[:2] + tuple(dims), float("nan"), dtype=torch.bfloat16, device=dev)
    ct.ct_avgpool3d(xg, 3, 2, 1, True, out=out)
    torch.cuda.synchronize()
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return synth.bf16_bits_to_f32(o).reshape(o.shape)


@pytest.mark.parametrize("shape", POOL_SMALL, ids=lambda s: "x".join(map(str, s)))
def test_pool_bf16_small(dev, shape):
    log(f"pool bf16 {shape}")
    x = bf16_round(synth.normal(2500 + sum(shape), 0, shape))
    assert_close(pool_bf16(dev, x), oracle.avgpool3d(x, 3, 2, 1, True), POOL_BF16_TOL,
                 f"pool bf16 {shape}")


@pytest.mark.parametrize("shape", [(2, 2, 6, 7, 64), (2, 2, 6, 70, 64)],
                         ids=["small-plane element loads", "element kernel"])
@pytest.mark.parametrize("shift", [1, 2], ids=["2-byte", "4-byte"])
def test_pool_bf16_misaligned_input_takes_element_loads(dev, shift, shape):
    x = bf16_round(synth.normal(33, 0, shape))
    assert_close(pool_bf16(dev, x, shift), oracle.avgpool3d(x, 3, 2, 1, True), POOL_BF16_TOL,
                 f"pool bf16 shifted by {shift}")


def test_pool_plane_of_2_30_bytes_takes_element_path(dev):
    """A [16384, 16384] plane (2^30 bytes) is past the vector kernel's plane
    limit and runs on the element kernel; every output against the oracle."""
    H = W = 16384
    log(f"pool (1, 1, 1, {H}, {W}) element path")
    x = synth.normal(2077, 0, (1, 1, 1, H, W))
    xg = torch.from_numpy(x).to(dev)
    out = nan_like((1, 1, 1, H // 2, W // 2), dev)
    ct.ct_avgpool3d(xg, 3, 2, 1, True, out=out)
    torch.cuda.synchronize()
    del xg
    assert_close(out.cpu().numpy(), oracle.avgpool3d(x, 3, 2, 1, True), F32_TOL,
                 "pool 2^30-byte plane")


def test_pool_grid_beyond_one_dispatch_takes_general_path(dev):
    """4.2 M slices of [1, 1, 4]: the streaming kernel would need more than
    2^32 work-items (one 1024-thread workgroup per slice), so the call runs on
    the grid-striding general kernel."""
    shape = (4200000, 1, 1, 1, 4)
    log(f"pool {shape}")
    x = synth.normal(2099, 0, shape)
    out = nan_like((4200000, 1, 1, 1, 2), dev)
    ct.ct_avgpool3d(torch.from_numpy(x).to(dev), 3, 2, 1, True, out=out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), oracle.avgpool3d(x, 3, 2, 1, True), F32_TOL, "pool 4.2M slices")


# -------------------------------------------------------------- convT1d ----
CONV1D_SMALL = [
    # N, Cin, Cout, L, K, dilation, bias
    (1, 1, 1, 10, 1, 1, False),
    (2, 32, 64, 700, 5, 3, False),
    (1, 3, 5, 50, 4, 2, True),
    (2, 8, 70, 300, 3, 7, True),
    (1, 4, 16, 5, 5, 3, False),          # L shorter than the halo
    (1, 36, 64, 513, 5, 3, False),
    (3, 32, 64, 256, 5, 3, True),
    (1, 32, 70, 520, 5, 3, True),        # two output-channel groups, ragged
    (2, 32, 16, 8, 5, 3, False),         # one tile per item, most waves idle
    (1, 32, 64, 4, 5, 3, True),          # shortest fast-path input
    (5, 32, 64, 1028, 5, 3, False),      # tiles straddling batch items
    (8, 32, 64, 20004, 5, 3, True),      # more tiles than waves: halos carried between tiles
]


@pytest.mark.parametrize("case", CONV1D_SMALL, ids=lambda s: "x".join(map(str, s)))
def test_conv1d_small(dev, case):
    N, Cin, Cout, L, K, d, with_bias = case
    log(f"convT1d {case}")
    seed = 3000 + N + Cin + Cout + L
    x = synth.normal(seed, 0, (N, Cin, L))
    bnd = 1.0 / np.sqrt(Cin * K)
    w = synth.uniform(seed, 1, (Cin, Cout, K), -bnd, bnd)
    b = synth.normal(seed, 2, (Cout,)) if with_bias else None
    Lo = L + d * (K - 1)
    out = nan_like((N, Cout, Lo), dev)
    ct.ct_convT1d(torch.from_numpy(x).to(dev), torch.from_numpy(w).to(dev),
                  None if b is None else torch.from_numpy(b).to(dev), 1, 0, d, out=out)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), oracle.convT1d(x, w, b, 1, 0, d), F32_TOL, f"convT1d {case}")
