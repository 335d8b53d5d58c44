"""Seeded random-shape parity of every entry point with the fp64 oracle.

The other parity tests use hand-picked shapes.  Here each case draws its
sizes and geometry from a fixed seed (numpy's PCG64, so the set is the same
on every run) over the space of valid calls, and its data from the seeded
Philox generators the other tests use.  The draws reach every dispatch
branch: the page geometries' fast kernels (fp32 slab and direct fused
kernels, the bf16 fused kernel with and without the straight-to-register
weights, the vector and element pool kernels, the stride-1 and stride-2
matrix-core 1D convs, the bf16 1D conv) and the general kernels.

Tolerances as elsewhere: fp32 inputs atol 1e-4, rtol 1e-5; bf16 inputs
atol 1e-4, rtol 2e-2 (the oracle takes the same bf16-rounded values); bf16
pool outputs 1e-5 + 2^-8 relative.  Outputs are NaN-prefilled, so an element
no kernel writes fails.
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
POOL_BF16_TOL = (1e-5, 2.0 ** -8)
CASES = 24


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def rng(tag, i):
    return np.random.default_rng([0xF022, tag, i])


def data(seed, x_shape, w_shape, Cout, bf16, with_cb):
    x = synth.normal(seed, 0, x_shape)
    fan = int(np.prod(w_shape)) // Cout
    w = synth.uniform(seed, 1, w_shape, -1.0 / np.sqrt(fan), 1.0 / np.sqrt(fan))
    if bf16:
        x, w = bf16_round(x), bf16_round(w)
    b = synth.normal(seed, 2, (Cout,))
    cb = synth.normal(seed, 3, (Cout,)) if with_cb else None
    return x, w, b, cb


# ------------------------------------------------------------ fused chain --
def draw_fused(i):
    """Half the cases at the page's geometry (k3 s2 p1, 2-pool), the rest general."""
    r = rng(1, i)
    bf16 = bool(r.integers(0, 3) == 0)
    while True:
        if i % 2 == 0:
            k, s, p, op, pk, ps = 3, 2, 1, int(r.integers(0, 2)) if not bf16 else 0, 2, 2
        else:
            k = int(r.integers(1, 5))
            s = int(r.integers(1, 4))
            p = int(r.integers(0, k))
            op = int(r.integers(0, s))
            pk = int(r.integers(1, 4))
            ps = int(r.integers(0, 4))
        Cin = int(r.choice([1, 2, 3, 4, int(r.integers(5, 40))]))
        Cout = int(r.choice([16, 64, int(r.integers(1, 80))]))
        N = int(r.integers(1, 4))
        D, H = int(r.integers(2, 7)), int(r.integers(2, 26))
        W = int(r.choice([8 * int(r.integers(1, 7)), int(r.integers(2, 50))]))
        dims = ct._fused_dims(D, H, W, k, s, p, op, pk, ps)
        work = N * Cin * D * H * W * Cout * k ** 3
        if min(dims) > 0 and work < 3e8:
            return N, Cin, Cout, D, H, W, k, s, p, op, pk, ps, bf16


@pytest.mark.parametrize("i", range(2 * CASES))
def test_fuzz_fused(dev, i):
    N, Cin, Cout, D, H, W, k, s, p, op, pk, ps, bf16 = c = draw_fused(i)
    log(f"fuzz fused {c}")
    with_cb = bool(i % 3 == 1)
    x, w, b, cb = data(7000 + i, (N, Cin, D, H, W), (Cin, Cout, k, k, k), Cout, bf16, with_cb)
    dt = "bf16" if bf16 else "f32"
    dims = ct._fused_dims(D, H, W, k, s, p, op, pk, ps)
    out = nan_like((N, Cout) + dims, dev)
    ct.ct_convT3d_scale_pool_bias(to_dev(x, dev, dt), to_dev(w, dev, dt), opt(cb, dev),
                                  opt(b, dev), 0.5, 1.0, stride=s, pad=p, out_pad=op,
                                  pool_k=pk, pool_s=ps, out=out)
    torch.cuda.synchronize()
    ref = oracle.convT3d_scale_pool_bias(x, w, cb, b, 0.5, 1.0, s, p, op, pk, ps or pk)
    assert_close(out.cpu().numpy(), ref, BF16_TOL if bf16 else F32_TOL, f"fuzz fused {c}")


# ------------------------------------------------- ConvTranspose3d alone --
def draw_convT3d(i):
    r = rng(2, i)
    while True:
        if i % 2 == 0:
            k, s, p, op = 3, 2, 1, int(r.integers(0, 2))
        else:
            k, s = int(r.integers(1, 5)), int(r.integers(1, 4))
            p, op = int(r.integers(0, k)), int(r.integers(0, s))
        Cin, Cout = int(r.integers(1, 10)), int(r.integers(1, 20))
        N, D, H, W = (int(r.integers(1, 3)), int(r.integers(1, 6)), int(r.integers(1, 12)),
                      int(r.integers(1, 20)))
        dims = [ct.ct_convT_out_len(n, k, s, p, op, 1) for n in (D, H, W)]
        if min(dims) > 0:
            return N, Cin, Cout, D, H, W, k, s, p, op, bool(r.integers(0, 3) == 0)


@pytest.mark.parametrize("i", range(CASES))
def test_fuzz_convT3d(dev, i):
    N, Cin, Cout, D, H, W, k, s, p, op, bf16 = c = draw_convT3d(i)
    log(f"fuzz convT3d {c}")
    x, w, b, _ = data(7100 + i, (N, Cin, D, H, W), (Cin, Cout, k, k, k), Cout, bf16, False)
    bias = b if i % 2 else None
    dt = "bf16" if bf16 else "f32"
    dims = tuple(ct.ct_convT_out_len(n, k, s, p, op, 1) for n in (D, H, W))
    out = nan_like((N, Cout) + dims, dev)
    ct.ct_convT3d(to_dev(x, dev, dt), to_dev(w, dev, dt), opt(bias, dev), stride=s, pad=p,
                  out_pad=op, out=out)
    torch.cuda.synchronize()
    ref = oracle.convT3d(x, w, bias, s, p, op)
    assert_close(out.cpu().numpy(), ref, BF16_TOL if bf16 else F32_TOL, f"fuzz convT3d {c}")


# ---------------------------------------------------------------- pooling --
def draw_pool(i):
    """Even cases at the page's k3 s2 p1 (vector kernel when W % 4 == 0,
    element kernel otherwise), odd cases any valid k / stride / pad."""
    r = rng(3, i)
    while True:
        if i % 2 == 0:
            k, s, p = 3, 2, 1
        else:
            k = int(r.integers(1, 6))
            s = int(r.integers(0, 4))
            p = int(r.integers(0, k // 2 + 1))
        N, C = int(r.integers(1, 4)), int(r.integers(1, 5))
        D, H = int(r.integers(1, 12)), int(r.integers(1, 150))
        W = int(r.choice([4 * int(r.integers(1, 80)), int(r.integers(1, 300))]))
        dims = [ct.ct_pool_out_len(n, k, s, p) for n in (D, H, W)]
        if min(dims) > 0:
            return N, C, D, H, W, k, s, p, bool(r.integers(0, 2)), bool(r.integers(0, 3) == 0)


@pytest.mark.parametrize("i", range(2 * CASES))
def test_fuzz_pool(dev, i):
    N, C, D, H, W, k, s, p, incl, bf16 = c = draw_pool(i)
    log(f"fuzz pool {c}")
    x = synth.normal(7200 + i, 0, (N, C, D, H, W))
    if bf16:
        x = bf16_round(x)
    dims = tuple(ct.ct_pool_out_len(n, k, s, p) for n in (D, H, W))
    out = nan_like((N, C) + dims, dev, torch.bfloat16 if bf16 else torch.float32)
    ct.ct_avgpool3d(to_dev(x, dev, "bf16" if bf16 else "f32"), k, s, p, incl, out=out)
    torch.cuda.synchronize()
    got = bf16_tensor_to_f32(out) if bf16 else out.cpu().numpy()
    ref = oracle.avgpool3d(x, k, s or k, p, incl)
    assert_close(got, ref, POOL_BF16_TOL if bf16 else F32_TOL, f"fuzz pool {c}")


# -------------------------------------------------------- ConvTranspose1d --
def draw_convT1d(i):
    """A third of the cases at the page's channels and taps (Cin 32, K 5,
    dilation 3) with stride 1 or 2 and any pad and output padding, the rest
    any valid geometry."""
    r = rng(4, i)
    while True:
        bf16 = bool(r.integers(0, 3) == 0)
        if i % 3 == 0:
            Cin, K, d = 32, 5, 3
            s = 1 if bf16 else int(r.integers(1, 3))
            p = int(r.integers(0, 10))
            op = int(r.integers(0, 3))
            L = int(r.choice([8 * int(r.integers(1, 300)), int(r.integers(1, 2000))]))
        else:
            Cin, K, d = int(r.integers(1, 40)), int(r.integers(1, 7)), int(r.integers(1, 5))
            s = int(r.integers(1, 4))
            p = int(r.integers(0, 6))
            op = int(r.integers(0, max(s, d)))
            L = int(r.integers(1, 600))
        Cout = int(r.choice([64, int(r.integers(1, 130))]))
        N = int(r.integers(1, 4))
        Lo = ct.ct_convT_out_len(L, K, s, p, op, d)
        if Lo > 0:
            return N, Cin, Cout, L, K, s, p, d, op, bf16, bool(r.integers(0, 2))


@pytest.mark.parametrize("i", range(2 * CASES))
def test_fuzz_convT1d(dev, i):
    N, Cin, Cout, L, K, s, p, d, op, bf16, with_bias = c = draw_convT1d(i)
    log(f"fuzz convT1d {c}")
    x, w, b, _ = data(7300 + i, (N, Cin, L), (Cin, Cout, K), Cout, bf16, False)
    bias = b if with_bias else None
    dt = "bf16" if bf16 else "f32"
    Lo = ct.ct_convT_out_len(L, K, s, p, op, d)
    out = nan_like((N, Cout, Lo), dev)
    ct.ct_convT1d(to_dev(x, dev, dt), to_dev(w, dev, dt), opt(bias, dev), stride=s, pad=p,
                  dilation=d, out_pad=op, out=out)
    torch.cuda.synchronize()
    ref = oracle.convT1d(x, w, bias, s, p, d, op)
    assert_close(out.cpu().numpy(), ref, BF16_TOL if bf16 else F32_TOL, f"fuzz convT1d {c}")
