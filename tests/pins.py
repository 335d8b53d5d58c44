"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Every ``pin_*`` function takes an optional ``lib`` (an oracle library loaded
with ``oracle.load_library``; None = the normal build) and raises
AssertionError when the oracle disagrees with the pin.  ``test_oracle_pins.py``
runs them on the real oracle (all must pass) and ``test_oracle_mutants.py`` on
builds with planted mistakes (each mutant must fail at least one).

Sources (POPCORNBENCH pages, one problem each): [p50] "Kimi-K2.6 l2_p50"
(fused ConvTranspose3d chain), [p46] "Kimi-K2.6 l1_p46" (AvgPool3d),
[p74] "Kimi-K2.6 l1_p74" (dilated ConvTranspose1d).
"""
from __future__ import annotations

import os
import re

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln


# ---------------------------------------------------------------- shapes ----
def pin_output_sizes(lib=None):
    """Output-size formulas against the sizes the pages derive."""
    for ln in _lines("output_sizes.txt"):
        kind, *v = ln.split()
        v = [int(t) for t in v]
        if kind == "convT":
            n, k, s, p, op, d, exp = v
            got = oracle.convT_out_len(n, k, s, p, op, d, lib=lib)
        elif kind == "pool":
            n, k, s, p, exp = v
            got = oracle.pool_out_len(n, k, s, p, lib=lib)
        elif kind == "chain":
            n, exp = v
            got = oracle.pool_out_len(oracle.convT_out_len(n, 3, 2, 1, 0, 1, lib=lib),
                                      2, 2, 0, lib=lib)
        else:
            raise ValueError(kind)
        assert got == exp, f"{ln}: got {got}"


def pin_chain_shape_from_oracle(lib=None):
    """The fused oracle's output shape is (D-1, H-1, W-1) ([p50], any-size passage)."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((1, 2, 3, 5, 4)).astype(np.float32)
    w = rng.standard_normal((2, 3, 3, 3, 3)).astype(np.float32)
    y = oracle.convT3d_scale_pool_bias(x, w, None, None, 1.0, 1.0, lib=lib)
    assert y.shape == (1, 3, 2, 4, 3), y.shape


# ------------------------------------------------------- worked examples ----
def _eval_terms(expr, wv, xv):
    expr = expr.strip()
    if expr == "0":
        return 0.0
    tot = 0.0
    for term in expr.split("+"):
        m = re.fullmatch(r"w(\d+)\*x(\d+)", term.strip())
        assert m, term
        tot += wv[int(m.group(1))] * xv[int(m.group(2))]
    return tot


def pin_convT1d_worked_examples(lib=None):
    """[p74]'s worked transpose / dilation examples, term by term (exact integers)."""
    lines = list(_lines("p74_convT1d_worked.txt"))
    assert len(lines) % 2 == 0
    rng = np.random.default_rng(5)
    for i in range(0, len(lines), 2):
        m = re.fullmatch(r"case K=(\d+) dilation=(\d+) L=(\d+)", lines[i])
        assert m, lines[i]
        K, d, L = (int(g) for g in m.groups())
        exprs = lines[i + 1].split(None, 1)[1].split("|")
        wv = rng.integers(-9, 10, K).astype(np.float32)
        wv[wv == 0] = 3
        xv = rng.integers(-9, 10, L).astype(np.float32)
        xv[xv == 0] = 5
        got = oracle.convT1d(xv.reshape(1, 1, L), wv.reshape(1, 1, K), None,
                             1, 0, d, 0, lib=lib).reshape(-1)
        exp = np.array([_eval_terms(e, wv, xv) for e in exprs])
        assert got.shape == exp.shape, (lines[i], got.shape, exp.shape)
        assert np.array_equal(got, exp), (lines[i], got, exp)


def pin_parity_rule_depth2(lib=None):
    """[p50]'s stride-2 parity rule on a depth-2 input, in the 3D and 1D oracles."""
    lines = list(_lines("p50_parity_depth2.txt"))
    n_in = int(lines[0].split()[1])
    n_out = int(lines[1].split()[1])
    rules = {}
    for ln in lines[2:]:
        o, rest = ln.split(":")
        rules[int(o)] = [tuple(int(t) for t in pr.split(",")) for pr in rest.split()]
    xv = np.array([3.0, -7.0], dtype=np.float32)[:n_in]
    wk = np.array([2.0, 5.0, -11.0], dtype=np.float32)
    exp = np.array([sum(xv[i] * wk[k] for i, k in rules[o]) for o in range(n_out)])
    # 1D: ConvTranspose1d k3 s2 p1
    y1 = oracle.convT1d(xv.reshape(1, 1, n_in), wk.reshape(1, 1, 3), None, 2, 1, 1, 0,
                        lib=lib).reshape(-1)
    assert np.array_equal(y1, exp), (y1, exp)
    # 3D with H = W = 1: only the centre tap reaches the single output row/col.
    w3 = np.zeros((1, 1, 3, 3, 3), dtype=np.float32)
    w3[0, 0, :, 1, 1] = wk
    w3[0, 0, :, 0, :] = 1000.0   # taps that must never land in bounds
    w3[0, 0, :, 2, :] = 1000.0
    w3[0, 0, :, :, 0] = 1000.0
    w3[0, 0, :, :, 2] = 1000.0
    y3 = oracle.convT3d(xv.reshape(1, 1, n_in, 1, 1), w3, None, 2, 1, 0, lib=lib)
    assert y3.shape == (1, 1, n_out, 1, 1), y3.shape
    assert np.array_equal(y3.reshape(-1), exp), (y3.reshape(-1), exp)


def pin_grouped_sums_arange27(lib=None):
    """[p50]'s tap sums with weight = arange(27), via a delta input through the fused oracle."""
    table = {}
    for ln in _lines("p50_grouped_sums_arange27.txt"):
        a, b, c, s = (int(t) for t in ln.split())
        table[(a, b, c)] = s
    assert sum(table.values()) == sum(range(27)) == 351
    D = H = W = 6
    q = (3, 2, 4)
    x = np.zeros((1, 1, D, H, W), dtype=np.float32)
    x[0, 0][q] = 1.0
    w = np.arange(27, dtype=np.float32).reshape(1, 1, 3, 3, 3)
    y = oracle.convT3d_scale_pool_bias(x, w, None, None, 1.0, 1.0, lib=lib)[0, 0]
    assert y.shape == (D - 1, H - 1, W - 1)
    exp = np.zeros_like(y)
    for (a, b, c), s in table.items():
        exp[q[0] - a, q[1] - b, q[2] - c] = s / 8.0
    assert np.array_equal(y, exp), np.argwhere(y != exp)


def pin_partition_constant_input(lib=None):
    """Constant input c: out = ((c*sum(W[:,co])/8 + cb)*s1 + b)*s2 at every voxel.

    Each of the 27 weights of every (ci, co) meets one pooled voxel exactly once
    ([p50], passage listing all 27 flat indices once), and the conv bias passes
    through the average unchanged ([p50], passage on the epilogue algebra).
    """
    rng = np.random.default_rng(7)
    for (N, Cin, Cout, D, H, W) in [(2, 3, 4, 4, 5, 6), (1, 2, 2, 2, 2, 2), (1, 1, 3, 7, 3, 2)]:
        c = 0.75
        x = np.full((N, Cin, D, H, W), c, dtype=np.float32)
        w = rng.standard_normal((Cin, Cout, 3, 3, 3)).astype(np.float32)
        cb = rng.standard_normal(Cout).astype(np.float32)
        b = rng.standard_normal(Cout).astype(np.float32)
        s1, s2 = 0.37, -1.9
        y = oracle.convT3d_scale_pool_bias(x, w, cb, b, s1, s2, lib=lib)
        assert y.shape == (N, Cout, D - 1, H - 1, W - 1)
        wsum = w.astype(np.float64).sum(axis=(0, 2, 3, 4))
        exp = ((c * wsum / 8.0 + cb.astype(np.float64)) * s1 + b.astype(np.float64)) * s2
        err = np.abs(y - exp[None, :, None, None, None]).max()
        assert err <= 1e-12 * max(1.0, np.abs(exp).max()), err


# ------------------------------------------------------------- pooling ----
def pin_pool_border_divisors(lib=None):
    """[p46]'s constant-input border values on an even shape and on its own shape."""
    num = dict(ln.split() for ln in _lines("p46_border_divisors.txt"))
    num = {k: int(v) for k, v in num.items()}
    for shape in [(1, 1, 8, 8, 16), (1, 1, 128, 128, 256)]:
        x = np.ones(shape, dtype=np.float32)
        y = oracle.avgpool3d(x, 3, 2, 1, True, lib=lib)[0, 0]
        Do, Ho, Wo = (s // 2 for s in shape[2:])
        assert y.shape == (Do, Ho, Wo), y.shape
        lowfaces = (np.arange(Do)[:, None, None] == 0).astype(int) \
            + (np.arange(Ho)[None, :, None] == 0).astype(int) \
            + (np.arange(Wo)[None, None, :] == 0).astype(int)
        cls = {3: "corner", 2: "edge", 1: "face", 0: "interior"}
        exp = np.vectorize(lambda t: num[cls[t]] / 27.0)(lowfaces)
        assert np.array_equal(y, exp), np.argwhere(y != exp)[:5]


def pin_pool_exclude_pad_constant(lib=None):
    """count_include_pad off: a constant input averages to itself everywhere."""
    x = np.full((2, 3, 5, 6, 7), 2.5, dtype=np.float32)
    for (k, s, p) in [(3, 2, 1), (2, 2, 1), (3, 1, 1), (3, 3, 0)]:
        y = oracle.avgpool3d(x, k, s, p, False, lib=lib)
        assert np.allclose(y, 2.5, rtol=0, atol=1e-15), (k, s, p)


def _pool_brute(x, k, s, p, include):
    """Independent check: explicit zero-padded array and window means."""
    D, H, W = x.shape[-3:]
    xp = np.zeros(x.shape[:-3] + (D + 2 * p, H + 2 * p, W + 2 * p))
    xp[..., p:p + D, p:p + H, p:p + W] = x
    mp = np.zeros_like(xp)
    mp[..., p:p + D, p:p + H, p:p + W] = 1.0
    Do, Ho, Wo = ((n + 2 * p - k) // s + 1 for n in (D, H, W))
    out = np.empty(x.shape[:-3] + (Do, Ho, Wo))
    for od in range(Do):
        for oh in range(Ho):
            for ow in range(Wo):
                win = xp[..., od * s:od * s + k, oh * s:oh * s + k, ow * s:ow * s + k]
                msk = mp[..., od * s:od * s + k, oh * s:oh * s + k, ow * s:ow * s + k]
                div = k ** 3 if include else msk.sum(axis=(-1, -2, -3))
                out[..., od, oh, ow] = win.sum(axis=(-1, -2, -3)) / div
    return out


def pin_pool_bruteforce_padded_array(lib=None):
    """Oracle pool vs an explicitly padded array (different formulation), tiny shapes."""
    rng = np.random.default_rng(3)
    for shape, k, s, p in [((2, 2, 5, 6, 7), 3, 2, 1), ((1, 1, 4, 4, 4), 2, 2, 1),
                           ((1, 2, 6, 5, 4), 3, 1, 1), ((1, 1, 7, 7, 7), 3, 3, 0)]:
        x = rng.standard_normal(shape).astype(np.float32)
        for include in (True, False):
            got = oracle.avgpool3d(x, k, s, p, include, lib=lib)
            exp = _pool_brute(x.astype(np.float64), k, s, p, include)
            assert got.shape == exp.shape
            assert np.abs(got - exp).max() <= 1e-13, (shape, k, s, p, include)


# -------------------------------------------- transposed conv structure ----
def _conv1d_forward(y, w, s, p, d, L_in):
    """The convolution that ConvTranspose1d transposes: gather form.

    z[n,ci,i] = sum_co sum_k w[ci,co,k] * y[n,co,i*s - p + d*k] over in-bounds
    positions.  Its adjoint is the scatter oracle ([p74], passage deriving the
    transposed operator from <Wx, y> = <x, W^T y>).
    """
    N, Cout, Lo = y.shape
    Cin, _, K = w.shape
    z = np.zeros((N, Cin, L_in))
    for i in range(L_in):
        for k in range(K):
            o = i * s - p + d * k
            if 0 <= o < Lo:
                z[:, :, i] += np.einsum("nc,ic->ni", y[:, :, o], w[:, :, k])
    return z


def _conv3d_forward(y, w, s, p, shape_in):
    """Gather-form forward 3D convolution (the operator whose transpose is convT3d)."""
    N, Cout, Do, Ho, Wo = y.shape
    Cin, _, k, _, _ = w.shape
    D, H, W = shape_in
    z = np.zeros((N, Cin, D, H, W))
    for i in range(D):
        for j in range(H):
            for l in range(W):
                for kd in range(k):
                    od = i * s - p + kd
                    if not 0 <= od < Do:
                        continue
                    for kh in range(k):
                        oh = j * s - p + kh
                        if not 0 <= oh < Ho:
                            continue
                        for kw in range(k):
                            ow = l * s - p + kw
                            if not 0 <= ow < Wo:
                                continue
                            z[:, :, i, j, l] += np.einsum(
                                "nc,ic->ni", y[:, :, od, oh, ow], w[:, :, kd, kh, kw])
    return z


def pin_adjoint_1d(lib=None):
    """<convT1d(x), y> = <x, conv1d(y)> ([p74], adjoint derivation), fp64 to 1e-12."""
    rng = np.random.default_rng(21)
    for (N, Cin, Cout, L, K, s, p, d, op) in [(2, 3, 4, 9, 5, 1, 0, 3, 0),
                                               (1, 2, 3, 7, 3, 2, 1, 1, 1),
                                               (2, 1, 2, 6, 4, 3, 2, 2, 2),
                                               (1, 4, 1, 5, 2, 1, 1, 2, 0)]:
        x = rng.standard_normal((N, Cin, L)).astype(np.float32)
        w = rng.standard_normal((Cin, Cout, K)).astype(np.float32)
        yx = oracle.convT1d(x, w, None, s, p, d, op, lib=lib)
        Lo = (L - 1) * s - 2 * p + d * (K - 1) + op + 1
        assert yx.shape == (N, Cout, Lo), (yx.shape, Lo)
        y = rng.standard_normal(yx.shape)
        lhs = float((yx * y).sum())
        rhs = float((x.astype(np.float64) * _conv1d_forward(y, w.astype(np.float64), s, p, d, L)).sum())
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)), (lhs, rhs)


def pin_adjoint_3d(lib=None):
    """<convT3d(x), y> = <x, conv3d(y)> at k3 s2 p1 and other geometries, fp64."""
    rng = np.random.default_rng(22)
    for (N, Cin, Cout, D, H, W, k, s, p, op) in [(1, 2, 3, 3, 4, 2, 3, 2, 1, 0),
                                                  (2, 1, 2, 2, 3, 3, 3, 2, 1, 1),
                                                  (1, 2, 2, 3, 2, 3, 2, 1, 0, 0),
                                                  (1, 1, 1, 2, 2, 2, 4, 3, 1, 2)]:
        x = rng.standard_normal((N, Cin, D, H, W)).astype(np.float32)
        w = rng.standard_normal((Cin, Cout, k, k, k)).astype(np.float32)
        yx = oracle.convT3d(x, w, None, s, p, op, lib=lib)
        y = rng.standard_normal(yx.shape)
        lhs = float((yx * y).sum())
        rhs = float((x.astype(np.float64) * _conv3d_forward(y, w.astype(np.float64), s, p, (D, H, W))).sum())
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)), (lhs, rhs)


def pin_dense_matrix_1d(lib=None):
    """Brute force: the oracle's operator matrix equals M^T of the forward conv."""
    rng = np.random.default_rng(23)
    for (Cin, Cout, L, K, s, p, d) in [(2, 2, 4, 3, 1, 0, 2), (1, 2, 3, 2, 2, 1, 1)]:
        w = rng.standard_normal((Cin, Cout, K)).astype(np.float32)
        Lo = (L - 1) * s - 2 * p + d * (K - 1) + 1
        # M: forward conv as a matrix [Cin*L, Cout*Lo]
        M = np.zeros((Cin * L, Cout * Lo))
        for co in range(Cout):
            for o in range(Lo):
                e = np.zeros((1, Cout, Lo))
                e[0, co, o] = 1.0
                M[:, co * Lo + o] = _conv1d_forward(e, w.astype(np.float64), s, p, d, L).reshape(-1)
        T = np.zeros((Cout * Lo, Cin * L))
        for ci in range(Cin):
            for i in range(L):
                e = np.zeros((1, Cin, L), dtype=np.float32)
                e[0, ci, i] = 1.0
                T[:, ci * L + i] = oracle.convT1d(e, w, None, s, p, d, 0, lib=lib).reshape(-1)
        assert np.array_equal(T, M.T)


# ------------------------------------------------------ library routines ----
def pin_torch_cpu_fp64(lib=None):
    """Special cases that reduce to PyTorch's own CPU routines, in float64."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(31)
    # fused chain, several geometries (conv bias on and off)
    for (N, Cin, Cout, D, H, W, k, s, p, op, pk) in [(2, 3, 4, 3, 5, 4, 3, 2, 1, 0, 2),
                                                      (1, 2, 3, 4, 4, 3, 3, 2, 1, 1, 2),
                                                      (1, 2, 2, 3, 3, 3, 2, 1, 0, 0, 3)]:
        x = rng.standard_normal((N, Cin, D, H, W)).astype(np.float32)
        w = rng.standard_normal((Cin, Cout, k, k, k)).astype(np.float32)
        cb = rng.standard_normal(Cout).astype(np.float32)
        b = rng.standard_normal(Cout).astype(np.float32)
        for use_cb in (False, True):
            got = oracle.convT3d_scale_pool_bias(x, w, cb if use_cb else None, b, 0.5, 1.5,
                                                 s, p, op, pk, lib=lib)
            t = F.conv_transpose3d(torch.from_numpy(x).double(), torch.from_numpy(w).double(),
                                   torch.from_numpy(cb).double() if use_cb else None,
                                   stride=s, padding=p, output_padding=op)
            t = F.avg_pool3d(t * 0.5, pk)
            t = (t + torch.from_numpy(b).double().view(1, Cout, 1, 1, 1)) * 1.5
            assert got.shape == tuple(t.shape)
            assert np.abs(got - t.numpy()).max() <= 1e-12
    # pool
    for shape, k, s, p in [((2, 3, 6, 7, 8), 3, 2, 1), ((1, 2, 5, 5, 5), 2, 1, 1)]:
        x = rng.standard_normal(shape).astype(np.float32)
        for include in (True, False):
            got = oracle.avgpool3d(x, k, s, p, include, lib=lib)
            t = F.avg_pool3d(torch.from_numpy(x).double(), k, s, p, count_include_pad=include)
            assert np.abs(got - t.numpy()).max() <= 1e-13
    # convT1d
    for (N, Cin, Cout, L, K, s, p, d, op) in [(2, 3, 5, 20, 5, 1, 0, 3, 0),
                                               (1, 2, 3, 9, 3, 2, 1, 2, 1)]:
        x = rng.standard_normal((N, Cin, L)).astype(np.float32)
        w = rng.standard_normal((Cin, Cout, K)).astype(np.float32)
        b = rng.standard_normal(Cout).astype(np.float32)
        got = oracle.convT1d(x, w, b, s, p, d, op, lib=lib)
        t = F.conv_transpose1d(torch.from_numpy(x).double(), torch.from_numpy(w).double(),
                               torch.from_numpy(b).double(), stride=s, padding=p,
                               output_padding=op, dilation=d)
        assert got.shape == tuple(t.shape)
        assert np.abs(got - t.numpy()).max() <= 1e-12


def pin_flipped_conv1d_equivalence(lib=None):
    """convT1d (s1, p0, dilation d) = conv1d of the input padded by (K-1)d with W flipped.

    [p74], passages relating the transposed conv to an ordinary convolution
    with the kernel reversed and padding (K-1)*dilation; the gather form itself
    uses W unflipped.
    """
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(41)
    N, Cin, Cout, L, K, d = 2, 4, 3, 50, 5, 3
    x = rng.standard_normal((N, Cin, L)).astype(np.float32)
    w = rng.standard_normal((Cin, Cout, K)).astype(np.float32)
    got = oracle.convT1d(x, w, None, 1, 0, d, 0, lib=lib)
    wf = torch.from_numpy(w).double().permute(1, 0, 2).flip(2).contiguous()
    t = F.conv1d(torch.from_numpy(x).double(), wf, padding=(K - 1) * d, dilation=d)
    assert got.shape == tuple(t.shape)
    assert np.abs(got - t.numpy()).max() <= 1e-12


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
