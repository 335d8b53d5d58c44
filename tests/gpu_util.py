"""Helpers shared by the GPU parity tests: elementwise comparison with the
oracle, non-finite checks, bf16 conversions and device uploads."""
import numpy as np

import synth


def log(msg):
    print(msg, flush=True)


def assert_close(got, ref, tol, what=""):
    """|got - ref| <= atol + rtol * |ref| for every element (NaN fails)."""
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


def assert_close_nonfinite(got, ref, tol, what="", exact_nonfinite=True):
    """Finite oracle values within tolerance; where the oracle is not finite
    the GPU value is not finite either.  With exact_nonfinite the NaN and
    signed-infinity patterns must be identical; without it (results that
    depend on summation order, such as Inf * w summed over weights of both
    signs) only the non-finite set must match."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), (
        f"{what}: non-finite set differs; gpu {int((~np.isfinite(got)).sum())} vs oracle "
        f"{int((~fin).sum())}")
    if exact_nonfinite:
        assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{what}: NaN set differs"
        inf = np.isinf(ref)
        assert np.array_equal(np.sign(got[inf]), np.sign(ref[inf])), f"{what}: Inf signs differ"
    assert_close(got[fin], ref[fin], tol, what + " (finite part)")


def bf16_round(a):
    return synth.bf16_bits_to_f32(synth.to_bf16_bits(a)).reshape(a.shape)


def bf16_tensor_to_f32(t):
    """A torch bf16 tensor's values as a float32 numpy array."""
    import torch
    o = t.view(torch.int16).cpu().numpy().view(np.uint16)
    return synth.bf16_bits_to_f32(o).reshape(o.shape)


def to_dev(a, dev, dtype="f32"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(synth.to_bf16_bits(a).reshape(a.shape).view(np.int16)).to(
            dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def opt(a, dev):
    import torch
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def nan_like(shape, dev, dtype=None):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype or torch.float32, device=dev)
