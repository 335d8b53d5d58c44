"""HIP graph capture of the entry points.

Every entry point enqueues only kernel launches on the caller's stream: no
allocation, no memset, no synchronisation (its per-device queries are cached
by the first call).  A caller may therefore capture calls into a HIP graph
(torch.cuda.graph) and replay them, which takes the host launch cost off
launch-bound workloads.  Each case computes the eager result, captures the
same call writing to its own output, and replays the graph three times with
the output refilled with NaN by eager work in between; every replay must
equal the eager result bit for bit.
"""
import numpy as np
import pytest

import synth
from gpu_util import bf16_round, log, to_dev

torch = pytest.importorskip("torch")
import transposed_conv_pooling_amd as ct  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def weights(seed, shape, fan, bf16):
    w = synth.uniform(seed, 1, shape, -1.0 / np.sqrt(fan), 1.0 / np.sqrt(fan))
    return bf16_round(w) if bf16 else w


def case_inputs(name, dev):
    """(call(out), output shape, output dtype) for one case."""
    if name.startswith("fused"):
        bf16 = name.endswith("bf16")
        N, Cin, Cout, D, H, W = (2, 32, 64, 4, 9, 32) if bf16 else (2, 3, 16, 8, 16, 16)
        x = synth.normal(9100, 0, (N, Cin, D, H, W))
        x = bf16_round(x) if bf16 else x
        w = weights(9100, (Cin, Cout, 3, 3, 3), Cin * 27, bf16)
        dt = "bf16" if bf16 else "f32"
        xg, wg = to_dev(x, dev, dt), to_dev(w, dev, dt)
        b = to_dev(synth.normal(9100, 2, (Cout,)), dev)

        def call(out):
            ct.ct_convT3d_scale_pool_bias(xg, wg, None, b, 0.5, 1.0, out=out)
        return call, (N, Cout, D - 1, H - 1, W - 1), torch.float32
    if name == "fused_general":
        N, Cin, Cout, D, H, W = 2, 3, 5, 4, 5, 6
        x = synth.normal(9101, 0, (N, Cin, D, H, W))
        w = weights(9101, (Cin, Cout, 4, 4, 4), Cin * 64, False)
        xg, wg = to_dev(x, dev), to_dev(w, dev)
        cb = to_dev(synth.normal(9101, 3, (Cout,)), dev)
        dims = ct._fused_dims(D, H, W, 4, 2, 1, 1, 3, 2)

        def call(out):
            ct.ct_convT3d_scale_pool_bias(xg, wg, cb, None, 0.5, 1.0, stride=2, pad=1, out_pad=1,
                                          pool_k=3, pool_s=2, out=out)
        return call, (N, Cout) + dims, torch.float32
    if name.startswith("pool"):
        bf16 = name.endswith("bf16")
        shape = (2, 3, 9, 40, 64)
        x = synth.normal(9102, 0, shape)
        xg = to_dev(bf16_round(x) if bf16 else x, dev, "bf16" if bf16 else "f32")

        def call(out):
            ct.ct_avgpool3d(xg, 3, 2, 1, True, out=out)
        return call, (2, 3, 5, 20, 32), torch.bfloat16 if bf16 else torch.float32
    if name == "convT3d":
        x = synth.normal(9103, 0, (2, 3, 4, 5, 6))
        w = weights(9103, (3, 7, 3, 3, 3), 81, False)
        xg, wg = to_dev(x, dev), to_dev(w, dev)

        def call(out):
            ct.ct_convT3d(xg, wg, None, stride=2, pad=1, out_pad=0, out=out)
        return call, (2, 7, 7, 9, 11), torch.float32
    # 1D convs at the page's channels and taps: stride 1 fp32 and bf16 (pad 0,
    # and pad 1 with its output length % 4 != 0), stride 2 fp32
    bf16 = name.endswith("bf16")
    stride = 2 if "s2" in name else 1
    N, Cin, Cout, L = 2, 32, 64, 1024
    x = synth.normal(9104, 0, (N, Cin, L))
    x = bf16_round(x) if bf16 else x
    w = weights(9104, (Cin, Cout, 5), Cin * 5, bf16)
    dt = "bf16" if bf16 else "f32"
    xg, wg = to_dev(x, dev, dt), to_dev(w, dev, dt)
    pad, op = (1, 1) if stride == 2 else (1, 0) if "p1" in name else (0, 0)
    Lo = ct.ct_convT_out_len(L, 5, stride, pad, op, 3)

    def call(out):
        ct.ct_convT1d(xg, wg, None, stride=stride, pad=pad, dilation=3, out_pad=op, out=out)
    return call, (N, Cout, Lo), torch.float32


CASES = ["fused_f32", "fused_bf16", "fused_general", "pool_f32", "pool_bf16", "convT3d",
         "conv1d_f32", "conv1d_s2_f32", "conv1d_bf16", "conv1d_p1_f32", "conv1d_p1_bf16"]


@pytest.mark.parametrize("name", CASES)
def test_graph_replay_matches_eager(dev, name):
    log(f"graph capture {name}")
    call, shape, dtype = case_inputs(name, dev)
    ref = torch.full(shape, float("nan"), dtype=dtype, device=dev)
    call(ref)                                   # eager; also fills the per-device caches
    torch.cuda.synchronize()
    assert not torch.isnan(ref.float()).any(), f"{name}: eager output incomplete"
    out = torch.empty(shape, dtype=dtype, device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{name}: replay {r} differs from the eager result"
