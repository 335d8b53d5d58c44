"""The seeded input generator: Philox4x32-10 known-answer vectors, element-range
independence, distribution sanity and bf16 rounding.  CPU only."""
import numpy as np

import synth


def test_philox_known_answers():
    # Known-answer vectors published with the Random123 library
    # (Salmon et al., SC'11) for Philox4x32 with 10 rounds.
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]),
        ([0xffffffff] * 4, [0xffffffff] * 2, [0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd]),
        ([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344], [0xa4093822, 0x299f31d0],
         [0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1]),
    ]
    for ctr, key, exp in kat:
        assert synth.philox4x32_10(ctr, key) == exp


def test_ranges_are_independent():
    full = synth.normal(123, 0, (10007,))
    for first, n in [(0, 1), (1, 3), (5, 100), (4093, 2000), (10000, 7)]:
        part = synth.normal(123, 0, (n,), first=first)
        assert np.array_equal(part, full[first:first + n])
    fu = synth.uniform(9, 1, (999,), -2.0, 3.0)
    assert np.array_equal(synth.uniform(9, 1, (50,), -2.0, 3.0, first=333), fu[333:383])


def test_distributions():
    z = synth.normal(1, 0, (1 << 20,))
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1.0) < 5e-3
    u = synth.uniform(1, 1, (1 << 20,), -0.5, 0.5)
    assert u.min() >= -0.5 and u.max() < 0.5 and abs(u.mean()) < 2e-3
    # different streams / seeds differ
    assert not np.array_equal(synth.normal(1, 0, (64,)), synth.normal(1, 1, (64,)))
    assert not np.array_equal(synth.normal(1, 0, (64,)), synth.normal(2, 0, (64,)))


def test_bf16_round_nearest_even():
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20,
                     -2.5, 65504.0, np.inf, -np.inf], dtype=np.float32)
    exp_f = np.array([1.0, 1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -2.5, 65536.0, np.inf, -np.inf],
                     dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.to_bf16_bits(vals))
    assert np.array_equal(got, exp_f)
    nan = synth.bf16_bits_to_f32(synth.to_bf16_bits(np.array([np.nan], np.float32)))
    assert np.isnan(nan).all()


def test_workload_inputs_shapes():
    wl = synth.WORKLOADS["c1"]
    t = synth.make_inputs(wl, conv_bias=True)
    assert t["x"].shape == (2, 3, 8, 16, 16) and t["w"].shape == (3, 16, 3, 3, 3)
    assert t["bias"].shape == (16,) and t["conv_bias"].shape == (16,)
    assert np.abs(t["w"]).max() <= 1.0 / 9.0
    t5 = synth.make_inputs(synth.WORKLOADS["c5"])
    assert t5["x_bits"].dtype == np.uint16
    assert np.array_equal(synth.bf16_bits_to_f32(t5["x_bits"]).reshape(t5["x"].shape), t5["x"])
