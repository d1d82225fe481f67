"""The seeded input generator: published test vector, determinism, moments,
bf16 rounding, the row-scale recipes."""
import numpy as np

import synth


def test_splitmix64_published_vector():
    # SplitMix64 seeded with 1234567: the first five published outputs.
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    state = 1234567
    got = []
    for _ in range(5):
        got.append(synth.mix(state))
        state = (state + 0x9E3779B97F4A7C15) % (1 << 64)
    assert got == want


def test_deterministic_and_row_subset():
    wl = synth.get_workload("decode_m16_k4096_n6144")
    a = synth.make_inputs(wl)
    b = synth.make_inputs(wl)
    assert np.array_equal(a.bits["X"], b.bits["X"]) and np.array_equal(a.bits["W1"], b.bits["W1"])
    rows = [3, 0, 15]
    c = synth.make_inputs(wl, rows=rows, weights=False)
    assert np.array_equal(c.bits["X"], a.bits["X"][rows])


def test_moments():
    wl = synth.get_workload("decode_m16_k4096_n6144")
    inp = synth.make_inputs(wl)
    assert abs(inp.X.mean()) < 0.01 and abs(inp.X.std() - 1.0) < 0.01
    assert abs(inp.g.mean() - 1.0) < 0.01 and abs(inp.g.std() - 0.1) < 0.005
    assert abs(inp.W1.std() * np.sqrt(wl.K) - 1.0) < 0.01


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -1.0 - 2**-8,
                  257.0, 259.0, np.inf, -np.inf, 0.0, -0.0, 3.0e38], np.float32)
    want = np.array([1.0, 1.0, 1.0 + 2**-6, 1.0 + 2**-7, -1.0, 256.0, 260.0, np.inf, -np.inf,
                     0.0, -0.0, 3.0e38], np.float64)
    got = synth.bf16_bits_to_f32(synth.to_bf16_bits(f)).astype(np.float64)
    assert np.array_equal(got[:-1], want[:-1])
    assert abs(got[-1] / want[-1] - 1) < 2**-8
    nan = synth.bf16_bits_to_f32(synth.to_bf16_bits(np.array([np.nan], np.float32)))
    assert np.isnan(nan[0])


def test_row_scale_recipes():
    wl = synth.get_workload("prefill_m4096_k4096_n4096")
    s = synth.row_scales(wl)
    assert (s == 100.0).sum() == 41 and (s == 1.0).sum() == 4096 - 41
    wl5 = synth.get_workload("large_m8192_k8192_n28672")
    s5 = synth.row_scales(wl5)
    assert s5.min() >= 0.01 and s5.max() < 100.0
    # log10 of the scale is uniform on [-2, 2)
    assert abs(np.log10(s5).mean()) < 0.1


def test_exact_inputs_are_small_integers():
    inp = synth.make_exact_inputs(32, 64, 48, "bf16", seed=3, row_pow2=True)
    for a in (inp.g, inp.W1):
        assert np.array_equal(a, np.round(a))
    assert set(np.unique(inp.g)) <= {1.0, 2.0}
    assert set(np.unique(inp.W1)) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
    mag = np.abs(inp.X)
    assert np.all(mag == mag[:, :1])  # constant magnitude per row, a power of two
    assert np.all(np.log2(mag[:, 0]) == np.round(np.log2(mag[:, 0])))
