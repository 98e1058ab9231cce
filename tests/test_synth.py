"""The seeded input generator: determinism, counter property, distributions (no GPU)."""
import numpy as np

import synth


def test_splitmix64_reference_outputs():
    # SplitMix64 started from state 0 (Steele, Lea & Flood 2014; the widely published
    # reference sequence): first outputs of the sequential generator.
    assert [hex(v) for v in synth.u64(0, 3).tolist()] == [
        "0xe220a8397b1dcdaf", "0x6e789e6aa1b965f4", "0x6c45d188009454f"]


def test_counter_property_and_determinism():
    a = synth.u64(1234, 1000)
    b = synth.u64(1234, 400, start=600)
    assert np.array_equal(a[600:], b)
    assert np.array_equal(synth.trits(9, 33, 77), synth.trits(9, 33, 77))
    assert not np.array_equal(synth.trits(9, 33, 77), synth.trits(10, 33, 77))


def test_trit_distribution():
    for z in synth.P_ZERO_SWEEP:
        w = synth.trits(5, 1000, 1000, z)
        n = w.size
        f0 = np.mean(w == 0)
        fp = np.mean(w == 1)
        fm = np.mean(w == -1)
        sd = np.sqrt(z * (1 - z) / n)
        assert abs(f0 - z) < 6 * sd
        assert abs(fp - fm) < 6 * np.sqrt((1 - z) / n)
        assert set(np.unique(w).tolist()) <= {-1, 0, 1}


def test_activation_codes():
    x, s = synth.activation(3, 2560)
    v = synth.normal_f32(3, 2560)
    assert x.dtype == np.int8 and x.min() >= -127 and x.max() <= 127
    assert int(np.abs(x).max()) == 127
    assert np.float32(s) == np.float32(np.abs(v).max()) / np.float32(127.0)
    assert abs(v.mean()) < 0.1 and abs(v.std() - 1) < 0.05
    z, sz = synth.absmax_codes(np.zeros(10, np.float32))
    assert sz == 0.0 and not z.any()


def test_weight_scale_range_and_head():
    s = [synth.weight_scale(i) for i in range(200)]
    assert min(s) >= 0.5 and max(s) <= 2.0
    w, x = synth.head_case(4, rows=64, cols=128)
    wf = (w.astype(np.uint32) << 16).view(np.float32)
    assert abs(wf.std() - 0.02) < 0.002
    assert np.array_equal(synth.bf16_from_f32(wf), w)  # values already in bf16 round-trip
