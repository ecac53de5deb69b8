"""The seeded generator draws what the workload recipe says, reproducibly."""
import numpy as np

import synth


def test_trit_distribution_and_determinism():
    t = synth.trits(synth.rng(1, 0), 512, 1024)
    assert t.dtype == np.int8 and set(np.unique(t)) <= {-1, 0, 1}
    p0 = np.mean(t == 0)
    assert abs(p0 - 0.5) < 0.005 and abs(np.mean(t == 1) - 0.25) < 0.005
    assert np.array_equal(t, synth.trits(synth.rng(1, 0), 512, 1024))
    assert not np.array_equal(t, synth.trits(synth.rng(1, 0, 1), 512, 1024))


def test_scales_are_fp16_of_half_normal_plus_offset():
    s = synth.f16_bits_to_f64(synth.scales_f16(synth.rng(1, 1), 256, 1024))
    assert s.shape == (256, 8) and s.min() >= 1e-3 * 0.999
    assert abs(np.mean(s) - (0.02 * np.sqrt(2 / np.pi) + 1e-3)) < 1e-3


def test_activations_bf16_and_outliers():
    k = 5120
    oc = synth.outlier_channels(synth.rng(1, 4), k)
    assert len(oc) == 5 and len(set(oc.tolist())) == 5
    xb = synth.activations(synth.rng(1, 2), 64, k, oc, "bf16")
    x = synth.bf16_bits_to_f64(xb)
    # every value is representable in bf16: low 16 bits of its float32 pattern are zero
    assert np.all((x.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)
    big = np.abs(x[:, oc]).mean()
    rest = np.abs(np.delete(x, oc, axis=1)).mean()
    assert 12 < big / rest < 28


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.00390625], dtype=np.float32)
    got = synth.bf16_bits_to_f64(synth.f32_to_bf16_bits(vals))
    assert got.tolist() == [1.0, 1.0, 1.015625, -2.5, 1.0]


def test_sign_bits_tiled_per_block():
    w = synth.sign_bits(synth.rng(1, 3), 3072)
    assert w.dtype == np.uint32 and w.shape == (96,)
    assert np.array_equal(w[:32], w[32:64]) and np.array_equal(w[:32], w[64:])
    ones = sum(bin(int(v)).count("1") for v in w[:32])
    assert 400 < ones < 624
