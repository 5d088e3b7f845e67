"""The seeded input generator (CPU only): exact binary16 rounding, index-pure
draws, distribution moments, KV shaping (channel scales and outliers)."""
import math

import numpy as np
import pytest

import synth


def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(0)
    a = rng.standard_normal(200_000) * np.exp(rng.uniform(-35, 12, 200_000))
    a = np.concatenate([a, [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e300, -1e300, 2.0**-24, 2.0**-25,
                            3 * 2.0**-26, np.inf, -np.inf]])
    with np.errstate(over="ignore"):
        ref = a.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(synth.to_f16(a).view(np.uint16), ref)


def test_draws_are_pure_functions_of_index():
    whole = synth.normal(7, 3, 1000)
    parts = np.concatenate([synth.normal(7, 3, 333, 0), synth.normal(7, 3, 667, 333)])
    np.testing.assert_array_equal(whole, parts)
    assert not np.array_equal(synth.normal(7, 3, 100), synth.normal(7, 4, 100))
    assert not np.array_equal(synth.normal(7, 3, 100), synth.normal(8, 3, 100))
    np.testing.assert_array_equal(synth.normal_f16(7, 3, 1000), synth.to_f16(whole))
    np.testing.assert_array_equal(synth.normal_f32(7, 3, 1000), whole.astype(np.float32))


def test_moments():
    u = synth.uniform(1, 0, 400_000)
    assert u.min() >= 0.0 and u.max() < 1.0
    assert u.mean() == pytest.approx(0.5, abs=3e-3)
    z = synth.normal(1, 1, 400_000)
    assert z.mean() == pytest.approx(0.0, abs=6e-3)
    assert z.var() == pytest.approx(1.0, abs=1e-2)
    assert np.mean(z**4) == pytest.approx(3.0, abs=0.06)
    s = synth.signs(0, 2, 4096)
    assert set(np.unique(s)) == {-1.0, 1.0}
    assert abs(s.mean()) < 0.1


def test_kv_shaping_and_outliers():
    layers, heads, tokens, hd = 2, 3, 4096, 64
    k = synth.kv_tensor(0, layers, heads, 0, tokens, hd, f16=False)
    v = synth.kv_tensor(0, layers, heads, 1, tokens, hd, f16=False)
    assert not np.array_equal(k, v)
    k16 = synth.kv_tensor(0, layers, heads, 0, tokens, hd)
    np.testing.assert_array_equal(k16.view(np.uint16), synth.to_f16(k).view(np.uint16))
    plain = synth.kv_tensor(0, layers, heads, 0, tokens, hd, outlier_mult=1.0, f16=False)
    ratio = k / plain  # only the outlier multiplier differs
    for layer in range(layers):
        for h in range(heads):
            per_channel = ratio[layer, h, 0]
            np.testing.assert_allclose(ratio[layer, h], np.broadcast_to(per_channel, (tokens, hd)), rtol=1e-12)
            assert np.sum(np.isclose(per_channel, 10.0)) == 2
            assert np.sum(np.isclose(per_channel, 1.0)) == hd - 2
            # log of the channel scales (sample std per channel) has sd ~ sigma = 1
            log_s = np.log(plain[layer, h].std(axis=0))
            assert 0.6 < log_s.std() < 1.4
    k0 = synth.kv_tensor(0, 1, 1, 0, tokens, hd, n_outliers=0, f16=False)
    assert np.all(np.isfinite(k0))
