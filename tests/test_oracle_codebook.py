"""Pins for the oracle's Lloyd-Max codebook (CPU only).

What pins it, besides itself:
  * the 1-bit closed form (levels +-sqrt(2/pi), edge 0, distortion 1 - 2/pi);
  * the distortions printed in [Scratch] §3 (0.118 / 0.0345 / 0.0095 at 2/3/4 bits);
  * brute force: grid search (b = 1, 2) and direct numerical minimisation (b = 3)
    of the closed-form distortion land on the Lloyd fixed point;
  * the closed-form distortion equals adaptive quadrature of the same integral.
"""
import math

import numpy as np
import pytest
from scipy import integrate, optimize
from scipy.stats import norm

from oracle.codebook import Codebook, gaussian_distortion, lloyd_max_gaussian


def _printed_tolerance(value: float) -> float:
    """One unit in the last printed digit: the page quotes these as 'about' x."""
    text = repr(value)
    decimals = len(text.split(".")[1]) if "." in text else 0
    return 10.0 ** (-decimals)


def test_one_bit_closed_form():
    levels, edges = lloyd_max_gaussian(1)
    c = math.sqrt(2.0 / math.pi)
    assert levels == pytest.approx([-c, c], abs=1e-15)
    assert edges == pytest.approx([0.0], abs=0.0)
    assert gaussian_distortion(levels, edges) == pytest.approx(1.0 - 2.0 / math.pi, abs=1e-14)


def test_distortion_matches_printed_digits(golden):
    g = golden("scratch_distortion.json")
    for bits, printed in zip(g["bits"], g["relative_distortion"]):
        d = Codebook.build(bits, 128).distortion
        assert abs(d - printed) <= _printed_tolerance(printed), (bits, d, printed)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_fixed_point_and_symmetry(bits):
    levels, edges = lloyd_max_gaussian(bits)
    L = 1 << bits
    assert levels.shape == (L,) and edges.shape == (L - 1,)
    assert np.all(np.diff(levels) > 0) and np.all(np.diff(edges) > 0)
    np.testing.assert_array_equal(levels, -levels[::-1])
    np.testing.assert_array_equal(edges, -edges[::-1])
    # edges are midpoints
    np.testing.assert_allclose(edges, 0.5 * (levels[:-1] + levels[1:]), atol=1e-15)
    # one more conditional-mean step does not move the levels
    bnd = np.concatenate([[-np.inf], edges, [np.inf]])
    mass = norm.cdf(bnd[1:]) - norm.cdf(bnd[:-1])
    cond_mean = (norm.pdf(bnd[:-1]) - norm.pdf(bnd[1:])) / mass
    np.testing.assert_allclose(cond_mean, levels, atol=1e-12)


def test_closed_form_distortion_equals_quadrature():
    rng = np.random.default_rng(5)
    for _ in range(5):
        lv = np.sort(rng.normal(size=8))
        ed = 0.5 * (lv[:-1] + lv[1:])
        bnd = [-np.inf] + list(ed) + [np.inf]
        quad = sum(
            integrate.quad(lambda x, c=c: (x - c) ** 2 * norm.pdf(x), bnd[i], bnd[i + 1], epsabs=1e-13)[0]
            for i, c in enumerate(lv)
        )
        assert gaussian_distortion(lv, ed) == pytest.approx(quad, rel=1e-9)


def _sym_distortion(pos_levels):
    pos = np.sort(np.abs(np.asarray(pos_levels, dtype=np.float64)))
    lv = np.concatenate([-pos[::-1], pos])
    ed = 0.5 * (lv[:-1] + lv[1:])
    return gaussian_distortion(lv, ed)


def test_brute_force_one_bit():
    grid = np.arange(0.70, 0.90, 1e-5)
    vals = [_sym_distortion([c]) for c in grid]
    best = grid[int(np.argmin(vals))]
    assert best == pytest.approx(lloyd_max_gaussian(1)[0][1], abs=2e-5)


def test_brute_force_two_bit():
    levels = lloyd_max_gaussian(2)[0]
    a_grid = np.arange(0.30, 0.60, 2e-3)
    b_grid = np.arange(1.30, 1.70, 2e-3)
    best = min((_sym_distortion([a, b]), a, b) for a in a_grid for b in b_grid)
    a0, b0 = best[1], best[2]
    a_fine = np.arange(a0 - 3e-3, a0 + 3e-3, 5e-5)
    b_fine = np.arange(b0 - 3e-3, b0 + 3e-3, 5e-5)
    best = min((_sym_distortion([a, b]), a, b) for a in a_fine for b in b_fine)
    assert best[1] == pytest.approx(levels[2], abs=1e-4)
    assert best[2] == pytest.approx(levels[3], abs=1e-4)


def test_direct_minimisation_three_bit():
    levels = lloyd_max_gaussian(3)[0]
    res = optimize.minimize(_sym_distortion, x0=[0.3, 0.9, 1.5, 2.4], method="Nelder-Mead",
                            options={"xatol": 1e-9, "fatol": 1e-15, "maxiter": 20000, "maxfev": 40000})
    np.testing.assert_allclose(np.sort(np.abs(res.x)), levels[4:], atol=2e-4)
    assert res.fun == pytest.approx(Codebook.build(3, 64).distortion, rel=1e-7)


def test_scaling_to_dimension():
    cb = Codebook.build(3, 128)
    np.testing.assert_allclose(cb.levels * math.sqrt(128), cb.unit_levels, rtol=0, atol=1e-15)
    np.testing.assert_allclose(cb.bounds * math.sqrt(128), cb.unit_bounds, rtol=0, atol=1e-15)
