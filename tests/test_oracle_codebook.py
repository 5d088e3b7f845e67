"""Pins for the oracle's Lloyd-Max codebook (CPU only).

What pins it, besides itself:
  * the 1-bit closed form (levels +-sqrt(2/pi), edge 0, distortion 1 - 2/pi);
  * the distortions printed in [Scratch] §3 (0.118 / 0.0345 / 0.0095 at 2/3/4 bits);
  * brute force: grid search (b = 1, 2) and direct numerical minimisation (b = 3)
    of the closed-form distortion land on the Lloyd fixed point;
  * the closed-form distortion equals adaptive quadrature of the same integral;
  * at 5-8 bits (root finding instead of the slow iteration): agreement with the
    iteration at 5 bits, the conditional-mean fixed point, the approach of the
    distortion to the high-resolution (Panter-Dite) limit, sampling, and local
    optimality against random moves of the levels.

The Beta-marginal codebook (exact law of a rotated unit vector's coordinate) is
pinned by the uniform law at d = 3, the one-bit closed form E|T|, a Lloyd step
done in 40-digit quadrature, scipy-quadrature of its distortion, direct
minimisation, optimality against the Gaussian codebook with convergence to it
as d grows, and the MSE of quantized random unit vectors.
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


# ---------------------------------------------------------------------------
# Many levels (8-bit keys of [Scratch] §10): the conditions solved by root finding.
# ---------------------------------------------------------------------------
from oracle.codebook import _lloyd_max_gaussian_iter, _lloyd_max_gaussian_root  # noqa: E402


def test_root_solver_matches_the_iteration_at_five_bits():
    lv_i, ed_i = _lloyd_max_gaussian_iter(5)
    lv_r, ed_r = _lloyd_max_gaussian_root(5)
    np.testing.assert_allclose(lv_r, lv_i, atol=1e-11)
    np.testing.assert_allclose(ed_r, ed_i, atol=1e-11)


@pytest.mark.parametrize("bits", [5, 6, 7, 8])
def test_many_level_fixed_point(bits):
    levels, edges = lloyd_max_gaussian(bits)
    L = 1 << bits
    assert levels.shape == (L,) and edges.shape == (L - 1,)
    assert np.all(np.diff(levels) > 0)
    np.testing.assert_array_equal(levels, -levels[::-1])
    np.testing.assert_allclose(edges, 0.5 * (levels[:-1] + levels[1:]), atol=1e-15)
    bnd = np.concatenate([[-np.inf], edges, [np.inf]])
    mass = norm.sf(bnd[:-1]) - norm.sf(bnd[1:])
    cond_mean = (norm.pdf(bnd[:-1]) - norm.pdf(bnd[1:])) / mass
    np.testing.assert_allclose(cond_mean, levels, atol=1e-11)


def test_distortion_tends_to_the_high_resolution_limit():
    """Lloyd-Max distortion over the Panter-Dite value sqrt(3) pi / 2 * 4^-b (the [README]
    bound column) rises monotonically towards 1 as the codebook grows."""
    ratios = [Codebook.build(b, 128).distortion / (math.sqrt(3) * math.pi / 2 * 4.0 ** -b) for b in range(1, 9)]
    assert all(b > a for a, b in zip(ratios, ratios[1:]))
    assert 0.985 < ratios[-1] < 1.0


def test_eight_bit_distortion_by_sampling_and_local_optimality():
    """8 bits: the MSE of 2^21 N(0,1) samples matches the closed form within 4 standard errors,
    and random small moves of the levels (edges kept at midpoints) never lower the distortion."""
    import synth

    cb = Codebook.build(8, 128)
    x = synth.normal(3, 0, 1 << 21)
    q = cb.unit_levels[np.searchsorted(cb.unit_bounds, x, side="left")]
    err = (x - q) ** 2
    assert abs(err.mean() - cb.distortion) < 4 * err.std(ddof=1) / math.sqrt(len(err))
    rng = np.random.default_rng(8)
    half = cb.unit_levels[128:]
    for _ in range(20):
        pos = np.sort(half + rng.normal(scale=1e-3, size=half.size) * np.diff(np.concatenate([[0.0], half])))
        assert _sym_distortion(pos) >= cb.distortion - 1e-15


# ---------------------------------------------------------------------------
# Beta-marginal codebook ([Fork] "How it works": centroids solved for the
# Beta((d-1)/2, (d-1)/2) law of a rotated unit vector's coordinate).
# ---------------------------------------------------------------------------
from oracle.codebook import beta_distortion, lloyd_max_beta  # noqa: E402


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_beta_uniform_law_at_three_dimensions(bits):
    """d = 3: a coordinate of a uniform point on the 2-sphere is uniform on [-1, 1]
    (Archimedes' hat-box theorem), whose Lloyd-Max quantizer is the uniform one:
    levels at the cell midpoints, MSE (2/L)^2/12 per coordinate, i.e. 1/L^2 relative."""
    L = 1 << bits
    levels, edges = lloyd_max_beta(bits, 3)
    s = math.sqrt(3.0)
    np.testing.assert_allclose(levels, s * ((2 * np.arange(L) + 1) / L - 1), atol=1e-13)
    np.testing.assert_allclose(edges, s * (2 * np.arange(1, L) / L - 1), atol=1e-13)
    assert beta_distortion(levels, edges, 3) == pytest.approx(1.0 / L ** 2, abs=1e-14)


@pytest.mark.parametrize("dim", [4, 8, 32, 128, 4096])
def test_beta_one_bit_closed_form(dim):
    """One bit: the levels are +-E|T| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)), edge 0,
    relative MSE 1 - d E|T|^2 (evaluated here in 40-digit arithmetic)."""
    import mpmath

    mpmath.mp.dps = 40
    e_abs = mpmath.gamma(mpmath.mpf(dim) / 2) / (mpmath.sqrt(mpmath.pi) * mpmath.gamma(mpmath.mpf(dim + 1) / 2))
    levels, edges = lloyd_max_beta(1, dim)
    assert levels[1] == pytest.approx(float(mpmath.sqrt(dim) * e_abs), abs=2e-15)
    assert edges[0] == 0.0
    assert beta_distortion(levels, edges, dim) == pytest.approx(float(1 - dim * e_abs ** 2), abs=1e-14)


def test_beta_one_bit_level_is_mean_abs_coordinate():
    """Empirically: E|u_0| * sqrt(d) over uniform unit vectors (normalised Gaussians) in d = 32."""
    import synth

    x = synth.normal(11, 0, 200_000 * 32).reshape(200_000, 32)
    a = np.abs(x[:, 0]) / np.linalg.norm(x, axis=1) * math.sqrt(32)
    level = lloyd_max_beta(1, 32)[0][1]
    assert abs(a.mean() - level) < 4 * a.std(ddof=1) / math.sqrt(len(a))


@pytest.mark.parametrize("dim", [8, 32, 128])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_beta_fixed_point_in_high_precision(dim, bits):
    """One Lloyd step, with the cell integrals of the density c_d (1-t^2)^((d-3)/2) done by
    40-digit quadrature, leaves the oracle's levels in place; edges are midpoints; symmetric."""
    import mpmath

    mpmath.mp.dps = 40
    levels, edges = lloyd_max_beta(bits, dim)
    np.testing.assert_array_equal(levels, -levels[::-1])
    np.testing.assert_allclose(edges, 0.5 * (levels[:-1] + levels[1:]), atol=1e-15)
    s = mpmath.sqrt(dim)
    k = mpmath.mpf(dim - 3) / 2
    bnd = [mpmath.mpf(-1)] + [mpmath.mpf(float(e)) / s for e in edges] + [mpmath.mpf(1)]
    for i in range(len(levels)):
        m0 = mpmath.quad(lambda t: (1 - t * t) ** k, [bnd[i], bnd[i + 1]])
        m1 = mpmath.quad(lambda t: t * (1 - t * t) ** k, [bnd[i], bnd[i + 1]])
        assert float(s * m1 / m0) == pytest.approx(levels[i], abs=1e-12), (i, levels[i])


def test_beta_distortion_equals_quadrature():
    """beta_distortion against adaptive quadrature of (x - c)^2 under scipy's Beta(a, a) density."""
    from scipy.stats import beta as beta_law

    rng = np.random.default_rng(9)
    for dim in (8, 32, 128):
        a = (dim - 1) / 2
        s = math.sqrt(dim)
        for _ in range(3):
            lv = np.sort(rng.normal(size=8))
            ed = 0.5 * (lv[:-1] + lv[1:])
            bnd = [-s] + list(ed) + [s]
            # X = sqrt(d) T with (T + 1)/2 ~ Beta(a, a): density beta.pdf((x/s + 1)/2) / (2 s)
            pdf = lambda x: beta_law.pdf((x / s + 1) / 2, a, a) / (2 * s)
            quad = sum(integrate.quad(lambda x, c=c: (x - c) ** 2 * pdf(x), max(-s, bnd[i]), min(s, bnd[i + 1]),
                                      epsabs=1e-14, epsrel=1e-12)[0] for i, c in enumerate(lv))
            assert beta_distortion(lv, ed, dim) == pytest.approx(quad, rel=1e-9)


def test_beta_direct_minimisation_three_bit():
    """Nelder-Mead on the symmetric 3-bit distortion (d = 32) lands on the Lloyd fixed point."""
    levels = lloyd_max_beta(3, 32)[0]

    def f(pos):
        pos = np.sort(np.abs(np.asarray(pos, dtype=np.float64)))
        lv = np.concatenate([-pos[::-1], pos])
        return beta_distortion(lv, 0.5 * (lv[:-1] + lv[1:]), 32)

    res = optimize.minimize(f, x0=[0.3, 0.9, 1.5, 2.4], method="Nelder-Mead",
                            options={"xatol": 1e-9, "fatol": 1e-15, "maxiter": 20000, "maxfev": 40000})
    np.testing.assert_allclose(np.sort(np.abs(res.x)), levels[4:], atol=2e-4)
    assert res.fun == pytest.approx(Codebook.build_beta(3, 32).distortion, rel=1e-7)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_beta_codebook_beats_gaussian_and_tends_to_it(bits):
    """Under the exact law the Beta codebook's MSE is below the Gaussian codebook's (it is the
    optimum for that law), and the two codebooks merge as d grows (the law tends to N(0,1))."""
    g_lv, g_ed = lloyd_max_gaussian(bits)
    gaps = []
    for dim in (8, 32, 128, 512, 4096):
        cb = Codebook.build_beta(bits, dim)
        if dim <= 128:
            assert cb.distortion < beta_distortion(g_lv, g_ed, dim)
        gaps.append(np.max(np.abs(cb.unit_levels - g_lv)))
    assert all(b < a for a, b in zip(gaps, gaps[1:]))
    assert gaps[-1] < 2e-3
    # the Gaussian codebook's own distortion is the large-d limit (the law differs from N(0,1) at O(1/d))
    assert abs(Codebook.build_beta(bits, 4096).distortion - gaussian_distortion(g_lv, g_ed)) < 1.0 / 4096


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_beta_codebook_on_unit_vectors_in_32_dimensions(bits):
    """Quantizing uniform unit vectors in d = 32 (one block-32 unit): the mean MSE matches the
    Beta codebook's distortion, and the paired gain over the Gaussian codebook matches the
    exact difference of the two distortions under the Beta law, each within 4 standard errors."""
    import synth
    from oracle import dequantize, quantize

    n = 20_000
    x = synth.normal(0, 0, n * 32).reshape(n, 32)
    D = synth.signs(0, 2, 32)
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    err = {}
    cbs = {"beta": Codebook.build_beta(bits, 32), "gauss": Codebook.build(bits, 32)}
    for kind, cb in cbs.items():
        q = quantize(x, D, cb, norm_dtype=np.float64)
        err[kind] = np.sum((u - dequantize(q["codes"], np.ones(n), D, cb)) ** 2, axis=1)
    se = err["beta"].std(ddof=1) / math.sqrt(n)
    assert abs(err["beta"].mean() - cbs["beta"].distortion) < 4 * se
    gain = err["gauss"] - err["beta"]
    exact_gain = beta_distortion(cbs["gauss"].unit_levels, cbs["gauss"].unit_bounds, 32) - cbs["beta"].distortion
    assert exact_gain > 0
    assert abs(gain.mean() - exact_gain) < 4 * gain.std(ddof=1) / math.sqrt(n)
