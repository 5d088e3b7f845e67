"""Statistical pins for the oracle's reconstruction and QJL estimator (CPU only).

  * MSE of random unit vectors at d = 128: the empirical mean sits within 4
    standard errors of the exact finite-d expectation (coordinate marginal of a
    uniform unit vector, integrated per cell), the exact expectation agrees with
    the values printed in [README] "MSE Distortion" (for a 1000-vector sample),
    and stays below the printed upper-bound column, which equals
    sqrt(3) pi / 2 * 4^-b.
  * shrinkage: E||u~||^2 = 1 - MSE (orthogonality of the Lloyd-Max cells) and
    norm correction restores ||u~|| = 1 exactly ([Scratch] §6).
  * QJL: unbiased over many draws of S, with the closed-form per-draw variance
    rho^2/m ((pi/2)||q||^2 - <q, r/rho>^2); bias and correlation of [README]
    "Inner Product Accuracy"; and the dequantize path agrees with the score path.
"""
import math

import numpy as np
import pytest
from scipy import integrate, special

import synth
from oracle import QJL_CONST, Codebook, dequantize, qjl_scores, quantize

D_MODEL = 128


def _exact_unit_mse(cb: Codebook) -> float:
    d = cb.dim
    lc = special.gammaln(d / 2) - 0.5 * math.log(math.pi) - special.gammaln((d - 1) / 2)
    pdf = lambda t: math.exp(lc + (d - 3) / 2 * math.log1p(-t * t))
    edges = [-1.0] + list(cb.bounds) + [1.0]
    per_coord = sum(
        integrate.quad(lambda t, c=c: (t - c) ** 2 * pdf(t), edges[i], edges[i + 1], epsabs=1e-15, epsrel=1e-12)[0]
        for i, c in enumerate(cb.levels)
    )
    return d * per_coord


@pytest.fixture(scope="module")
def unit_vectors():
    x = synth.normal(0, 0, 1000 * D_MODEL).reshape(1000, D_MODEL)
    return x, synth.signs(0, 2, D_MODEL)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_mse_random_unit_vectors(bits, unit_vectors, golden):
    g = golden("readme_mse_table.json")
    row = g["bits"].index(bits)
    x, D = unit_vectors
    cb = Codebook.build(bits, D_MODEL)
    q = quantize(x, D, cb, norm_dtype=np.float64)
    rec = dequantize(q["codes"], np.ones(len(x)), D, cb)
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    err = np.sum((u - rec) ** 2, axis=1)
    mean, se = err.mean(), err.std(ddof=1) / math.sqrt(len(err))
    exact = _exact_unit_mse(cb)
    assert abs(mean - exact) < 4 * se, (mean, exact, se)
    # the page measured 1000 vectors too: its number must be a plausible sample of the exact mean
    printed = g["measured_mse"][row]
    assert abs(printed - exact) <= 0.5 * 10 ** -3 + 3 * se, (printed, exact)
    bound = math.sqrt(3) * math.pi / 2 * 4.0 ** (-bits)
    assert abs(bound - g["upper_bound"][row]) <= 0.5e-3
    assert exact < bound and mean < bound
    # finite-d MSE is slightly below the Gaussian distortion
    assert exact < cb.distortion


def test_shrinkage_and_norm_correction(unit_vectors):
    x, D = unit_vectors
    for bits in (2, 3, 4):
        cb = Codebook.build(bits, D_MODEL)
        q = quantize(x, D, cb, norm_dtype=np.float64)
        rec = dequantize(q["codes"], np.ones(len(x)), D, cb)
        sq = np.sum(rec * rec, axis=1)
        exact = _exact_unit_mse(cb)
        se = sq.std(ddof=1) / math.sqrt(len(sq))
        assert abs(sq.mean() - (1.0 - exact)) < 4 * se + 1e-12
        rec_nc = dequantize(q["codes"], np.ones(len(x)), D, cb, nc=True)
        np.testing.assert_allclose(np.linalg.norm(rec_nc, axis=1), 1.0, atol=1e-14)
        # MSE-only inner products are biased low: slope of <q, u~> on <q, u> is ~ 1 - MSE
        qv = synth.normal(9, 6, len(x) * D_MODEL).reshape(len(x), D_MODEL)
        u = x / np.linalg.norm(x, axis=1, keepdims=True)
        true_ip = np.sum(qv * u, axis=1)
        est_ip = np.sum(qv * rec, axis=1)
        slope = np.sum(true_ip * est_ip) / np.sum(true_ip * true_ip)
        assert slope == pytest.approx(1.0 - exact, abs=0.02)


def test_qjl_unbiased_over_projection_draws():
    d = m = D_MODEL
    cb = Codebook.build(2, d)
    D = synth.signs(11, 2, d)
    k = synth.normal(11, 0, d)
    qv = synth.normal(11, 6, d)
    exact = float(qv @ k)
    draws = 2000
    est = np.empty(draws)
    for s in range(draws):
        S = synth.gaussian_matrix(1000 + s, 0, m, d)
        enc = quantize(k[None, :], D, cb, norm_dtype=np.float64, S=S)
        est[s] = qjl_scores(qv[None, :], enc["codes"], enc["norms"], enc["qjl_bits"], enc["rho_exact"], D, cb, S)[0, 0]
    se = est.std(ddof=1) / math.sqrt(draws)
    assert abs(est.mean() - exact) < 4 * se, (est.mean(), exact, se)
    # closed-form variance (per draw)
    n = np.linalg.norm(k)
    enc = quantize(k[None, :], D, cb, norm_dtype=np.float64, S=np.eye(m))
    u_mse = dequantize(enc["codes"], np.ones(1), D, cb)[0]
    r = k / n - u_mse
    rho = np.linalg.norm(r)
    var = (n * rho) ** 2 / m * (math.pi / 2 * (qv @ qv) - (qv @ (r / rho)) ** 2)
    assert est.var(ddof=1) == pytest.approx(var, rel=0.1)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_readme_inner_product_table(bits, golden):
    g = golden("readme_inner_product_table.json")
    row = g["bits"].index(bits)
    d = m = D_MODEL
    n_pairs = g["n_pairs"]
    cb = Codebook.build(bits - 1, d)  # b-bit budget = (b-1)-bit MSE stage + 1-bit QJL stage
    keys = synth.normal(21, 0, n_pairs * d).reshape(n_pairs, d)
    keys /= np.linalg.norm(keys, axis=1, keepdims=True)
    qs = synth.normal(21, 6, n_pairs * d).reshape(n_pairs, d)
    qs /= np.linalg.norm(qs, axis=1, keepdims=True)
    D = synth.signs(21, 2, d)
    S = synth.gaussian_matrix(1, 0, m, d)
    enc = quantize(keys, D, cb, norm_dtype=np.float64, S=S)
    est = np.array([
        qjl_scores(qs[i:i + 1], enc["codes"][i:i + 1], enc["norms"][i:i + 1], enc["qjl_bits"][i:i + 1],
                   enc["rho_exact"][i:i + 1], D, cb, S)[0, 0]
        for i in range(n_pairs)
    ])
    true = np.sum(qs * keys, axis=1)
    diff = est - true
    se = diff.std(ddof=1) / math.sqrt(n_pairs)
    assert abs(diff.mean()) < 4 * se
    assert abs(g["bias"][row]) < 4 * se  # the printed bias is consistent with zero at this sample size
    corr = np.corrcoef(est, true)[0, 1]
    assert corr == pytest.approx(g["correlation"][row], abs=0.02)
    # closed form for random unit pairs with m = d: 1/sqrt(1 + (pi/2) * MSE_(b-1))
    assert corr == pytest.approx(1.0 / math.sqrt(1.0 + math.pi / 2 * cb.distortion), abs=0.02)


def test_dequantize_and_score_paths_agree():
    d = m = D_MODEL
    cb = Codebook.build(2, d)
    D = synth.signs(5, 2, d)
    S = synth.gaussian_matrix(1, 0, m, d)
    keys = synth.normal(5, 0, 64 * d).reshape(64, d) * 3.0
    qs = synth.normal(5, 6, 8 * d).reshape(8, d)
    enc = quantize(keys, D, cb, S=S)
    scores = qjl_scores(qs, enc["codes"], enc["norms"], enc["qjl_bits"], enc["rho"], D, cb, S)
    rec = dequantize(enc["codes"], enc["norms"], D, cb, qjl_bits=enc["qjl_bits"], rho=enc["rho"], S=S)
    np.testing.assert_allclose(scores, qs @ rec.T, rtol=1e-12, atol=1e-12)
    # the estimator constant is sqrt(pi/2)
    assert QJL_CONST == pytest.approx(1.2533141373155, abs=1e-12)
