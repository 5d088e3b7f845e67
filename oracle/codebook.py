"""Lloyd-Max scalar quantizer for a Gaussian coordinate (oracle side).

[Scratch] §2 step 3: each rotated coordinate is quantized with a Lloyd-Max
codebook built once for N(0, 1/d) at the chosen bit width, with no
calibration data.  [README]: the codebook is found by numerical integration
and precomputed once per bit width.  [Scratch] §2 (the fake-quant step) looks
the centroid up as ``code[bucketize(y, bounds)]``, so ``bounds`` are the L-1
interior cell edges.

The N(0, 1/d) codebook is the N(0, 1) codebook scaled by 1/sqrt(d) (the
quantizer of a scaled source is the scaled quantizer), so everything here is
computed for N(0, 1) and scaled by the caller.

Lloyd's two optimality conditions, iterated to the fixed point:
  * each edge is the midpoint of its two neighbouring centroids;
  * each centroid is the conditional mean of its cell,
        c = (phi(a) - phi(b)) / (Phi(b) - Phi(a))  on the cell [a, b].
The Gaussian density is log-concave, so the fixed point is unique and does
not depend on the starting point.  The codebook is symmetric about zero; the
iteration works on the non-negative half and mirrors it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _pdf(x: float) -> float:
    if math.isinf(x):
        return 0.0
    return _INV_SQRT_2PI * math.exp(-0.5 * x * x)


def _upper_tail(x: float) -> float:
    """Q(x) = P(X > x) for X ~ N(0,1), accurate in the upper tail."""
    return 0.5 * math.erfc(x / math.sqrt(2.0))


def _cdf(x: float) -> float:
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def _inverse_cdf(p: float) -> float:
    from scipy.special import ndtri

    return float(ndtri(p))


def lloyd_max_gaussian(bits: int, tol: float = 1e-15, max_iter: int = 1_000_000):
    """Return (levels[L], edges[L-1]) of the Lloyd-Max quantizer for N(0,1), float64.

    Starts from the equal-probability partition and iterates until no
    centroid moves by more than ``tol``.  Above 4 bits the iteration needs
    millions of steps (its contraction factor tends to 1 as L grows), so
    there the same two conditions are solved as a root-finding problem
    instead (``_lloyd_max_gaussian_root``).
    """
    if bits < 1:
        raise ValueError("bits >= 1")
    if bits > 4:
        return _lloyd_max_gaussian_root(bits)
    return _lloyd_max_gaussian_iter(bits, tol, max_iter)


def _lloyd_max_gaussian_iter(bits: int, tol: float = 1e-15, max_iter: int = 1_000_000):
    """Lloyd's iteration of the two conditions (see lloyd_max_gaussian)."""
    L = 1 << bits
    half = L // 2
    # non-negative half: edges e_0 = 0 < e_1 < ... < e_{half-1} < e_half = +inf
    e = [0.0] + [_inverse_cdf(0.5 + 0.5 * k / half) for k in range(1, half)] + [math.inf]
    c = [0.0] * half
    for _ in range(max_iter):
        new_c = []
        for i in range(half):
            a, b = e[i], e[i + 1]
            mass = _upper_tail(a) - _upper_tail(b)
            new_c.append((_pdf(a) - _pdf(b)) / mass)
        moved = max(abs(x - y) for x, y in zip(new_c, c))
        c = new_c
        e = [0.0] + [0.5 * (c[i - 1] + c[i]) for i in range(1, half)] + [math.inf]
        if moved <= tol:
            break
    pos_levels = np.array(c, dtype=np.float64)
    levels = np.concatenate([-pos_levels[::-1], pos_levels])
    pos_edges = np.array(e[1:half], dtype=np.float64)
    edges = np.concatenate([-pos_edges[::-1], [0.0], pos_edges])
    return levels, edges


def _lloyd_max_gaussian_root(bits: int):
    """Lloyd-Max for N(0,1) at many levels: the non-negative half's centroids c solve
    c_i = E[X | e_i < X < e_{i+1}] with e_0 = 0, e_i = (c_{i-1} + c_i)/2, e_half = +inf
    (the same two conditions as the iteration), found with MINPACK's hybrid method
    (scipy.optimize.root) from the high-resolution starting point: edges at the
    quantiles of N(0, 3), the point density proportional to phi^(1/3) (Panter-Dite).

    The conditions are ill-conditioned along one smooth direction (the reason the
    plain iteration is slow), so a residual of ~1e-14 leaves the levels within about
    1e-9 of the exact fixed point.
    """
    from scipy.optimize import root
    from scipy.special import erfc, ndtri

    half = 1 << (bits - 1)

    def tail(x):
        return 0.5 * erfc(x / math.sqrt(2.0))

    def pdf(x):
        return np.where(np.isinf(x), 0.0, _INV_SQRT_2PI * np.exp(-0.5 * np.where(np.isinf(x), 0.0, x) ** 2))

    def cond_means(e):
        lo, hi = e[:-1], e[1:]
        return (pdf(lo) - pdf(hi)) / (tail(lo) - tail(hi))

    def edges_of(c):
        return np.concatenate([[0.0], 0.5 * (c[:-1] + c[1:]), [np.inf]])

    e0 = np.array([0.0] + [math.sqrt(3.0) * float(ndtri(0.5 + 0.5 * k / half)) for k in range(1, half)] + [np.inf])
    sol = root(lambda c: c - cond_means(edges_of(c)), cond_means(e0), method="hybr", options={"xtol": 1e-15})
    c = sol.x
    if not (np.all(np.diff(c) > 0) and np.max(np.abs(c - cond_means(edges_of(c)))) < 1e-12):
        raise RuntimeError(f"Lloyd-Max root solve did not converge at {bits} bits")
    levels = np.concatenate([-c[::-1], c])
    pos_edges = edges_of(c)[1:half]
    edges = np.concatenate([-pos_edges[::-1], [0.0], pos_edges])
    return levels, edges


def gaussian_distortion(levels, edges) -> float:
    """E[(X - Q(X))^2] for X ~ N(0,1) and the quantizer (levels, edges), closed form.

    On a cell [a, b] with reconstruction c,
        int (x - c)^2 phi = (Phi(b)-Phi(a)) (1 + c^2) - (b phi(b) - a phi(a)) - 2c (phi(a) - phi(b)),
    using int x^2 phi = Phi - x phi and int x phi = -phi.
    """
    levels = [float(v) for v in levels]
    bnd = [-math.inf] + [float(v) for v in edges] + [math.inf]
    total = 0.0
    for i, c in enumerate(levels):
        a, b = bnd[i], bnd[i + 1]
        if a >= 0.0:
            mass = _upper_tail(a) - _upper_tail(b)
        else:
            mass = _cdf(b) - _cdf(a)
        xa = 0.0 if math.isinf(a) else a * _pdf(a)
        xb = 0.0 if math.isinf(b) else b * _pdf(b)
        total += mass * (1.0 + c * c) - (xb - xa) - 2.0 * c * (_pdf(a) - _pdf(b))
    return total


# ---------------------------------------------------------------------------
# Beta-marginal codebook: the exact coordinate law of a rotated unit vector.
#
# [Fork] "How it works": the centroids are precomputed for the
# Beta((d-1)/2, (d-1)/2) law that a coordinate of H D u follows when u is a
# unit vector in d dimensions; [README] (stage 1) notes that this law is close to
# N(0, 1/d) for the usual head sizes.  Concretely, (T + 1)/2 ~ Beta(a, a) with
# a = (d-1)/2, i.e. T has density c_d (1 - t^2)^((d-3)/2) on [-1, 1] with
# c_d = 1 / B(1/2, a), and T^2 ~ Beta(1/2, a).  Its variance is 1/d, so the
# unit-variance variable is sqrt(d) T, the analogue of the N(0,1) scale above.
#
# The cell integrals come from the regularized incomplete beta function
# I_x(p, q) (scipy.special.betainc):
#   P(T > t)           = I_{1-t^2}(a, 1/2) / 2                     (t >= 0)
#   int_x^y t p(t) dt  = c_d ((1-x^2)^a - (1-y^2)^a) / (d - 1)
#   E[T^2; T <= x]     = (1 + I_{x^2}(3/2, a)) / (2d)               (x >= 0)
#                      = I_{1-x^2}(a, 3/2) / (2d)                   (x <  0)
# (the last from E[V; V <= v] = E[V] I_v(p+1, q) for V ~ Beta(p, q)).  The
# density is log-concave for d >= 3, so Lloyd's fixed point is again unique.
# ---------------------------------------------------------------------------
def _beta_norm(d: int) -> float:
    """c_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)), from Gamma(x+1) = x Gamma(x).

    The ratio of gammas is a product of (d-2)/2 factors; their logarithms are
    summed exactly (fsum), which keeps c_d to an ulp or two even at d = 4096,
    where a difference of log-gammas loses about 1e-12.
    """
    if d % 2 == 0:  # Gamma(m) / Gamma(m - 1/2) = prod_{j<m} j / (j - 1/2) / sqrt(pi)
        return math.exp(math.fsum(-math.log1p(-0.5 / j) for j in range(1, d // 2))) / math.pi
    # Gamma(m + 1/2) / Gamma(m) = sqrt(pi) / 2 * prod_{j<m} (j + 1/2) / j, m = (d-1)/2
    return math.exp(math.fsum(math.log1p(0.5 / j) for j in range(1, (d - 1) // 2))) / 2.0


def _beta_upper_tail(t: float, d: int) -> float:
    """P(T > t) for t >= 0."""
    from scipy.special import betainc

    if t >= 1.0:
        return 0.0
    return 0.5 * float(betainc((d - 1) / 2.0, 0.5, 1.0 - t * t))


def _beta_first_moment(x: float, y: float, d: int) -> float:
    """int_x^y t p(t) dt for -1 <= x <= y <= 1."""
    a = (d - 1) / 2.0
    return _beta_norm(d) * ((1.0 - x * x) ** a - (1.0 - y * y) ** a) / (d - 1)


def lloyd_max_beta(bits: int, dim: int, tol: float = 1e-15, max_iter: int = 1_000_000):
    """(levels[L], edges[L-1]) of the Lloyd-Max quantizer for sqrt(dim) T, float64.

    T is one coordinate of a uniformly random unit vector in ``dim``
    dimensions (the Beta((dim-1)/2, (dim-1)/2) law of [Fork] "How it works").
    The iteration runs on T itself over the non-negative half, starting from
    the equal-probability partition, and stops when no centroid moves by more
    than ``tol`` in the unit-variance scale; the result is returned in that
    scale, like ``lloyd_max_gaussian``.
    """
    from scipy.special import betaincinv

    if bits < 1:
        raise ValueError("bits >= 1")
    if dim < 3:
        raise ValueError("dim >= 3 (the marginal is log-concave from there on)")
    L = 1 << bits
    half = L // 2
    a = (dim - 1) / 2.0
    # edges with P(T > e_k) = (1 - k/half) / 2, i.e. 1 - e_k^2 = I^{-1}(a, 1/2; 1 - k/half)
    e = [0.0] + [math.sqrt(1.0 - float(betaincinv(a, 0.5, 1.0 - k / half))) for k in range(1, half)] + [1.0]
    c = [0.0] * half
    step_tol = tol / math.sqrt(dim)
    for _ in range(max_iter):
        new_c = []
        for i in range(half):
            lo, hi = e[i], e[i + 1]
            mass = _beta_upper_tail(lo, dim) - _beta_upper_tail(hi, dim)
            new_c.append(_beta_first_moment(lo, hi, dim) / mass)
        moved = max(abs(x - y) for x, y in zip(new_c, c))
        c = new_c
        e = [0.0] + [0.5 * (c[i - 1] + c[i]) for i in range(1, half)] + [1.0]
        if moved <= step_tol:
            break
    s = math.sqrt(dim)
    pos_levels = s * np.array(c, dtype=np.float64)
    levels = np.concatenate([-pos_levels[::-1], pos_levels])
    pos_edges = s * np.array(e[1:half], dtype=np.float64)
    edges = np.concatenate([-pos_edges[::-1], [0.0], pos_edges])
    return levels, edges


def beta_distortion(levels, edges, dim: int) -> float:
    """E[(X - Q(X))^2] for X = sqrt(dim) T (unit variance), T the Beta-law coordinate.

    ``levels``/``edges`` are in the unit-variance scale.  Per cell [x, y] of T
    with reconstruction c: E[T^2; cell] - 2 c int t p + c^2 P(cell), summed and
    multiplied by dim.  Edges at or beyond +-1 are clipped to the support.
    """
    from scipy.special import betainc

    d = dim
    a = (d - 1) / 2.0
    s = math.sqrt(d)

    def cdf(x):  # P(T <= x)
        if x <= -1.0:
            return 0.0
        if x >= 1.0:
            return 1.0
        tail = 0.5 * float(betainc(a, 0.5, 1.0 - x * x))
        return tail if x < 0 else 1.0 - tail

    def second(x):  # E[T^2; T <= x]
        if x <= -1.0:
            return 0.0
        if x >= 1.0:
            return 1.0 / d
        if x < 0:
            return float(betainc(a, 1.5, 1.0 - x * x)) / (2 * d)
        return (1.0 + float(betainc(1.5, a, x * x))) / (2 * d)

    lv = [float(v) / s for v in levels]
    bnd = [-1.0] + [min(1.0, max(-1.0, float(v) / s)) for v in edges] + [1.0]
    total = 0.0
    for i, c in enumerate(lv):
        x, y = bnd[i], bnd[i + 1]
        total += (second(y) - second(x)) - 2.0 * c * _beta_first_moment(x, y, d) + c * c * (cdf(y) - cdf(x))
    return d * total


@dataclass(frozen=True)
class Codebook:
    """Codebook for a coordinate of variance 1/d: ``levels``/``bounds`` are the
    unit-variance values (N(0,1), or sqrt(d) T for the Beta marginal) divided by sqrt(d)."""

    bits: int
    dim: int
    unit_levels: np.ndarray  # unit-variance centroids, ascending
    unit_bounds: np.ndarray  # unit-variance interior edges, ascending
    distortion: float  # relative distortion E[(X-Q(X))^2] / E[X^2] of the unit-variance quantizer

    @property
    def levels(self) -> np.ndarray:
        return self.unit_levels / math.sqrt(self.dim)

    @property
    def bounds(self) -> np.ndarray:
        return self.unit_bounds / math.sqrt(self.dim)

    @staticmethod
    def build(bits: int, dim: int) -> "Codebook":
        lv, ed = lloyd_max_gaussian(bits)
        return Codebook(bits, dim, lv, ed, gaussian_distortion(lv, ed))

    @staticmethod
    def build_beta(bits: int, dim: int) -> "Codebook":
        """The codebook for the exact Beta marginal ([Fork] "How it works");
        ``distortion`` is then the relative MSE under that marginal."""
        lv, ed = lloyd_max_beta(bits, dim)
        return Codebook(bits, dim, lv, ed, beta_distortion(lv, ed, dim))
