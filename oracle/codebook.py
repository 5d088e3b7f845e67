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
    centroid moves by more than ``tol``.
    """
    if bits < 1:
        raise ValueError("bits >= 1")
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


@dataclass(frozen=True)
class Codebook:
    """Codebook for N(0, 1/d): ``levels``/``bounds`` are the N(0,1) values divided by sqrt(d)."""

    bits: int
    dim: int
    unit_levels: np.ndarray  # N(0,1) centroids, ascending
    unit_bounds: np.ndarray  # N(0,1) interior edges, ascending
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
