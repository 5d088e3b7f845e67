"""Comparison helpers for GPU-vs-oracle parity (test infrastructure).

Tolerances (the accuracy criteria this quantizer is held to, read as follows):
  * codes: bit-exact except coordinates whose oracle value sqrt(dt)*y lies
    within BAND = 1e-6 of a cell edge (0 included); there the GPU code must be
    one of the two cells next to that edge.  The in-band fraction is reported.
  * QJL sign bits: bit-exact except projections with |z| < 1e-6 * rho (z is
    N(0, rho^2) for S with N(0,1) entries, so this is the same 1e-6-of-sigma
    band as for the codes).
  * norms: fp16 within 1 ulp of the oracle's fp16(n); fp32 within 2 ulp.
  * dequantized values: |x~_gpu - x~_orc| / n <= 1e-5 on fp32 output (n the
    stored norm both sides use); fp16 output within 1 fp16 ulp of the oracle's
    value, or within that same 1e-5 * n where it is the larger (near zero).
  * the in-band count (assert_band_rate): at 1..4 bits the fraction of
    coordinates inside the band must stay under 1e-5.  That is a rate: on the
    large full-size samples the count itself must be below 1e-5 of the
    coordinates; a small sample passes when its count is within the one-sided
    99.9% Poisson quantile of that rate.  At 8 bits the 255 edges alone put
    about 2 * BAND * sum_k phi(t_k) = 1.03e-4 of N(0,1) coordinates inside the
    band, so the 1e-5 bound cannot hold for any encoder; there the in-band
    fraction must stay under twice that geometric rate, and the codes that
    actually differ from the oracle's under 1e-5 of the coordinates.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import code_to_index, unpack_codes, unpack_sign_bits

BAND = 1e-6
IN_BAND_RATE = 1e-5      # bound on the in-band fraction at 1..4 bits
MISMATCH_RATE_8 = 1e-5   # bound on the fraction of differing codes at 8 bits


def _normal_pdf(x: np.ndarray) -> np.ndarray:
    return np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def band_rate_bound(cb) -> float:
    """Bound on the fraction of coordinates inside the edge band for codebook cb (see the header)."""
    if cb.bits <= 4:
        return IN_BAND_RATE
    return 2.0 * 2.0 * BAND * float(_normal_pdf(np.asarray(cb.unit_bounds, dtype=np.float64)).sum())


def poisson_upper(lam: float, p: float = 1e-3) -> int:
    """Smallest k with P(Poisson(lam) > k) < p."""
    k, term = 0, math.exp(-lam)
    cdf = term
    while 1.0 - cdf >= p:
        k += 1
        term *= lam / k
        cdf += term
    return k


def assert_rate(count: int, n: int, rate: float, literal: bool, what: str) -> None:
    """count out of n against a rate bound: literal, count < rate * n (samples whose expected count is
    tens); otherwise count within the one-sided 99.9% Poisson quantile of rate * n."""
    limit = rate * n if literal else poisson_upper(rate * n)
    ok = count < limit if literal else count <= limit
    assert ok, f"{count} of {n} {what} ({count / max(n, 1):.3g}); bound {rate:.3g} of them ({limit:.4g})"


def assert_band_rate(stats: dict, cb, literal: bool = False) -> None:
    """In-band count of a check_codes result against band_rate_bound; at 8 bits the codes that differ
    from the oracle's must also stay under MISMATCH_RATE_8."""
    n = stats["coords"]
    assert_rate(stats["in_band"], n, band_rate_bound(cb), literal, "coordinates lie within the edge band")
    if cb.bits > 4:
        assert_rate(stats["in_band_mismatch"], n, MISMATCH_RATE_8, literal, "codes differ from the oracle's")


def assert_sign_band_rate(stats: dict, literal: bool = False) -> None:
    """In-band count of a check_sign_bits result (|z| < BAND * rho) against the 1e-5 bound."""
    assert_rate(stats["in_band"], stats["bits"], IN_BAND_RATE, literal, "projections lie within the zero band")


def edge_distance(y_unit: np.ndarray, cb) -> np.ndarray:
    """Distance of each value to its nearest cell edge (the edges are sorted, so the nearest is one of
    the two around the value's insertion point)."""
    edges = np.asarray(cb.unit_bounds, dtype=np.float64)
    y = np.asarray(y_unit, dtype=np.float64)
    i = np.searchsorted(edges, y)
    lo = edges[np.clip(i - 1, 0, len(edges) - 1)]
    hi = edges[np.clip(i, 0, len(edges) - 1)]
    return np.minimum(np.abs(y - lo), np.abs(y - hi))


def check_codes(gpu_codes: np.ndarray, orc: dict, cb, bits: int, dt: int) -> dict:
    g = unpack_codes(gpu_codes.reshape(-1, dt * bits // 8), bits, dt)
    o = unpack_codes(orc["codes"], bits, dt)
    dist = edge_distance(orc["y_unit"], cb)
    in_band = dist < BAND
    mism = g != o
    out_of_band = mism & ~in_band
    gi, oi = code_to_index(g, bits), code_to_index(o, bits)
    assert not out_of_band.any(), (
        f"{int(out_of_band.sum())} code mismatches outside the band; first at {np.argwhere(out_of_band)[:5].tolist()}, "
        f"gpu idx {gi[out_of_band][:5].tolist()} oracle idx {oi[out_of_band][:5].tolist()} "
        f"dist {dist[out_of_band][:5].tolist()}")
    assert np.all(np.abs(gi[mism] - oi[mism]) <= 1), "in-band mismatch is not a neighbouring cell"
    return {"coords": int(g.size), "in_band": int(in_band.sum()), "in_band_mismatch": int(mism.sum())}


def f16_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|a - b| in units of binary16 ulps (monotone integer mapping of the bit patterns)."""
    def key(x):
        u = np.asarray(x, dtype=np.float16).view(np.uint16).astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(key(a) - key(b))


def f32_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def key(x):
        u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.int64)
        return np.where(u & 0x80000000, -(u & 0x7FFFFFFF), u)
    return np.abs(key(a) - key(b))


def check_norms(gpu_norms: np.ndarray, orc_norms: np.ndarray) -> dict:
    if orc_norms.dtype == np.float16:
        d = f16_ulp_diff(gpu_norms, orc_norms)
        assert d.max(initial=0) <= 1, f"fp16 norms differ by {d.max()} ulp"
    else:
        d = f32_ulp_diff(gpu_norms, orc_norms)
        assert d.max(initial=0) <= 2, f"fp32 norms differ by {d.max()} ulp"
    return {"norms": int(d.size), "norm_ulp_mismatch": int((d > 0).sum())}


def check_decoded_f32(gpu: np.ndarray, orc: np.ndarray, norms: np.ndarray, dt: int, tol: float = 1e-5) -> float:
    g = gpu.reshape(-1, dt).astype(np.float64)
    o = orc.reshape(-1, dt)
    n = np.asarray(norms, dtype=np.float64).reshape(-1)
    safe = np.where(n > 0, n, 1.0)
    err = np.abs(g - o) / safe[:, None]
    err[n == 0] = np.abs(g[n == 0] - o[n == 0])
    worst = float(err.max(initial=0.0))
    assert worst <= tol, f"decoded values differ by {worst:.3g} (relative to the unit norm)"
    return worst


def check_decoded_f16(gpu: np.ndarray, orc: np.ndarray, norms: np.ndarray, dt: int, tol: float = 1e-5) -> int:
    """fp16 output: within one fp16 ulp of the oracle value, or within the fp32 decode tolerance
    (tol * n) where that is larger (near zero the fp16 ulp is far below the fp32 rounding)."""
    g = gpu.reshape(-1, dt).astype(np.float64)
    o = orc.reshape(-1, dt)
    n = np.asarray(norms, dtype=np.float64).reshape(-1, 1)
    ulp = np.spacing(np.abs(o).astype(np.float16)).astype(np.float64)
    err = np.abs(g - o)
    ok = err <= np.maximum(ulp, tol * n)
    assert ok.all(), f"fp16 outputs off by {err[~ok][:5]} (ulp {ulp[~ok][:5]}, n {np.broadcast_to(n, err.shape)[~ok][:5]})"
    d = f16_ulp_diff(gpu.reshape(-1), orc.reshape(-1).astype(np.float16))
    return int((d > 0).sum())


def check_sign_bits(gpu_bits: np.ndarray, orc: dict, m: int) -> dict:
    g = unpack_sign_bits(gpu_bits.reshape(-1, m // 8), m)
    o = unpack_sign_bits(orc["qjl_bits"], m)
    z = orc["z"]
    rho = orc["rho_exact"][:, None]
    in_band = np.abs(z) < BAND * rho
    mism = g != o
    bad = mism & ~in_band
    assert not bad.any(), f"{int(bad.sum())} sign-bit mismatches outside the band; |z|/rho = {(np.abs(z)/rho)[bad][:5]}"
    return {"bits": int(g.size), "in_band": int(in_band.sum()), "in_band_mismatch": int(mism.sum())}
