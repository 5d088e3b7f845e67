"""Quantize / dequantize / QJL, the oracle side.  float64 throughout.

What one quantizer call computes, per unit (a d_t-long slice of a head vector:
the whole vector, or one 32-value block in the block-32 layout of [Scratch]
§7 and [Fork] "GGML Types"):

  1. n = ||x||_2, stored as fp16 (or fp32); u = x / n          [Scratch] §2 step 1
  2. y = H D u with D a fixed random +-1 diagonal and H the
     orthonormal Walsh-Hadamard matrix                          [Scratch] §2 step 2
  3. idx_i = bucketize(y_i, bounds): the number of cell edges
     strictly below y_i                                         [Scratch] §2 step 3
  4. store idx as a b-bit code, 32 coordinates per packed word  [Fork] "GGML Types"
  5. (QJL) r = u - D H c[idx]; keep rho = ||r|| and
     sign(S r), one bit per projection                          [Scratch] §2, [README]
Dequantize reverses it: c[idx] -> D H c (H is its own inverse) -> optional
QJL correction -> optional norm correction -> times the stored n
([Scratch] §2 and §6).

Readings taken where the pages are silent:
  * u is formed with the unrounded n; decode multiplies by the stored n.
  * a zero unit stores n = 0 and u = 0 (so idx = bucketize(0) = L/2 - 1).
  * stored code: sign-magnitude form of idx.  With h = L/2, idx >= h stores
    (0, idx - h) and idx < h stores (1, h - 1 - idx) as (sign bit, magnitude)
    = sign << (b-1) | magnitude.  A bijection of idx; the pages fix only the
    byte count (12 B per 32 values at 3 bits, 16 B at 4 bits).
  * packing: per 32-coordinate group a little-endian bit stream, coordinate j
    in bits [b*j, b*j + b); groups in coordinate order; codes and norms in
    separate planes.
  * QJL: S has i.i.d. N(0,1) entries (m x d_t), the estimator constant is
    sqrt(pi/2)/m ([README] estimator; [Scratch] divides by d with m = d),
    sign(0) = +1 ([Blog] Part 2 maps exact zeros to +1), bit 1 means +1,
    rho is stored as fp16.
  * norm correction with QJL is applied after the QJL term ([Scratch] §2
    order of the optional stages).
"""
from __future__ import annotations

import math

import numpy as np

from .codebook import Codebook

QJL_CONST = math.sqrt(math.pi / 2.0)


# ---------------------------------------------------------------------------
# rotation
# ---------------------------------------------------------------------------
def fwht(v) -> np.ndarray:
    """Orthonormal Walsh-Hadamard transform of the last axis ([Scratch] §2 fwht).

    For every index bit k in turn, each pair (i, i | 2^k) with bit k of i clear
    becomes (a + b, a - b); the result is divided by sqrt(d).  This is the
    Sylvester-ordered matrix H_ij = (-1)^popcount(i & j) / sqrt(d).
    """
    out = np.array(v, dtype=np.float64, copy=True)
    d = out.shape[-1]
    if d & (d - 1):
        raise ValueError("length must be a power of two")
    index = np.arange(d)
    bit = 1
    while bit < d:
        lo = index[(index & bit) == 0]
        hi = lo + bit
        a = out[..., lo].copy()
        b = out[..., hi].copy()
        out[..., lo] = a + b
        out[..., hi] = a - b
        bit <<= 1
    return out / math.sqrt(d)


def hadamard_matrix(d: int) -> np.ndarray:
    """Explicit H_ij = (-1)^popcount(i & j) / sqrt(d) (the definition the transform must equal)."""
    i = np.arange(d)[:, None]
    j = np.arange(d)[None, :]
    parity = np.vectorize(lambda v: bin(int(v)).count("1") & 1)(i & j)
    return np.where(parity == 1, -1.0, 1.0) / math.sqrt(d)


# ---------------------------------------------------------------------------
# codes and packing
# ---------------------------------------------------------------------------
def index_to_code(idx, bits: int) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.int64)
    h = 1 << (bits - 1)
    neg = idx < h
    mag = np.where(neg, h - 1 - idx, idx - h)
    return (neg.astype(np.int64) << (bits - 1)) | mag


def code_to_index(code, bits: int) -> np.ndarray:
    code = np.asarray(code, dtype=np.int64)
    h = 1 << (bits - 1)
    neg = (code >> (bits - 1)) & 1
    mag = code & (h - 1)
    return np.where(neg == 1, h - 1 - mag, h + mag)


def pack_codes(codes, bits: int) -> np.ndarray:
    """[N, dt] b-bit codes -> [N, dt*b/8] bytes (32-coordinate little-endian groups)."""
    codes = np.asarray(codes, dtype=np.int64)
    n, dt = codes.shape
    if dt % 32:
        raise ValueError("unit length must be a multiple of 32")
    groups = codes.reshape(n, dt // 32, 32)
    out = np.zeros((n, dt // 32, 4 * bits), dtype=np.uint8)
    for j in range(32):
        for k in range(bits):
            pos = bits * j + k
            bit = ((groups[:, :, j] >> k) & 1).astype(np.uint8)
            out[:, :, pos // 8] |= bit << np.uint8(pos % 8)
    return out.reshape(n, dt * bits // 8)


def unpack_codes(packed, bits: int, dt: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    groups = packed.reshape(n, dt // 32, 4 * bits).astype(np.int64)
    codes = np.zeros((n, dt // 32, 32), dtype=np.int64)
    for j in range(32):
        for k in range(bits):
            pos = bits * j + k
            codes[:, :, j] |= ((groups[:, :, pos // 8] >> (pos % 8)) & 1) << k
    return codes.reshape(n, dt)


def pack_sign_bits(positive) -> np.ndarray:
    """[N, m] booleans (True = +1) -> [N, m/8] bytes, projection i at bit i%8 of byte i//8."""
    positive = np.asarray(positive, dtype=bool)
    n, m = positive.shape
    out = np.zeros((n, m // 8), dtype=np.uint8)
    for i in range(m):
        out[:, i // 8] |= positive[:, i].astype(np.uint8) << np.uint8(i % 8)
    return out


def unpack_sign_bits(packed, m: int) -> np.ndarray:
    """Inverse of pack_sign_bits, as +-1.0 values."""
    packed = np.asarray(packed, dtype=np.uint8)
    bits = np.zeros((packed.shape[0], m), dtype=np.float64)
    for i in range(m):
        bits[:, i] = (packed[:, i // 8] >> (i % 8)) & 1
    return 2.0 * bits - 1.0


# ---------------------------------------------------------------------------
# quantize / dequantize
# ---------------------------------------------------------------------------
def _units(x, dt: int) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] % dt:
        raise ValueError("head_dim must be a multiple of the unit length")
    return x.reshape(-1, dt)


def encode_indices(x, signs, cb: Codebook):
    """Steps 1-3 for units of any power-of-two length: returns (n, u, y, idx), float64.

    n = ||x|| per unit, u = x/n (0 for a zero unit), y = H D u, idx = bucketize(y, bounds).
    """
    units = _units(x, cb.dim)
    n = np.sqrt(np.sum(units * units, axis=1))
    u = np.zeros_like(units)
    nz = n > 0
    u[nz] = units[nz] / n[nz, None]
    y = fwht(u * np.asarray(signs, dtype=np.float64))
    idx = np.searchsorted(cb.bounds, y, side="left")
    return n, u, y, idx


def quantize(x, signs, cb: Codebook, norm_dtype=np.float16, S=None) -> dict:
    """Encode ``x`` (any shape whose last axis is a multiple of cb.dim).

    Returns a dict with
      codes   [N_u, dt*b/8] uint8   packed codes
      norms   [N_u]         stored norms (norm_dtype)
      y_unit  [N_u, dt]     sqrt(dt) * y in float64 (diagnostic: distance to cell edges)
      and, when S is given (QJL):
      qjl_bits [N_u, m/8] uint8, rho [N_u] float16, z [N_u, m] float64 (diagnostic)
    """
    dt, bits = cb.dim, cb.bits
    d_signs = np.asarray(signs, dtype=np.float64)
    n, u, y, idx = encode_indices(x, d_signs, cb)
    out = {
        "codes": pack_codes(index_to_code(idx, bits), bits),
        "norms": n.astype(norm_dtype),
        "y_unit": y * math.sqrt(dt),
    }
    if S is not None:
        S = np.asarray(S, dtype=np.float64)
        u_mse = fwht(cb.levels[idx]) * d_signs
        r = u - u_mse
        z = r @ S.T
        out["z"] = z
        out["rho_exact"] = np.sqrt(np.sum(r * r, axis=1))
        out["rho"] = out["rho_exact"].astype(np.float16)
        out["qjl_bits"] = pack_sign_bits(z >= 0.0)
    return out


def dequantize(codes, norms, signs, cb: Codebook, nc: bool = False, qjl_bits=None, rho=None, S=None) -> np.ndarray:
    """Decode packed codes to [N_u, dt] float64 (multiply by the stored norms)."""
    dt, bits = cb.dim, cb.bits
    idx = code_to_index(unpack_codes(codes, bits, dt), bits)
    u = fwht(cb.levels[idx]) * np.asarray(signs, dtype=np.float64)
    if qjl_bits is not None:
        S = np.asarray(S, dtype=np.float64)
        m = S.shape[0]
        sigma = unpack_sign_bits(qjl_bits, m)
        rho64 = np.asarray(rho, dtype=np.float64)
        u = u + QJL_CONST * rho64[:, None] / m * (sigma @ S)
    if nc:
        length = np.sqrt(np.sum(u * u, axis=1))
        u = u / length[:, None]
    return np.asarray(norms, dtype=np.float64)[:, None] * u


def qjl_scores(q, codes, norms, qjl_bits, rho, signs, cb: Codebook, S) -> np.ndarray:
    """Inner-product estimates <q_i, k_j> from QJL-quantized keys ([README] combined estimator).

        score_ij = n_j * ( <q_i, u_mse_j> + rho_j * sqrt(pi/2)/m * <S q_i, sign(S r_j)> )

    with u_mse_j = D H c[idx_j] the MSE reconstruction of the unit key and
    n_j, rho_j the stored (rounded) norms.  Returns [n_q, n_k] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    m = S.shape[0]
    dt, bits = cb.dim, cb.bits
    idx = code_to_index(unpack_codes(codes, bits, dt), bits)
    u_mse = fwht(cb.levels[idx]) * np.asarray(signs, dtype=np.float64)
    sigma = unpack_sign_bits(qjl_bits, m)
    p = q @ S.T
    mse_term = q @ u_mse.T
    qjl_term = (p @ sigma.T) * (QJL_CONST / m) * np.asarray(rho, dtype=np.float64)[None, :]
    return np.asarray(norms, dtype=np.float64)[None, :] * (mse_term + qjl_term)
