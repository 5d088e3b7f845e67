"""The fork's block format: 32-value records carrying their unit's norm (oracle side).

TEST INFRASTRUCTURE ONLY (see the package header).

[Fork] "GGML Types": a turbo3 block holds 32 values in 14 bytes (a 2-byte
norm and 12 packed bytes), a turbo4 block 18 bytes (2 + 16).  [Fork] "How it
works": the transform walks each row in 128-value chunks, every chunk is a
unit with its own L2 norm and FWHT, and the chunk's norm is stored in each of
its 32-value blocks, which is why splitting a 256-value head into two chunks
adds no bytes.

Readings (the pages give the byte counts, not the byte order):
  * a record is the fp16 norm of the block's unit (little-endian) followed by
    the block's packed codes, i.e. the same 4*bits bytes the separate-plane
    layout stores for that 32-coordinate group;
  * records follow the coordinate order of the rows (block g covers
    coordinates 32 (g mod head_dim/32) .. +31 of row g div (head_dim/32));
  * on decode each block is scaled by the norm its own record carries (a
    block is self-describing; for records written by the encoder all copies
    of a unit's norm are equal).
The format is defined for any unit length dt (a multiple of 32) and bit width;
the fork's own types are dt = 128 at 3 and 4 bits.
"""
from __future__ import annotations

import numpy as np

from .codebook import Codebook
from .quantizer import dequantize


def record_bytes(bits: int) -> int:
    return 2 + 4 * bits


def to_blocks(codes, norms, bits: int, dt: int) -> np.ndarray:
    """(codes [n_units, dt*bits/8] uint8, norms [n_units] fp16) -> records [n_units * dt/32, 2 + 4*bits] uint8."""
    codes = np.asarray(codes, dtype=np.uint8)
    norms = np.asarray(norms, dtype=np.float16)
    n = codes.shape[0]
    per = dt // 32
    out = np.zeros((n, per, record_bytes(bits)), dtype=np.uint8)
    norm_bytes = norms.astype("<f2").view(np.uint8).reshape(n, 2)
    groups = codes.reshape(n, per, 4 * bits)
    for b in range(per):
        out[:, b, 0:2] = norm_bytes
        out[:, b, 2:] = groups[:, b]
    return out.reshape(n * per, record_bytes(bits))


def from_blocks(records, bits: int, dt: int):
    """Inverse of to_blocks: (codes [n_units, dt*bits/8], block norms [n_units, dt/32] fp16)."""
    rec = np.asarray(records, dtype=np.uint8).reshape(-1, dt // 32, record_bytes(bits))
    n, per = rec.shape[0], dt // 32
    norms = np.ascontiguousarray(rec[:, :, 0:2]).view("<f2").reshape(n, per).astype(np.float16)
    codes = np.ascontiguousarray(rec[:, :, 2:]).reshape(n, per * 4 * bits)
    return codes, norms


def dequantize_blocks(records, signs, cb: Codebook, nc: bool = False) -> np.ndarray:
    """Decode records: the unit's reconstruction at unit norm, each block times its own stored norm.

    Returns [n_units, dt] float64 (reshape to rows as the caller's head_dim requires).
    """
    dt, bits = cb.dim, cb.bits
    codes, bn = from_blocks(records, bits, dt)
    unit = dequantize(codes, np.ones(codes.shape[0]), signs, cb, nc=nc)
    n = codes.shape[0]
    return (unit.reshape(n, dt // 32, 32) * bn.astype(np.float64)[:, :, None]).reshape(n, dt)
