"""The split-precision projection of the head_dim-128 QJL encode, simulated on the CPU.

The GPU computes z = S~ e with e (scaled by 2^10) and S~ each split into fp16 pieces x = hi + lo
(hi = fp16(x), lo = fp16(x - hi)) and z = hi.hi + hi.lo + lo.hi accumulated in fp32.  This test runs
the same arithmetic in numpy (fp16 pieces, fp32 products and sums) against the exact projection of the
oracle's residuals and requires what the sign-bit parity rests on: the error stays within a few 1e-6
of rho, no larger than that of plain fp32 products, and no sign differs outside |z| < 1e-6 rho.
"""
import math

import numpy as np

from oracle import Codebook
from oracle.quantizer import fwht, hadamard_matrix
from synth.workloads import qjl_keys

BAND = 1e-6


def _split(a, scale):
    a = a.astype(np.float32) * np.float32(scale)
    hi = a.astype(np.float16)
    lo = (a - hi.astype(np.float32)).astype(np.float16)
    return hi.astype(np.float32), lo.astype(np.float32)


def test_split_fp16_projection_matches_fp32_error():
    w = qjl_keys(n_keys=8192, n_queries=32)
    x = w["keys"].astype(np.float64)
    signs = np.asarray(w["signs"], dtype=np.float64)
    S = np.asarray(w["S"], dtype=np.float64)
    dt = x.shape[1]
    cb = Codebook.build(2, dt)
    u = x / np.linalg.norm(x, axis=1)[:, None]
    y = fwht(u * signs)
    e_u = y - cb.levels[np.searchsorted(cb.bounds, y, side="left")]
    St = S @ np.diag(signs) @ hadamard_matrix(dt)  # S~ = S D H
    z = e_u @ St.T
    rho = np.linalg.norm(e_u, axis=1)[:, None]
    sc = math.sqrt(dt)
    e32 = (e_u * sc).astype(np.float32)  # the kernel's N(0,1) units
    S32 = St.astype(np.float32)
    z32 = (e32 @ S32.T).astype(np.float64) / sc
    eh, el = _split(e32, 1024.0)
    sh, sl = _split(S32, 1.0)
    z3 = ((eh @ sh.T).astype(np.float32) + (eh @ sl.T).astype(np.float32) + (el @ sh.T).astype(np.float32))
    z3 = z3.astype(np.float64) / 1024.0 / sc
    err32 = np.abs(z32 - z) / rho
    err3 = np.abs(z3 - z) / rho
    assert float(np.median(err3)) < 2.0 * float(np.median(err32)) + 1e-8
    assert float(err3.max()) < 1e-5
    band = np.abs(z) < BAND * rho
    assert not (((z3 >= 0) != (z >= 0)) & ~band).any()
