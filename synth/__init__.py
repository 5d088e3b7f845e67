"""Seeded synthetic inputs, shared by the HIP path's tests and benchmark and by
the CPU oracle.

This module holds no quantizer arithmetic.  It draws counter-based uniforms
(splitmix64's output function on a counter) and normals (Box-Muller), shapes
them like a KV cache (per-channel log-normal scales, outlier channels), and
rounds them to binary16/binary32.  The random numbers the quantizer itself
needs (the random signs D and the Gaussian projection S) are drawn here too
and handed to both sides as inputs.

The generator is a small C library (``synth.c``) loaded with ctypes; build it
with :func:`build` (``__graft_entry__.build()`` does).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

# stream numbers (one per kind of draw)
STREAM_K = 0
STREAM_V = 1
STREAM_SIGNS_K = 2
STREAM_SIGNS_V = 3
STREAM_CHANNEL_SCALE = 4  # used inside synth.c
STREAM_OUTLIER = 5  # used inside synth.c
STREAM_QUERY = 6


def build() -> str:
    """Compile ``libsynth.so`` next to this file (always recompiles)."""
    src = os.path.join(_HERE, "synth.c")
    tmp = _SO + ".tmp"
    subprocess.run(
        ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp,
         "-lm", "-lpthread"],
        check=True,
    )
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    u64, i64, c_int, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    vp = ctypes.c_void_p
    lib.synth_uniform.argtypes = [u64, u64, u64, u64, vp]
    lib.synth_normal.argtypes = [u64, u64, u64, u64, vp]
    lib.synth_f64_to_f16.argtypes = [vp, u64, vp]
    lib.synth_kv.argtypes = [u64, c_int, c_int, c_int, i64, c_int, dbl, c_int, dbl, c_int, vp, vp, c_int]
    lib.synth_kv.restype = c_int
    lib.synth_normal_rounded.argtypes = [u64, u64, u64, vp, vp, c_int]
    _lib = lib
    return lib


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def uniform(seed: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform(seed, stream, start, n, out.ctypes.data)
    return out


def normal(seed: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_normal(seed, stream, start, n, out.ctypes.data)
    return out


def to_f16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to binary16 (round-to-nearest-even)."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().synth_f64_to_f16(a.ctypes.data, a.size, out.ctypes.data)
    return out.view(np.float16)


def normal_f16(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    _load().synth_normal_rounded(seed, stream, n, out.ctypes.data, None, _threads())
    return out.view(np.float16)


def normal_f32(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal_rounded(seed, stream, n, None, out.ctypes.data, _threads())
    return out


def kv_tensor(seed: int, layers: int, heads: int, kv: int, tokens: int, head_dim: int, sigma: float = 1.0,
              n_outliers: int = 2, outlier_mult: float = 10.0, data_stream: int | None = None,
              f16: bool = True, out: np.ndarray | None = None) -> np.ndarray:
    """One half (kv=0: K, kv=1: V) of a KV cache, shape [layers, heads, tokens, head_dim].

    Entries are N(0,1) times a per-channel log-normal scale exp(sigma * N(0,1)),
    with ``n_outliers`` channels per (layer, head, K|V) multiplied by
    ``outlier_mult``.  Returned as float16 (``f16``) or float64.
    """
    if data_stream is None:
        data_stream = STREAM_K if kv == 0 else STREAM_V
    shape = (layers, heads, tokens, head_dim)
    if out is None:
        out = np.empty(shape, dtype=np.float16 if f16 else np.float64)
    assert out.shape == shape and out.flags.c_contiguous
    p16 = out.ctypes.data if f16 else None
    p64 = None if f16 else out.ctypes.data
    rc = _load().synth_kv(seed, layers, heads, kv, tokens, head_dim, sigma, n_outliers, outlier_mult, data_stream,
                          p16, p64, _threads())
    if rc != 0:
        raise ValueError("synth_kv: bad arguments")
    return out


def signs(seed: int, stream: int, d: int) -> np.ndarray:
    """Random +-1 vector of length d (float32): +1 where U < 1/2."""
    u = uniform(seed, stream, d)
    return np.where(u < 0.5, 1.0, -1.0).astype(np.float32)


def gaussian_matrix(seed: int, stream: int, m: int, d: int) -> np.ndarray:
    """m x d matrix of N(0,1) draws rounded to float32 (row-major)."""
    return normal(seed, stream, m * d).astype(np.float32).reshape(m, d)
