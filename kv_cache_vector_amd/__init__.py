"""MI355X-native TurboQuant KV-cache quantizer: Python binding of libtq.

Argument marshalling only.  Every step of the quantizer runs in the HIP
kernels of ``libtq.so`` (built from ``csrc/`` by ``kv_cache_vector_amd.build``);
the functions here have the names of the C ABI in ``include/tq.h`` and pass
device pointers (torch tensors' ``data_ptr()``) and the current HIP stream
through.  There is no fallback: if the library is missing, importing the
binding's functions raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_WORKSPACE, TQ_ERR_HIP = range(5)
TQ_F16, TQ_F32 = 0, 1
TQ_NORM_CORRECT, TQ_QJL, TQ_BLOCKS = 1, 2, 4
TQ_OP_QJL_SCORES, TQ_OP_DECODE_ATTN, TQ_OP_MULTI_ATTN = 1, 2, 3

EXPORTED = ("tq_codebook_init", "tq_codebook_init_beta", "tq_qjl_params_size", "tq_qjl_prepare", "tq_quantize", "tq_dequantize",
            "tq_qjl_scores", "tq_decode_attn", "tq_decode_attn_noalloc", "tq_multi_attn", "tq_workspace_size",
            "tq_status_str",
            "tq_last_error")


class TqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class tq_codebook(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int), ("dim", ctypes.c_int), ("unit_centroids", ctypes.c_double * 256),
                ("unit_bounds", ctypes.c_double * 255), ("centroids", ctypes.c_float * 256),
                ("bounds", ctypes.c_float * 255), ("distortion", ctypes.c_double)]


class tq_config(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int), ("dt", ctypes.c_int), ("bits", ctypes.c_int), ("flags", ctypes.c_uint),
                ("qjl_m", ctypes.c_int), ("x_dtype", ctypes.c_int), ("norm_dtype", ctypes.c_int),
                ("cb", ctypes.POINTER(tq_codebook)), ("signs", ctypes.POINTER(ctypes.c_float)),
                ("qjl_params", ctypes.c_void_p)]


_lib = None


def lib():
    """The loaded libtq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m kv_cache_vector_amd.build` "
                          "(or __graft_entry__.build()); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, c_int, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    cfgp = ctypes.POINTER(tq_config)
    L.tq_codebook_init.argtypes = [ctypes.POINTER(tq_codebook), c_int, c_int]
    L.tq_codebook_init_beta.argtypes = [ctypes.POINTER(tq_codebook), c_int, c_int]
    L.tq_qjl_params_size.argtypes = [c_int, c_int]
    L.tq_qjl_params_size.restype = sz
    L.tq_qjl_prepare.argtypes = [cfgp, vp, vp, sz, vp]
    L.tq_quantize.argtypes = [cfgp, vp, i64, i64, vp, vp, vp, vp, vp]
    L.tq_dequantize.argtypes = [cfgp, vp, vp, vp, vp, i64, vp, c_int, i64, vp]
    L.tq_qjl_scores.argtypes = [cfgp, vp, c_int, i64, i64, vp, vp, vp, vp, i64, vp, i64, vp, sz, vp]
    L.tq_decode_attn.argtypes = [cfgp, cfgp, vp, c_int, c_int, c_int, i64, vp, vp, vp, vp, ctypes.c_float, vp, vp, sz,
                                 vp]
    L.tq_decode_attn_noalloc.argtypes = [cfgp, cfgp, vp, c_int, c_int, c_int, i64, vp, vp, vp, vp, ctypes.c_float,
                                         vp, vp]
    L.tq_multi_attn.argtypes = [cfgp, cfgp, vp, c_int, i64, c_int, c_int, i64, vp, vp, vp, vp, c_int, ctypes.c_float,
                                vp, vp, sz, vp]
    L.tq_workspace_size.argtypes = [c_int, cfgp, i64, i64, i64]
    L.tq_workspace_size.restype = sz
    L.tq_status_str.argtypes = [c_int]
    L.tq_status_str.restype = ctypes.c_char_p
    L.tq_last_error.restype = ctypes.c_char_p
    for name in ("tq_codebook_init", "tq_codebook_init_beta", "tq_qjl_prepare", "tq_quantize", "tq_dequantize", "tq_qjl_scores",
                 "tq_decode_attn", "tq_decode_attn_noalloc", "tq_multi_attn"):
        getattr(L, name).restype = c_int
    _lib = L
    return L


def _check(status: int):
    if status != TQ_OK:
        raise TqError(status, lib().tq_last_error().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------------------
# configuration objects (host data)
# ---------------------------------------------------------------------------
def tq_codebook_init(bits: int, dim: int) -> tq_codebook:
    cb = tq_codebook()
    _check(lib().tq_codebook_init(ctypes.byref(cb), bits, dim))
    return cb


def tq_codebook_init_beta(bits: int, dim: int) -> tq_codebook:
    cb = tq_codebook()
    _check(lib().tq_codebook_init_beta(ctypes.byref(cb), bits, dim))
    return cb


CODEBOOKS = {"gaussian": tq_codebook_init, "beta": tq_codebook_init_beta}


class Quantizer:
    """A ``tq_config`` plus the host data it points to (kept alive here)."""

    def __init__(self, head_dim: int, dt: int, bits: int, signs, flags: int = 0, qjl_m: int = 0,
                 x_dtype: int = TQ_F16, norm_dtype: int = TQ_F16, codebook: str = "gaussian"):
        self.codebook = CODEBOOKS[codebook](bits, dt)
        self.signs = np.ascontiguousarray(np.asarray(signs, dtype=np.float32))
        self.params = None
        self.cfg = tq_config(head_dim, dt, bits, flags, qjl_m, x_dtype, norm_dtype, ctypes.pointer(self.codebook),
                             self.signs.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), None)

    @property
    def units_per_row(self) -> int:
        return self.cfg.head_dim // self.cfg.dt

    def code_bytes(self) -> int:
        """Bytes of packed codes per unit."""
        return self.cfg.dt * self.cfg.bits // 8

    def record_bytes(self) -> int:
        """Bytes of one 32-value record of the TQ_BLOCKS format (fp16 norm + codes)."""
        return 2 + 4 * self.cfg.bits

    def attach_params(self, params_tensor):
        self.params = params_tensor
        self.cfg.qjl_params = _ptr(params_tensor)


def tq_qjl_params_size(m: int, dt: int) -> int:
    return lib().tq_qjl_params_size(m, dt)


def tq_qjl_prepare(qz: Quantizer, S_host: np.ndarray, params, stream=None):
    S = np.ascontiguousarray(np.asarray(S_host, dtype=np.float32))
    _check(lib().tq_qjl_prepare(ctypes.byref(qz.cfg), S.ctypes.data, _ptr(params), params.numel() * params.element_size(),
                                _stream(stream)))
    qz.attach_params(params)


def tq_quantize(qz: Quantizer, x, n_rows: int, ld_x: int, codes, norms, qjl_bits=None, qjl_rnorm=None, stream=None):
    _check(lib().tq_quantize(ctypes.byref(qz.cfg), _ptr(x), n_rows, ld_x, _ptr(codes), _ptr(norms), _ptr(qjl_bits),
                             _ptr(qjl_rnorm), _stream(stream)))


def tq_dequantize(qz: Quantizer, codes, norms, qjl_bits, qjl_rnorm, n_rows: int, y, y_dtype: int, ld_y: int,
                  stream=None):
    _check(lib().tq_dequantize(ctypes.byref(qz.cfg), _ptr(codes), _ptr(norms), _ptr(qjl_bits), _ptr(qjl_rnorm),
                               n_rows, _ptr(y), y_dtype, ld_y, _stream(stream)))


def tq_workspace_size(op: int, qz: Quantizer, a: int, b: int = 0, c: int = 0) -> int:
    return lib().tq_workspace_size(op, ctypes.byref(qz.cfg), a, b, c)


def tq_qjl_scores(qz: Quantizer, q, q_dtype: int, n_q: int, ld_q: int, codes, norms, qjl_bits, qjl_rnorm, n_k: int,
                  scores, ld_s: int, ws=None, ws_bytes: int = 0, stream=None):
    _check(lib().tq_qjl_scores(ctypes.byref(qz.cfg), _ptr(q), q_dtype, n_q, ld_q, _ptr(codes), _ptr(norms),
                               _ptr(qjl_bits), _ptr(qjl_rnorm), n_k, _ptr(scores), ld_s, _ptr(ws), ws_bytes,
                               _stream(stream)))


def tq_decode_attn(kq: Quantizer, vq: Quantizer, q, q_dtype: int, n_q_heads: int, n_kv_heads: int, n_tokens: int,
                   k_codes, k_norms, v_codes, v_norms, scale: float, out, ws=None, ws_bytes: int = 0, stream=None):
    _check(lib().tq_decode_attn(ctypes.byref(kq.cfg), ctypes.byref(vq.cfg), _ptr(q), q_dtype, n_q_heads, n_kv_heads,
                                n_tokens, _ptr(k_codes), _ptr(k_norms), _ptr(v_codes), _ptr(v_norms), scale,
                                _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))


def tq_decode_attn_noalloc(kq: Quantizer, vq: Quantizer, q, q_dtype: int, n_q_heads: int, n_kv_heads: int,
                           n_tokens: int, k_codes, k_norms, v_codes, v_norms, scale: float, out, stream=None):
    _check(lib().tq_decode_attn_noalloc(ctypes.byref(kq.cfg), ctypes.byref(vq.cfg), _ptr(q), q_dtype, n_q_heads,
                                        n_kv_heads, n_tokens, _ptr(k_codes), _ptr(k_norms), _ptr(v_codes),
                                        _ptr(v_norms), scale, _ptr(out), _stream(stream)))


def tq_multi_attn(kq: Quantizer, vq: Quantizer, q, q_dtype: int, n_q: int, n_q_heads: int, n_kv_heads: int,
                  n_tokens: int, k_codes, k_norms, v_codes, v_norms, causal: bool, scale: float, out, ws=None,
                  ws_bytes: int = 0, stream=None):
    _check(lib().tq_multi_attn(ctypes.byref(kq.cfg), ctypes.byref(vq.cfg), _ptr(q), q_dtype, n_q, n_q_heads,
                               n_kv_heads, n_tokens, _ptr(k_codes), _ptr(k_norms), _ptr(v_codes), _ptr(v_norms),
                               1 if causal else 0, scale, _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))
