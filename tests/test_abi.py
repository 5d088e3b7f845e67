"""C ABI checks that need no GPU: the library loads and exports every symbol
include/tq.h declares, the host codebook solver agrees with the oracle, and
argument validation rejects bad calls before anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_vector_amd as tq
from oracle import Codebook

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FAKE = 0x100000  # an aligned, never-dereferenced address: every call below fails validation first


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"^\s*(?:tq_status|size_t|const char\*)\s+(tq_\w+)\s*\(", text, re.M))
    return names


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"tq_codebook_init", "tq_quantize", "tq_dequantize", "tq_qjl_scores", "tq_decode_attn"} <= names
    lib = ctypes.CDLL(tq.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert names == set(tq.EXPORTED)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("dim", [32, 64, 128, 256])
def test_host_codebook_matches_oracle(bits, dim):
    """Up to 4 bits both sides iterate Lloyd's conditions; above, the host runs Newton's method and
    the oracle MINPACK's hybrid root finder on them (agreement limited by the conditioning)."""
    cb = tq.tq_codebook_init(bits, dim)
    orc = Codebook.build(bits, dim)
    L = 1 << bits
    tol = 1e-12 if bits <= 4 else 1e-10
    np.testing.assert_allclose(np.array(cb.unit_centroids[:L]), orc.unit_levels, atol=tol, rtol=0)
    np.testing.assert_allclose(np.array(cb.unit_bounds[:L - 1]), orc.unit_bounds, atol=tol, rtol=0)
    np.testing.assert_array_equal(np.array(cb.centroids[:L], dtype=np.float32), orc.levels.astype(np.float32))
    np.testing.assert_array_equal(np.array(cb.bounds[:L - 1], dtype=np.float32), orc.bounds.astype(np.float32))
    assert cb.distortion == pytest.approx(orc.distortion, abs=1e-12)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("dim", [4, 32, 64, 128, 256, 4096])
def test_host_beta_codebook_matches_oracle(bits, dim):
    """The host solver (theta-substitution quadrature) against the oracle (incomplete beta function)."""
    cb = tq.tq_codebook_init_beta(bits, dim)
    orc = Codebook.build_beta(bits, dim)
    L = 1 << bits
    tol = 1e-11 if dim > 256 else 1e-12  # Lloyd's contraction slows at large d and 4 bits
    np.testing.assert_allclose(np.array(cb.unit_centroids[:L]), orc.unit_levels, atol=tol, rtol=0)
    np.testing.assert_allclose(np.array(cb.unit_bounds[:L - 1]), orc.unit_bounds, atol=tol, rtol=0)
    np.testing.assert_array_equal(np.array(cb.centroids[:L], dtype=np.float32), orc.levels.astype(np.float32))
    np.testing.assert_array_equal(np.array(cb.bounds[:L - 1], dtype=np.float32), orc.bounds.astype(np.float32))
    assert cb.distortion == pytest.approx(orc.distortion, abs=1e-12)
    assert (cb.bits, cb.dim) == (bits, dim)


def test_beta_codebook_init_rejects_bad_arguments():
    cb = tq.tq_codebook()
    L = tq.lib()
    assert L.tq_codebook_init_beta(ctypes.byref(cb), 0, 32) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_codebook_init_beta(ctypes.byref(cb), 5, 32) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_codebook_init_beta(ctypes.byref(cb), 3, 2) == tq.TQ_ERR_INVALID_ARG  # below 4: not log-concave
    assert L.tq_codebook_init_beta(ctypes.byref(cb), 3, 48) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_codebook_init_beta(ctypes.byref(cb), 3, 8192) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_codebook_init_beta(None, 3, 32) == tq.TQ_ERR_INVALID_ARG


def test_codebook_init_rejects_bad_arguments():
    cb = tq.tq_codebook()
    L = tq.lib()
    assert L.tq_codebook_init(ctypes.byref(cb), 0, 32) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_codebook_init(ctypes.byref(cb), 9, 32) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_codebook_init(ctypes.byref(cb), 3, 48) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_codebook_init(None, 3, 32) == tq.TQ_ERR_INVALID_ARG


def _q(**kw):
    args = dict(head_dim=128, dt=32, bits=3, signs=np.ones(kw.get("dt", 32)))
    args.update(kw)
    return tq.Quantizer(**args)


def _quantize(qz, x=FAKE, n_rows=4, ld=None, codes=FAKE, norms=FAKE, bits=None, rnorm=None):
    ld = qz.cfg.head_dim if ld is None else ld
    return tq.lib().tq_quantize(ctypes.byref(qz.cfg), x, n_rows, ld, codes, norms, bits, rnorm, None)


def test_quantize_validation():
    E, U, OK = tq.TQ_ERR_INVALID_ARG, tq.TQ_ERR_UNSUPPORTED, tq.TQ_OK
    qz = _q()
    assert _quantize(qz, n_rows=0) == OK  # empty input is a no-op
    assert _quantize(qz, n_rows=-1) == E
    assert _quantize(qz, x=None) == E
    assert _quantize(qz, x=FAKE + 2) == E  # misaligned rows
    assert _quantize(qz, ld=100) == E  # stride below head_dim
    assert _quantize(qz, ld=132) == E  # stride not a multiple of 16 bytes
    assert _quantize(qz, codes=FAKE + 2) == E
    assert _quantize(qz, norms=None) == E
    assert _quantize(qz, n_rows=1 << 60) == E  # size overflow
    bad = _q()
    bad.cfg.bits = 5
    assert _quantize(bad) == U
    bad = _q()
    bad.cfg.dt = 48
    assert _quantize(bad) == E
    assert _quantize(_q(head_dim=96, dt=64, signs=np.ones(64))) == E
    s = np.ones(32)
    s[3] = 0.5
    assert _quantize(_q(signs=s)) == E
    bad = _q()
    bad.cfg.flags = 8
    assert _quantize(bad) == E
    bad = _q()
    bad.cfg.bits = 4  # codebook built for 3 bits
    assert _quantize(bad) == E
    assert _quantize(_q(flags=tq.TQ_QJL, qjl_m=128)) == U  # QJL needs dt == head_dim
    qj = _q(head_dim=128, dt=128, bits=2, signs=np.ones(128), flags=tq.TQ_QJL, qjl_m=128)
    assert _quantize(qj, bits=FAKE, rnorm=FAKE) == E  # no prepared parameters
    qj.cfg.qjl_params = FAKE
    assert _quantize(qj) == E  # no sign-bit / residual-norm outputs
    qj.cfg.qjl_m = 100
    assert _quantize(qj, bits=FAKE, rnorm=FAKE) == E
    assert "qjl_m" in tq.lib().tq_last_error().decode()
    qj8 = _q(head_dim=128, dt=128, bits=8, signs=np.ones(128), flags=tq.TQ_QJL, qjl_m=128)
    qj8.cfg.qjl_params = FAKE
    assert _quantize(qj8, bits=FAKE, rnorm=FAKE) == U  # the QJL stage takes a 1..4-bit MSE stage
    for b in (5, 6, 7):
        bad = _q()
        bad.cfg.bits = b
        assert _quantize(bad) == U


@pytest.mark.parametrize("bits", [4, 8])
def test_bucket_table_codebook_limit(bits):
    """A codebook with a cell too narrow for the 4- or 8-bit encoder's bin table (1.6 bins per narrowest
    cell, at most 256 / 1024 entries) is rejected before any launch: here two neighbouring edges 1e-5
    apart, which would need about 4e5 bins."""
    qz = _q(bits=bits)
    h = 1 << (bits - 1)
    cb = qz.codebook
    cb.unit_bounds[h + 1] = cb.unit_bounds[h] + 1e-5
    assert _quantize(qz) == tq.TQ_ERR_INVALID_ARG
    assert "narrowest cell" in tq.lib().tq_last_error().decode()


def test_blocks_validation():
    """TQ_BLOCKS: fp16 norms only, no QJL, 16-byte aligned records, norms must be NULL."""
    E, U = tq.TQ_ERR_INVALID_ARG, tq.TQ_ERR_UNSUPPORTED
    L = tq.lib()
    qz = _q(dt=128, signs=np.ones(128), flags=tq.TQ_BLOCKS)
    q = lambda codes=FAKE, norms=None: L.tq_quantize(ctypes.byref(qz.cfg), FAKE, 4, 128, codes, norms, None, None,
                                                      None)
    d = lambda codes=FAKE, norms=None: L.tq_dequantize(ctypes.byref(qz.cfg), codes, norms, None, None, 4, FAKE,
                                                        tq.TQ_F16, 128, None)
    assert q(norms=FAKE) == E and d(norms=FAKE) == E  # the norms live in the records
    assert q(codes=FAKE + 4) == E and d(codes=FAKE + 8) == E  # records are 16-byte aligned
    assert q(codes=None) == E and d(codes=None) == E
    assert "NULL" in L.tq_last_error().decode()
    bad = _q(dt=128, signs=np.ones(128), flags=tq.TQ_BLOCKS, norm_dtype=tq.TQ_F32)
    assert L.tq_quantize(ctypes.byref(bad.cfg), FAKE, 4, 128, FAKE, None, None, None, None) == E
    qj = _q(head_dim=128, dt=128, bits=2, signs=np.ones(128), flags=tq.TQ_QJL | tq.TQ_BLOCKS, qjl_m=128)
    assert L.tq_quantize(ctypes.byref(qj.cfg), FAKE, 4, 128, FAKE, None, FAKE, FAKE, None) == U
    # records are not an attention cache format
    assert L.tq_decode_attn(ctypes.byref(qz.cfg), ctypes.byref(qz.cfg), FAKE, tq.TQ_F16, 4, 1, 8, FAKE, FAKE, FAKE,
                            FAKE, 0.0, FAKE, FAKE, 1 << 20, None) == U


def test_dequantize_validation():
    E, OK = tq.TQ_ERR_INVALID_ARG, tq.TQ_OK
    qz = _q()
    L = tq.lib()
    call = lambda **k: L.tq_dequantize(ctypes.byref(qz.cfg), k.get("codes", FAKE), k.get("norms", FAKE), None, None,
                                       k.get("n", 4), k.get("y", FAKE), k.get("yt", tq.TQ_F16), k.get("ld", 128), None)
    assert call(n=0) == OK
    assert call(yt=7) == E
    assert call(y=None) == E
    assert call(y=FAKE + 8) == E
    assert call(ld=64) == E
    assert call(codes=None) == E


def test_status_strings():
    L = tq.lib()
    assert L.tq_status_str(tq.TQ_OK) == b"ok"
    assert L.tq_status_str(tq.TQ_ERR_WORKSPACE).startswith(b"workspace")
    assert L.tq_status_str(99) == b"unknown status"


def _attn_ws(qz, rows, n_kv, tokens, op=None):
    return tq.lib().tq_workspace_size(tq.TQ_OP_MULTI_ATTN if op is None else op, ctypes.byref(qz.cfg), rows, n_kv,
                                      tokens)


def test_attention_validation():
    """tq_decode_attn / tq_multi_attn reject bad formats and arguments before any launch."""
    E, U, W, OK = tq.TQ_ERR_INVALID_ARG, tq.TQ_ERR_UNSUPPORTED, tq.TQ_ERR_WORKSPACE, tq.TQ_OK
    L = tq.lib()
    k3 = _q(head_dim=256, signs=np.ones(32))
    v3 = _q(head_dim=256, signs=np.ones(32))
    big = 1 << 24

    def multi(kq=k3, vq=v3, q=FAKE, qt=tq.TQ_F16, n_q=4, hq=8, hkv=2, T=1000, codes=FAKE, causal=1, scale=0.0,
              out=FAKE, ws=FAKE, wsb=big):
        return L.tq_multi_attn(ctypes.byref(kq.cfg), ctypes.byref(vq.cfg), q, qt, n_q, hq, hkv, T, codes, FAKE, codes,
                               FAKE, causal, scale, out, ws, wsb, None)

    assert multi(n_q=0) == OK and multi(T=0, causal=0) == OK  # nothing to do
    assert multi(T=0) == E  # a causal chunk longer than the (empty) cache
    assert multi(n_q=-1) == E
    assert multi(n_q=1001) == E  # a causal chunk longer than the cache
    assert multi(hq=6, hkv=4) == E  # query heads not a multiple of KV heads
    assert multi(qt=5) == E
    assert multi(q=None) == E and multi(out=FAKE + 2) == E
    assert multi(codes=FAKE + 2) == E
    assert multi(scale=float("nan")) == E
    assert multi(ws=None) == W and multi(wsb=256) == W and multi(ws=FAKE + 64) == W
    assert multi(vq=_q(head_dim=256, bits=8, signs=np.ones(32))) == U  # 8-bit values
    assert multi(kq=_q(head_dim=256, bits=2, signs=np.ones(32))) == U  # 2-bit keys
    assert multi(kq=_q(head_dim=64, dt=32, signs=np.ones(32)), vq=_q(head_dim=64, dt=32, signs=np.ones(32))) == U
    assert multi(kq=_q(head_dim=256, dt=64, signs=np.ones(64)), vq=_q(head_dim=256, dt=64, signs=np.ones(64))) == U
    assert multi(vq=_q(head_dim=128, signs=np.ones(32))) == E  # K and V head_dim differ
    nc = _q(head_dim=256, signs=np.ones(32), flags=tq.TQ_NORM_CORRECT)
    assert multi(kq=nc) == U
    assert L.tq_decode_attn(ctypes.byref(k3.cfg), ctypes.byref(v3.cfg), FAKE, tq.TQ_F16, 8, 2, 1000, FAKE, FAKE, FAKE,
                            FAKE, 0.0, FAKE, None, 0, None) == W


def test_decode_attn_noalloc_validation():
    """tq_decode_attn_noalloc rejects bad arguments, and calls whose partials exceed its 16 MiB static
    scratch, before it resolves the scratch or launches anything."""
    E, U, OK = tq.TQ_ERR_INVALID_ARG, tq.TQ_ERR_UNSUPPORTED, tq.TQ_OK
    L = tq.lib()
    k3 = _q(head_dim=256, signs=np.ones(32))
    v3 = _q(head_dim=256, signs=np.ones(32))

    def call(hq=16, hkv=1, T=1000, kq=k3, vq=v3, qt=tq.TQ_F16):
        return L.tq_decode_attn_noalloc(ctypes.byref(kq.cfg), ctypes.byref(vq.cfg), FAKE, qt, hq, hkv, T, FAKE, FAKE,
                                        FAKE, FAKE, 0.0, FAKE, None)

    assert _attn_ws(k3, 16, 1, 8_400_000, tq.TQ_OP_DECODE_ATTN) > 16 << 20
    assert call(T=8_400_000) == U and "scratch" in L.tq_last_error().decode()
    assert call(hq=64, hkv=4, T=2_100_000) == U
    assert call(hq=16, hkv=3) == E  # query heads not a multiple of KV heads
    assert call(vq=_q(head_dim=256, bits=8, signs=np.ones(32))) == U  # 8-bit values
    assert call(T=-1) == E
    assert call(T=0) == OK and call(T=0, qt=5) == E  # nothing to do, but the arguments are still checked


def test_attention_workspace_sizes():
    """Partials: one (head_dim + 2)-float record per row and token range; up to 16 rows per KV head
    form one group (decode kernel), more go in 128-row groups (prefill kernel)."""
    qz = _q(head_dim=256, signs=np.ones(32))
    dec = tq.lib().tq_workspace_size(tq.TQ_OP_DECODE_ATTN, ctypes.byref(qz.cfg), 16, 4, 131072)
    assert dec > 0 and dec == _attn_ws(qz, 16, 4, 131072)  # one query token = the decode call
    assert dec % 256 == 0 and dec >= 16 * 258 * 4
    # more rows never shrink the workspace, and a 128-row group holds every row it serves
    sizes = [_attn_ws(qz, 16 * n_q, 4, 131072) for n_q in (1, 2, 4, 8, 64)]
    assert all(b >= a for a, b in zip(sizes, sizes[1:]))
    assert _attn_ws(qz, 16 * 64, 4, 131072) >= 16 * 64 * 258 * 4
    assert _attn_ws(qz, 0, 4, 100) == 0 and _attn_ws(qz, 6, 4, 100) == 0  # no rows / not a multiple
