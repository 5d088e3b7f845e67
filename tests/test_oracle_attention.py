"""Pins for the oracle's decode attention (CPU only).

  * equals a per-token pure-Python loop (exp, sum, weighted sum) on tiny inputs;
  * special cases: one token gives v~_0; a zero query gives the mean of v~;
  * the rotated-domain identities of [Fork] "Fused tile path"
    (<D H c, q> = <c, H D q> and sum_j p_j D H c_j = D H sum_j p_j c_j), in float64.
"""
import math

import numpy as np
import pytest

import synth
from oracle import Codebook, decode_attention, dequantize, fwht, quantize


def _cache(n_kv, tokens, hd, bits=3, seed=0):
    cb = Codebook.build(bits, 32)
    k = synth.kv_tensor(seed, 1, n_kv, 0, tokens, hd)
    v = synth.kv_tensor(seed, 1, n_kv, 1, tokens, hd)
    dk, dv = synth.signs(seed, 2, 32), synth.signs(seed, 3, 32)
    ek, ev = quantize(k, dk, cb), quantize(v, dv, cb)
    return cb, dk, dv, ek, ev


def test_matches_per_token_loop():
    n_kv, n_q, tokens, hd = 2, 4, 5, 64
    cb, dk, dv, ek, ev = _cache(n_kv, tokens, hd)
    q = synth.normal_f16(0, 6, n_q * hd).reshape(n_q, hd)
    out = decode_attention(q, ek["codes"], ek["norms"], ev["codes"], ev["norms"], dk, dv, cb, cb, n_kv, tokens, hd)
    kd = dequantize(ek["codes"], ek["norms"], dk, cb).reshape(n_kv, tokens, hd)
    vd = dequantize(ev["codes"], ev["norms"], dv, cb).reshape(n_kv, tokens, hd)
    for h in range(n_q):
        g = h // (n_q // n_kv)
        logits = [sum(float(q[h, i]) * kd[g, j, i] for i in range(hd)) / math.sqrt(hd) for j in range(tokens)]
        mx = max(logits)
        w = [math.exp(s - mx) for s in logits]
        tot = sum(w)
        ref = [sum(w[j] * vd[g, j, i] for j in range(tokens)) / tot for i in range(hd)]
        np.testing.assert_allclose(out[h], ref, rtol=1e-12, atol=1e-12)


def test_single_token_and_zero_query():
    n_kv, n_q, hd = 1, 2, 64
    cb, dk, dv, ek, ev = _cache(n_kv, 1, hd)
    q = synth.normal_f16(1, 6, n_q * hd).reshape(n_q, hd)
    out = decode_attention(q, ek["codes"], ek["norms"], ev["codes"], ev["norms"], dk, dv, cb, cb, n_kv, 1, hd)
    vd = dequantize(ev["codes"], ev["norms"], dv, cb).reshape(1, hd)
    np.testing.assert_allclose(out, np.repeat(vd, n_q, axis=0), rtol=1e-14)
    tokens = 9
    cb, dk, dv, ek, ev = _cache(n_kv, tokens, hd, seed=4)
    out = decode_attention(np.zeros((n_q, hd)), ek["codes"], ek["norms"], ev["codes"], ev["norms"], dk, dv, cb, cb,
                           n_kv, tokens, hd)
    vd = dequantize(ev["codes"], ev["norms"], dv, cb).reshape(tokens, hd)
    np.testing.assert_allclose(out, np.repeat(vd.mean(axis=0, keepdims=True), n_q, axis=0), rtol=1e-13)


def test_rotated_domain_identities():
    rng = np.random.default_rng(2)
    d = 32
    D = np.where(rng.random(d) < 0.5, 1.0, -1.0)
    c = rng.normal(size=(7, d))
    q = rng.normal(size=d)
    p = rng.random(7)
    np.testing.assert_allclose((fwht(c) * D) @ q, c @ fwht(q * D), rtol=1e-13)
    np.testing.assert_allclose(p @ (fwht(c) * D), fwht(p @ c) * D, rtol=1e-13)
