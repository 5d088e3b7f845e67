"""Pins for the oracle's decode attention (CPU only).

  * equals a per-token pure-Python loop (exp, sum, weighted sum) on tiny inputs;
  * special cases: one token gives v~_0; a zero query gives the mean of v~;
  * several query tokens (with and without the causal mask) against a loop over the visible
    tokens, against decode calls over the visible prefix, and the first causal row = v~_0;
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


def _multi(q, cache, n_kv, tokens, hd, causal):
    from oracle import multi_attention

    cb, dk, dv, ek, ev = cache
    return multi_attention(q, ek["codes"], ek["norms"], ev["codes"], ev["norms"], dk, dv, cb, cb, n_kv, tokens, hd,
                           causal=causal)


def test_multi_query_matches_per_token_loop_with_mask():
    """Several query tokens with the causal mask against a pure-Python loop over the visible tokens."""
    n_kv, G, n_q, tokens, hd = 2, 2, 3, 6, 32
    cache = _cache(n_kv, tokens, hd, seed=5)
    cb, dk, dv, ek, ev = cache
    q = synth.normal_f16(5, 6, n_q * n_kv * G * hd).reshape(n_q, n_kv * G, hd)
    out = _multi(q, cache, n_kv, tokens, hd, causal=True)
    kd = dequantize(ek["codes"], ek["norms"], dk, cb).reshape(n_kv, tokens, hd)
    vd = dequantize(ev["codes"], ev["norms"], dv, cb).reshape(n_kv, tokens, hd)
    for i in range(n_q):
        visible = tokens - n_q + i + 1
        for h in range(n_kv * G):
            g = h // G
            logits = [sum(float(q[i, h, c]) * kd[g, j, c] for c in range(hd)) / math.sqrt(hd) for j in range(visible)]
            mx = max(logits)
            w = [math.exp(s - mx) for s in logits]
            ref = [sum(w[j] * vd[g, j, c] for j in range(visible)) / sum(w) for c in range(hd)]
            np.testing.assert_allclose(out[i, h], ref, rtol=1e-12, atol=1e-12)


def test_multi_query_reduces_to_decode():
    """Without the mask every query token is a decode call; with it, row i is a decode call over the
    first n_tokens - n_q + i + 1 tokens; a causal chunk as long as the cache starts with v~_0."""
    n_kv, G, n_q, tokens, hd = 1, 4, 5, 40, 64
    cache = _cache(n_kv, tokens, hd, seed=6)
    cb, dk, dv, ek, ev = cache
    q = synth.normal_f16(6, 6, n_q * G * hd).reshape(n_q, G, hd)
    full = _multi(q, cache, n_kv, tokens, hd, causal=False)
    masked = _multi(q, cache, n_kv, tokens, hd, causal=True)
    upt = hd // 32
    for i in range(n_q):
        dec = decode_attention(q[i], ek["codes"], ek["norms"], ev["codes"], ev["norms"], dk, dv, cb, cb, n_kv, tokens,
                               hd)
        np.testing.assert_allclose(full[i], dec, rtol=1e-13, atol=1e-15)
        t = tokens - n_q + i + 1
        dec = decode_attention(q[i], ek["codes"][:t * upt], ek["norms"][:t * upt], ev["codes"][:t * upt],
                               ev["norms"][:t * upt], dk, dv, cb, cb, n_kv, t, hd)
        np.testing.assert_allclose(masked[i], dec, rtol=1e-13, atol=1e-15)
    q = synth.normal_f16(7, 6, tokens * G * hd).reshape(tokens, G, hd)
    first = _multi(q, cache, n_kv, tokens, hd, causal=True)[0]
    vd = dequantize(ev["codes"][:upt], ev["norms"][:upt], dv, cb).reshape(hd)
    np.testing.assert_allclose(first, np.repeat(vd[None], G, axis=0), rtol=1e-14)
