"""Single-token decode attention over a quantized KV cache (oracle side).

Plain softmax attention over the dequantized cache: every cached key and value
is decoded with the oracle's ``dequantize`` (one inverse rotation per block,
exactly as the method defines the reconstruction), then

    s_hj = <q_h, k~_j> * scale,   p = softmax_j(s_h),   out_h = sum_j p_hj v~_j

with scale = 1/sqrt(head_dim) ([Blog] Part 3 divides the logits by sqrt(d_k)
before the softmax) and query head h reading KV head h // (H_q / H_kv).
[Fork] "Fused tile path" computes the same thing in the rotated domain; the
oracle deliberately does not use that shortcut.
"""
from __future__ import annotations

import math

import numpy as np

from .codebook import Codebook
from .quantizer import dequantize


def decode_attention(q, k_codes, k_norms, v_codes, v_norms, k_signs, v_signs, k_cb: Codebook, v_cb: Codebook,
                     n_kv_heads: int, n_tokens: int, head_dim: int, scale: float | None = None) -> np.ndarray:
    """q: [H_q, head_dim]; codes/norms: [H_kv * n_tokens * head_dim/dt] units in
    (kv head, token, block) order.  Returns [H_q, head_dim] float64."""
    q = np.asarray(q, dtype=np.float64)
    n_q_heads = q.shape[0]
    if n_q_heads % n_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    group = n_q_heads // n_kv_heads
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    k = dequantize(k_codes, k_norms, k_signs, k_cb).reshape(n_kv_heads, n_tokens, head_dim)
    v = dequantize(v_codes, v_norms, v_signs, v_cb).reshape(n_kv_heads, n_tokens, head_dim)
    out = np.zeros((n_q_heads, head_dim), dtype=np.float64)
    for h in range(n_q_heads):
        g = h // group
        s = (k[g] @ q[h]) * scale
        w = np.exp(s - s.max())
        out[h] = (w / w.sum()) @ v[g]
    return out


def multi_attention(q, k_codes, k_norms, v_codes, v_norms, k_signs, v_signs, k_cb: Codebook, v_cb: Codebook,
                    n_kv_heads: int, n_tokens: int, head_dim: int, causal: bool = False,
                    scale: float | None = None) -> np.ndarray:
    """Several query tokens over the same cache: q [n_q, H_q, head_dim].  Query token i sees every
    cached token, or with ``causal`` the tokens j <= n_tokens - n_q + i (the queries are the last
    n_q positions of the cache, as in a prefill chunk whose K and V were appended first).  The
    softmax is taken over the visible tokens only.  Returns [n_q, H_q, head_dim] float64."""
    q = np.asarray(q, dtype=np.float64)
    n_q, n_q_heads = q.shape[0], q.shape[1]
    if n_q_heads % n_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    if causal and n_q > n_tokens:
        raise ValueError("a causal chunk cannot be longer than the cache")
    group = n_q_heads // n_kv_heads
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    k = dequantize(k_codes, k_norms, k_signs, k_cb).reshape(n_kv_heads, n_tokens, head_dim)
    v = dequantize(v_codes, v_norms, v_signs, v_cb).reshape(n_kv_heads, n_tokens, head_dim)
    out = np.zeros((n_q, n_q_heads, head_dim), dtype=np.float64)
    for i in range(n_q):
        last = n_tokens - n_q + i if causal else n_tokens - 1
        for h in range(n_q_heads):
            g = h // group
            s = (k[g, :last + 1] @ q[i, h]) * scale
            w = np.exp(s - s.max())
            out[i, h] = (w / w.sum()) @ v[g, :last + 1]
    return out
