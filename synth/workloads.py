"""Input recipes for the five measured configurations (shapes, seeds, streams).

Pure input generation: every function returns numpy arrays drawn with the
generator in this package.  The shapes stand in for real KV tensors of the
models the pages measure on (their weights and corpora are not available):

  vectors_fp32   4096 random vectors, d = 128, fp32, N(0,1) entries, seed 0
  llama_1b_kv    16 layers x 8 KV heads x 2048 tokens x head_dim 64, fp16
  qwen3_8b_kv    36 layers x 8 KV heads x 16384 tokens x head_dim 128, fp16
                 (sign vectors for 32-value blocks; qwen3_8b_kv_chunk128: the
                 same tensors with sign vectors for 128-value chunks)
  qjl_keys       65536 keys x 128 fp16 (per-channel log-normal, no outliers),
                 4096 queries (32 heads x 128) ~ N(0,1) fp16, S: 128 x 128 N(0,1), seed 1
  decode_cache   1 layer x 4 KV heads x 131072 tokens x head_dim 256 fp16,
                 16 query heads x 256 ~ N(0,1) fp16

KV entries: N(0,1) times a per-channel log-normal scale exp(1.0 * N(0,1)),
with 2 outlier channels per (layer, KV head, K|V) multiplied by 10.
Every size argument can be shrunk for tests; the recipe stays the same.
"""
from __future__ import annotations

import numpy as np

from . import (STREAM_K, STREAM_QUERY, STREAM_SIGNS_K, STREAM_SIGNS_V, STREAM_V, gaussian_matrix, kv_tensor,
               normal_f16, normal_f32, signs)

SEED = 0
QJL_SEED = 1


def vectors_fp32(n: int = 4096, d: int = 128, seed: int = SEED):
    x = normal_f32(seed, STREAM_K, n * d).reshape(n, d)
    return {"x": x, "signs": signs(seed, STREAM_SIGNS_K, d)}


def kv_pair(layers: int, heads: int, tokens: int, head_dim: int, dt: int, seed: int = SEED, n_outliers: int = 2,
            out_k=None, out_v=None):
    return {
        "k": kv_tensor(seed, layers, heads, 0, tokens, head_dim, n_outliers=n_outliers, out=out_k),
        "v": kv_tensor(seed, layers, heads, 1, tokens, head_dim, n_outliers=n_outliers, out=out_v),
        "signs_k": signs(seed, STREAM_SIGNS_K, dt),
        "signs_v": signs(seed, STREAM_SIGNS_V, dt),
    }


def llama_1b_kv(layers: int = 16, heads: int = 8, tokens: int = 2048, head_dim: int = 64, seed: int = SEED):
    return kv_pair(layers, heads, tokens, head_dim, dt=head_dim, seed=seed)


def qwen3_8b_kv(layers: int = 36, heads: int = 8, tokens: int = 16384, head_dim: int = 128, seed: int = SEED,
                out_k=None, out_v=None):
    return kv_pair(layers, heads, tokens, head_dim, dt=32, seed=seed, out_k=out_k, out_v=out_v)


def qwen3_8b_kv_chunk128(layers: int = 36, heads: int = 8, tokens: int = 16384, seed: int = SEED):
    return kv_pair(layers, heads, tokens, 128, dt=128, seed=seed)


def qjl_keys(n_keys: int = 65536, d: int = 128, n_queries: int = 4096, m: int = 128, seed: int = SEED):
    keys = kv_tensor(seed, 1, 1, 0, n_keys, d, n_outliers=0).reshape(n_keys, d)
    q = normal_f16(seed, STREAM_QUERY, n_queries * d).reshape(n_queries, d)
    return {"keys": keys, "q": q, "signs": signs(seed, STREAM_SIGNS_K, d), "S": gaussian_matrix(QJL_SEED, 0, m, d)}


def decode_cache(kv_heads: int = 4, tokens: int = 131072, head_dim: int = 256, q_heads: int = 16, seed: int = SEED):
    c = kv_pair(1, kv_heads, tokens, head_dim, dt=32, seed=seed)
    c["q"] = normal_f16(seed, STREAM_QUERY, q_heads * head_dim).reshape(q_heads, head_dim)
    return c
