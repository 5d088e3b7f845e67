"""Pins for the oracle's record format of the fork ([Fork] "GGML Types", "How it works",
"KV Cache Memory"; CPU only).

  * record sizes equal the printed block sizes (14 B turbo3, 18 B turbo4) and
    bits per value, and the 131072-token cache of the "KV Cache Memory" table
    (head_dim 256 split into two 128-value chunks, one norm per chunk copied
    into each 32-value block) comes to the printed MiB exactly: the copies add
    no bytes;
  * every block of a chunk carries the fp16 norm of that chunk, computed here
    independently of the quantizer;
  * to_blocks / from_blocks round-trip exactly and the record's code bytes are
    the separate-plane bytes of the same group;
  * a 256-value head encoded as two 128-value chunks equals each half encoded
    on its own ([Fork] "How it works": each half is its own unit vector);
  * decoding records equals the pinned dequantize when all copies agree, and
    scales a block by its own copy otherwise.
"""
import numpy as np
import pytest

import synth
from oracle import Codebook, dequantize, dequantize_blocks, from_blocks, quantize, record_bytes, to_blocks


@pytest.mark.parametrize("name,bits", [("turbo3", 3), ("turbo4", 4)])
def test_record_size_and_cache_bytes(name, bits, golden):
    g = golden("fork_block_bytes.json")
    assert record_bytes(bits) == g[name]["block_bytes"]
    assert 8 * record_bytes(bits) / g["block_values"] == g[name]["bpw"]
    hd, layers, tokens = g["kv_cache_131072_head_dim"], g["kv_cache_131072_layers"], 131072
    kv_heads = 4  # from the f16 column: 4096 MiB / (8 layers * 2 * 131072 * 256 * 2 B)
    assert g["kv_cache_131072_mib"]["f16"] * 2**20 == layers * 2 * kv_heads * tokens * hd * 2
    cb = Codebook.build(bits, 128)
    x = synth.normal(1, 0, 3 * hd).reshape(3, hd)
    q = quantize(x, np.ones(128), cb)
    rec = to_blocks(q["codes"], q["norms"], bits, 128)
    bytes_per_vector = rec.size // 3
    assert bytes_per_vector == hd // 32 * g[name]["block_bytes"]
    total = layers * 2 * kv_heads * tokens * bytes_per_vector
    assert total == g["kv_cache_131072_mib"][name] * 2**20


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_norm_copied_into_every_block(bits):
    x = synth.kv_tensor(5, 1, 1, 0, 40, 256).reshape(40, 256)
    cb = Codebook.build(bits, 128)
    q = quantize(x, synth.signs(5, 2, 128), cb)
    rec = to_blocks(q["codes"], q["norms"], bits, 128).reshape(40, 2, 4, record_bytes(bits))
    chunk_norms = np.linalg.norm(x.astype(np.float64).reshape(40, 2, 128), axis=2).astype(np.float16)
    stored = np.ascontiguousarray(rec[..., :2]).view("<f2")[..., 0]
    np.testing.assert_array_equal(stored, np.repeat(chunk_norms[:, :, None], 4, axis=2))
    # the code bytes of block b are the separate-plane bytes of group b
    planes = q["codes"].reshape(40, 2, 4, 4 * bits)
    np.testing.assert_array_equal(rec[..., 2:], planes)


@pytest.mark.parametrize("dt,bits", [(128, 3), (128, 4), (32, 3), (64, 2), (256, 1)])
def test_round_trip(dt, bits):
    rng = np.random.default_rng(dt + bits)
    n = 17
    codes = rng.integers(0, 256, size=(n, dt * bits // 8), dtype=np.uint8)
    norms = rng.normal(size=n).astype(np.float16)
    rec = to_blocks(codes, norms, bits, dt)
    assert rec.shape == (n * dt // 32, record_bytes(bits))
    c2, bn = from_blocks(rec, bits, dt)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(bn, np.repeat(norms[:, None], dt // 32, axis=1))


def test_head_256_is_two_independent_chunks():
    x = synth.kv_tensor(8, 1, 1, 0, 25, 256).reshape(25, 256)
    D = synth.signs(8, 2, 128)
    cb = Codebook.build(3, 128)
    whole = quantize(x, D, cb)
    halves = [quantize(x[:, 128 * h:128 * (h + 1)], D, cb) for h in (0, 1)]
    np.testing.assert_array_equal(whole["codes"].reshape(25, 2, -1)[:, 0], halves[0]["codes"])
    np.testing.assert_array_equal(whole["codes"].reshape(25, 2, -1)[:, 1], halves[1]["codes"])
    np.testing.assert_array_equal(whole["norms"].reshape(25, 2)[:, 1], halves[1]["norms"])


@pytest.mark.parametrize("nc", [False, True])
def test_decode_matches_dequantize_and_uses_each_copy(nc):
    x = synth.kv_tensor(9, 1, 1, 0, 30, 128).reshape(30, 128)
    D = synth.signs(9, 2, 128)
    cb = Codebook.build_beta(3, 128)
    q = quantize(x, D, cb)
    rec = to_blocks(q["codes"], q["norms"], 3, 128)
    ref = dequantize(q["codes"], q["norms"], D, cb, nc=nc)
    np.testing.assert_allclose(dequantize_blocks(rec, D, cb, nc=nc), ref, rtol=0, atol=1e-15)
    # change the copy in block 2 of unit 5: only that block's 32 outputs scale
    rec2 = rec.copy().reshape(30, 4, 14)
    rec2[5, 2, :2] = np.array([np.float16(2.0) * q["norms"][5]], dtype="<f2").view(np.uint8)
    out = dequantize_blocks(rec2.reshape(-1, 14), D, cb, nc=nc)
    np.testing.assert_allclose(out[5, 64:96], 2.0 * ref[5, 64:96], rtol=1e-15)
    np.testing.assert_array_equal(np.delete(out, np.s_[64:96], axis=1), np.delete(ref, np.s_[64:96], axis=1))
