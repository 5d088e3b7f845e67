"""Pins for the oracle's rotation, bucketize, codes and packing (CPU only).

  * fwht equals the explicit (-1)^popcount(i&j)/sqrt(d) matrix; H H = I; H = H^T;
    Parseval; H e_0 = 1/sqrt(d).
  * quantize picks, by brute force over every index tuple of a tiny unit, the
    codeword D H c nearest to the unit vector (so encode and decode rotations
    are each other's inverse and bucketize picks the nearest centroid).
  * index histograms on random unit vectors follow the cell probabilities of
    the exact coordinate marginal (chi-square).
  * packing: a worked example written with Python integers; round trips; the
    byte counts printed in [Fork] "GGML Types" / "KV Cache Memory".
"""
import itertools
import math

import numpy as np
import pytest
from scipy import integrate, special, stats

from oracle import (Codebook, code_to_index, dequantize, encode_indices, fwht, hadamard_matrix, index_to_code, pack_codes,
                    pack_sign_bits, quantize, unpack_codes, unpack_sign_bits)


@pytest.mark.parametrize("d", [2, 4, 8, 16, 32, 64, 128, 256])
def test_fwht_is_the_hadamard_matrix(d):
    rng = np.random.default_rng(d)
    v = rng.normal(size=(3, d))
    H = hadamard_matrix(d)
    np.testing.assert_allclose(fwht(v), v @ H.T, atol=1e-13)
    np.testing.assert_allclose(H @ H, np.eye(d), atol=1e-14)
    np.testing.assert_array_equal(H, H.T)
    np.testing.assert_allclose(np.linalg.norm(fwht(v), axis=1), np.linalg.norm(v, axis=1), rtol=1e-14)
    e0 = np.zeros(d)
    e0[0] = 1.0
    np.testing.assert_allclose(fwht(e0), np.full(d, 1.0 / math.sqrt(d)), atol=1e-16)
    np.testing.assert_allclose(fwht(fwht(v)), v, atol=1e-13)


def test_hadamard_entries_by_popcount():
    H = hadamard_matrix(8) * math.sqrt(8)
    assert H[3, 5] == -1.0  # 3 & 5 = 1 -> one set bit
    assert H[3, 3] == 1.0  # popcount(3) = 2
    assert H[7, 7] == -1.0  # popcount(7) = 3


@pytest.mark.parametrize("d,bits", [(2, 1), (2, 2), (2, 3), (4, 1), (4, 2), (4, 3), (8, 1), (8, 2)])
def test_brute_force_nearest_codeword(d, bits):
    # Brute force in the UNROTATED domain, with codewords built from the
    # explicit Hadamard matrix: the nearest of all L^d codewords D H c(idx)
    # to u must be the index tuple the oracle's encoder picked.
    cb_unit = Codebook.build(bits, 32)
    cb = Codebook(bits, d, cb_unit.unit_levels, cb_unit.unit_bounds, cb_unit.distortion)
    rng = np.random.default_rng(100 * d + bits)
    D = np.where(rng.random(d) < 0.5, 1.0, -1.0)
    L = 1 << bits
    tuples = np.array(list(itertools.product(range(L), repeat=d)))
    words = (cb.levels[tuples] @ hadamard_matrix(d).T) * D  # [L^d, d]
    x = rng.normal(size=(40, d))
    n, u, _, idx = encode_indices(x, D, cb)
    np.testing.assert_allclose(n, np.linalg.norm(x, axis=1), rtol=1e-15)
    for r in range(40):
        best = tuples[np.argmin(np.sum((words - u[r]) ** 2, axis=1))]
        np.testing.assert_array_equal(idx[r], best)


def test_brute_force_through_full_quantize_path():
    # d = 32 cannot be enumerated; check instead that quantize -> dequantize
    # returns the codeword that is nearest coordinate-by-coordinate in the
    # rotated domain, and that no single-coordinate change of the index
    # brings the reconstruction closer to u.
    cb = Codebook.build(3, 32)
    rng = np.random.default_rng(7)
    D = np.where(rng.random(32) < 0.5, 1.0, -1.0)
    x = rng.normal(size=(16, 32))
    q = quantize(x, D, cb, norm_dtype=np.float64)
    rec = dequantize(q["codes"], np.ones(16), D, cb)
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    idx = code_to_index(unpack_codes(q["codes"], 3, 32), 3)
    base = np.sum((rec - u) ** 2, axis=1)
    for j in range(32):
        for delta in (-1, 1):
            alt = idx.copy()
            alt[:, j] = np.clip(alt[:, j] + delta, 0, 7)
            rec_alt = fwht(cb.levels[alt]) * D
            assert np.all(np.sum((rec_alt - u) ** 2, axis=1) >= base - 1e-15)


def test_index_histogram_chi_square():
    d, bits = 128, 3
    cb = Codebook.build(bits, d)
    import synth

    x = synth.normal(3, 0, 4000 * d).reshape(4000, d)
    D = synth.signs(3, 2, d)
    q = quantize(x, D, cb, norm_dtype=np.float64)
    idx = code_to_index(unpack_codes(q["codes"], bits, d), bits).ravel()
    counts = np.bincount(idx, minlength=8)
    # exact marginal of one coordinate of a uniform unit vector in R^d
    lc = special.gammaln(d / 2) - 0.5 * math.log(math.pi) - special.gammaln((d - 1) / 2)
    pdf = lambda t: math.exp(lc + (d - 3) / 2 * math.log1p(-t * t))
    edges = [-1.0] + list(cb.bounds) + [1.0]
    probs = np.array([integrate.quad(pdf, edges[i], edges[i + 1], epsabs=1e-13)[0] for i in range(8)])
    assert probs.sum() == pytest.approx(1.0, abs=1e-9)
    # coordinates of one vector are weakly dependent; the chi-square is still a good check at this size
    chi2, p = stats.chisquare(counts, probs * counts.sum())
    assert p > 1e-4, (counts, probs * counts.sum())


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_code_bijection_and_zero(bits):
    L = 1 << bits
    idx = np.arange(L)
    code = index_to_code(idx, bits)
    assert sorted(code.tolist()) == list(range(L))
    np.testing.assert_array_equal(code_to_index(code, bits), idx)
    h = L // 2
    # the two cells next to zero have magnitude 0; the top bit marks the negative half
    assert code[h] == 0 and code[h - 1] == (1 << (bits - 1))
    assert code[0] == (1 << (bits - 1)) | (h - 1) and code[L - 1] == h - 1


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_pack_worked_example_and_round_trip(bits):
    L = 1 << bits
    codes = (np.arange(64) * 5 + 3) % L
    codes = codes.reshape(1, 64)
    packed = pack_codes(codes, bits)
    assert packed.shape == (1, 64 * bits // 8)
    # reference: each 32-group is the integer sum(code_j << (bits*j)) written little-endian
    expected = b""
    for g in range(2):
        word = sum(int(codes[0, 32 * g + j]) << (bits * j) for j in range(32))
        expected += word.to_bytes(4 * bits, "little")
    assert bytes(packed[0]) == expected
    np.testing.assert_array_equal(unpack_codes(packed, bits, 64), codes)
    rng = np.random.default_rng(bits)
    c = rng.integers(0, L, size=(50, 128))
    np.testing.assert_array_equal(unpack_codes(pack_codes(c, bits), bits, 128), c)


def test_sign_bit_packing():
    rng = np.random.default_rng(1)
    pos = rng.random((7, 128)) < 0.5
    packed = pack_sign_bits(pos)
    assert packed.shape == (7, 16)
    for r in range(7):
        word = sum(int(pos[r, i]) << i for i in range(128))
        assert bytes(packed[r]) == word.to_bytes(16, "little")
    np.testing.assert_array_equal(unpack_sign_bits(packed, 128), np.where(pos, 1.0, -1.0))


def test_block_bytes_match_fork_tables(golden):
    g = golden("fork_block_bytes.json")
    for name, bits in (("turbo3", 3), ("turbo4", 4)):
        cb = Codebook.build(bits, 32)
        q = quantize(np.ones((1, 32)), np.ones(32), cb)
        packed = q["codes"].shape[1]
        norm = q["norms"].dtype.itemsize
        assert packed == g[name]["packed_bytes"] and norm == g[name]["norm_bytes"]
        assert packed + norm == g[name]["block_bytes"]
        assert 8 * (packed + norm) / g["block_values"] == g[name]["bpw"]
        assert (packed + norm) / g["block_values"] == g[name]["bytes_per_element"]
    # one attention layer of the 131072-token cache (4 KV heads of 256, by the MiB table's arithmetic)
    mib = g["kv_cache_131072_mib"]
    layers, hd, tokens = g["kv_cache_131072_layers"], g["kv_cache_131072_head_dim"], 131072
    kv_heads = mib["f16"] * 2**20 / (layers * 2 * tokens * hd * g["f16_bytes_per_element"])
    assert kv_heads == 4
    turbo3_layer = 2 * kv_heads * tokens * hd * g["turbo3"]["bytes_per_element"]
    assert turbo3_layer == mib["turbo3"] * 2**20 / layers == 112 * 2**20


def test_zero_unit():
    for bits in (1, 2, 3, 4):
        cb = Codebook.build(bits, 32)
        q = quantize(np.zeros((2, 32)), np.ones(32), cb)
        assert np.all(q["norms"] == 0)
        idx = code_to_index(unpack_codes(q["codes"], bits, 32), bits)
        assert np.all(idx == (1 << (bits - 1)) - 1)
        assert np.all(dequantize(q["codes"], q["norms"], np.ones(32), cb) == 0)


def test_decode_uses_stored_norm_and_sign_vector():
    cb = Codebook.build(4, 64)
    rng = np.random.default_rng(3)
    D = np.where(rng.random(64) < 0.5, 1.0, -1.0)
    x = rng.normal(size=(5, 64)) * 3.3
    q = quantize(x, D, cb)
    unit = dequantize(q["codes"], np.ones(5), D, cb)
    scaled = dequantize(q["codes"], q["norms"], D, cb)
    np.testing.assert_allclose(scaled, unit * q["norms"].astype(np.float64)[:, None], rtol=1e-15)
    # flipping D changes the reconstruction (D is applied on the way out)
    other = dequantize(q["codes"], np.ones(5), -D, cb)
    np.testing.assert_allclose(other, -unit, atol=1e-15)
