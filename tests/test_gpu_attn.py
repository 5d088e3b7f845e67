"""GPU parity of tq_decode_attn against the oracle's plain softmax attention.

K and V are encoded on the GPU (block-32, fp16 norms); the oracle then decodes
the GPU's own codes and norms and runs softmax attention in float64, so the
comparison isolates the attention kernels.

Tolerance, derived from the kernel's arithmetic (per query head h and 32-block
b of the output):
  * value side: the weight p_j * n_jb and each centroid enter the MFMA as fp16
    (unit roundoff u = 2^-11); a weight below the fp16 normal range loses at
    most 2^-25 absolutely.  In the rotated domain the accumulated error of
    coordinate k is at most E_k = 2u sum_j p_j n_jb |c_jbk| + 2^-25 sum_j |c_jbk|
    (c: N(0,1)-scale centroids); the output is that vector rotated back by an
    orthonormal map and divided by sqrt(32) * sum_j p_j, so each output entry
    errs by at most ||E||_2 / (sqrt(32) L).
  * key side: query and centroids are split into fp16 hi + lo parts (relative
    error 2^-22 per product, fp32 sums), so every score errs by at most
    eps = 4e-6 * scale * sum_b n_jb ||q_b|| ||c_jb|| / sqrt(32) (+1e-6 for exp);
    a score perturbation of eps moves the output by at most 2 eps max_j |v_jb|.
The test allows 1.25x the sum of both bounds.
"""
import math

import numpy as np
import pytest

import synth
from oracle import Codebook, decode_attention, dequantize
from oracle.quantizer import unpack_codes, code_to_index

torch = pytest.importorskip("torch")
import kv_cache_vector_amd as tq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"
U16 = 2.0 ** -11


class Cache:
    """n_kv_heads x n_tokens x head_dim K and V, encoded on the GPU in the block-32 layout."""

    def __init__(self, k, v, kbits, vbits, signs_k, signs_v, codebook="gaussian"):
        self.H, self.T, self.hd = k.shape
        self.kbits, self.vbits = kbits, vbits
        self.signs_k, self.signs_v = signs_k, signs_v
        self.codebook = codebook
        self.kq = tq.Quantizer(self.hd, 32, kbits, signs_k, codebook=codebook)
        self.vq = tq.Quantizer(self.hd, 32, vbits, signs_v, codebook=codebook)
        self.kc, self.kn = self._encode(self.kq, k, kbits)
        self.vc, self.vn = self._encode(self.vq, v, vbits)

    def _encode(self, qz, x, bits):
        rows = self.H * self.T
        xt = torch.from_numpy(np.ascontiguousarray(x.reshape(rows, self.hd))).to(DEV)
        units = rows * self.hd // 32
        codes = torch.empty(units * 4 * bits, dtype=torch.uint8, device=DEV)
        norms = torch.empty(units, dtype=torch.float16, device=DEV)
        tq.tq_quantize(qz, xt, rows, self.hd, codes, norms)
        return codes, norms

    def attend(self, q, scale=0.0):
        hq = q.shape[0]
        qt = torch.from_numpy(np.ascontiguousarray(q)).to(DEV)
        qtype = tq.TQ_F32 if q.dtype == np.float32 else tq.TQ_F16
        out = torch.full((hq + 1, self.hd), -7.0, dtype=torch.float32, device=DEV)  # one guard row
        wsb = tq.tq_workspace_size(tq.TQ_OP_DECODE_ATTN, self.kq, hq, self.H, self.T)
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
        tq.tq_decode_attn(self.kq, self.vq, qt, qtype, hq, self.H, self.T, self.kc, self.kn, self.vc, self.vn, scale,
                          out, ws, wsb)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.all(o[hq] == -7.0), "output written past the last query head"
        return o[:hq]

    def host(self, kv_heads=None):
        """Codes and norms of the given KV heads (all by default), as the oracle takes them."""
        upt = self.hd // 32
        kc = self.kc.cpu().numpy().reshape(self.H, self.T * upt, -1)
        vc = self.vc.cpu().numpy().reshape(self.H, self.T * upt, -1)
        kn = self.kn.cpu().numpy().reshape(self.H, -1)
        vn = self.vn.cpu().numpy().reshape(self.H, -1)
        sel = list(range(self.H)) if kv_heads is None else list(kv_heads)
        return (kc[sel].reshape(-1, kc.shape[2]), kn[sel].reshape(-1), vc[sel].reshape(-1, vc.shape[2]),
                vn[sel].reshape(-1))

    def oracle(self, q, kv_heads=None, scale=None):
        sel = list(range(self.H)) if kv_heads is None else list(kv_heads)
        G = q.shape[0] // self.H
        qs = np.concatenate([q[g * G:(g + 1) * G] for g in sel])
        kc, kn, vc, vn = self.host(sel)
        build = Codebook.build_beta if self.codebook == "beta" else Codebook.build
        kcb, vcb = build(self.kbits, 32), build(self.vbits, 32)
        out = decode_attention(qs.astype(np.float64), kc, kn, vc, vn, self.signs_k, self.signs_v, kcb, vcb, len(sel),
                               self.T, self.hd, scale)
        bound = self._bound(qs.astype(np.float64), kc, kn, vc, vn, kcb, vcb, len(sel), G,
                            scale if scale else 1.0 / math.sqrt(self.hd))
        return out, bound

    def _bound(self, q, kc, kn, vc, vn, kcb, vcb, H, G, scale):
        T, hd, nb = self.T, self.hd, self.hd // 32
        k = dequantize(kc, kn, self.signs_k, kcb).reshape(H, T, hd)
        v = dequantize(vc, vn, self.signs_v, vcb).reshape(H, T, hd)
        cv = np.abs(vcb.unit_levels[code_to_index(unpack_codes(vc, self.vbits, 32), self.vbits)])
        cv = cv.reshape(H, T, nb, 32)
        ck = kcb.unit_levels[code_to_index(unpack_codes(kc, self.kbits, 32), self.kbits)]
        ckn = np.linalg.norm(ck, axis=1).reshape(H, T, nb)
        knn = kn.astype(np.float64).reshape(H, T, nb)
        vnn = vn.astype(np.float64).reshape(H, T, nb)
        bound = np.zeros(q.shape)
        for h in range(q.shape[0]):
            g = h // G
            s = k[g] @ q[h] * scale
            p = np.exp(s - s.max())
            L = p.sum()
            qb = np.linalg.norm(q[h].reshape(nb, 32), axis=1)
            eps = 4e-6 * scale * np.max((knn[g] * ckn[g]) @ qb) / math.sqrt(32) + 1e-6
            for b in range(nb):
                E = 2 * U16 * ((p * vnn[g, :, b]) @ cv[g, :, b]) + 2.0 ** -25 * cv[g, :, b].sum(axis=0)
                vmax = np.abs(v[g, :, 32 * b:32 * (b + 1)]).max()
                bound[h, 32 * b:32 * (b + 1)] = 1.25 * (np.linalg.norm(E) / (math.sqrt(32) * L) + 2 * eps * vmax)
        return bound + 1e-7


def _check(gpu, orc, bound, what):
    err = np.abs(gpu.astype(np.float64) - orc)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    worst = float(np.max(err / bound))
    assert np.all(err <= bound), f"{what}: error exceeds the derived bound by {worst:.3g}x"
    rel = float(np.max(err) / np.max(np.abs(orc)))
    print(f"{what}: max error {np.max(err):.3g} ({rel:.2e} of max |out|), {worst:.3f} of the bound")


def _data(seed, H, T, hd):
    k = synth.kv_tensor(seed, 1, H, 0, T, hd)[0]
    v = synth.kv_tensor(seed, 1, H, 1, T, hd)[0]
    return k, v, synth.signs(seed, 2, 32), synth.signs(seed, 3, 32)


@pytest.mark.parametrize("hd,H,G,T,kbits,vbits,qdt", [
    (128, 2, 4, 1000, 3, 3, np.float16),   # ragged against the 32-token tile, 256-token wave, 1024-token group
    (256, 1, 16, 2500, 4, 4, np.float32),  # 16 query heads per KV head
    (128, 3, 1, 33, 3, 4, np.float16),     # one query head per KV head, one token past a tile
    (256, 2, 3, 1, 4, 3, np.float32),      # a single token, a group that is not a power of two
    (128, 1, 8, 5000, 4, 4, np.float16),   # several token ranges per KV head
    (256, 4, 4, 3000, 3, 3, np.float16),   # the decode workload's head layout at a short length
    (128, 2, 4, 1000, 8, 4, np.float16),   # 8-bit keys, 4-bit values
    (256, 2, 4, 2100, 8, 3, np.float32),   # 8-bit keys, 3-bit values, ragged tail
    (256, 1, 16, 70, 8, 4, np.float16),    # 8-bit keys with 16 query heads, one tile and a bit
    (128, 1, 32, 500, 3, 3, np.float16),   # 32 query heads per KV head: two 16-row groups
    (128, 2, 20, 300, 4, 3, np.float32),   # 20 heads per KV head: a full and a partial row group
])
def test_attn_matrix(hd, H, G, T, kbits, vbits, qdt):
    k, v, sk, sv = _data(hd + T, H, T, hd)
    c = Cache(k, v, kbits, vbits, sk, sv)
    q = synth.normal_f16(T, 6, H * G * hd).reshape(H * G, hd).astype(qdt)
    gpu = c.attend(q)
    orc, bound = c.oracle(q)
    _check(gpu, orc, bound, f"hd={hd} H={H} G={G} T={T} K{kbits}V{vbits}")


@pytest.mark.parametrize("kbits,vbits", [(3, 3), (4, 3)])
def test_attn_beta_codebook(kbits, vbits):
    """K and V block-32 codebooks solved for the exact marginal of a 32-long unit block."""
    k, v, sk, sv = _data(31, 2, 1500, 128)
    c = Cache(k, v, kbits, vbits, sk, sv, codebook="beta")
    q = synth.normal_f16(31, 6, 8 * 128).reshape(8, 128)
    gpu = c.attend(q)
    orc, bound = c.oracle(q)
    _check(gpu, orc, bound, f"beta codebook K{kbits}V{vbits}")


def test_attn_explicit_scale():
    k, v, sk, sv = _data(7, 2, 700, 128)
    c = Cache(k, v, 3, 3, sk, sv)
    q = synth.normal_f16(7, 6, 4 * 128).reshape(4, 128)
    gpu = c.attend(q, scale=0.02)
    orc, bound = c.oracle(q, scale=0.02)
    _check(gpu, orc, bound, "scale=0.02")


def test_attn_peaked_softmax():
    """One key aligned with a large query dominates: the output is close to that token's value."""
    hd, T = 128, 4096
    k, v, sk, sv = _data(11, 1, T, hd)
    q = np.zeros((2, hd), dtype=np.float32)
    q[0] = k[0, 1234].astype(np.float32) * 4.0
    q[1] = -q[0]
    c = Cache(k, v, 4, 4, sk, sv)
    gpu = c.attend(q)
    orc, bound = c.oracle(q)
    _check(gpu, orc, bound, "peaked")


def test_attn_zero_tokens_is_noop():
    k, v, sk, sv = _data(1, 1, 32, 128)
    c = Cache(k, v, 3, 3, sk, sv)
    out = torch.full((4, 128), 5.0, dtype=torch.float32, device=DEV)
    q = torch.zeros((4, 128), dtype=torch.float16, device=DEV)
    tq.tq_decode_attn(c.kq, c.vq, q, tq.TQ_F16, 4, 1, 0, c.kc, c.kn, c.vc, c.vn, 0.0, out, None, 0)
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)


def test_attn_rejects_bad_args():
    k, v, sk, sv = _data(1, 1, 32, 128)
    c = Cache(k, v, 3, 3, sk, sv)
    q = torch.zeros((4, 128), dtype=torch.float16, device=DEV)
    out = torch.empty((4, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(tq.TqError) as e:  # no workspace
        tq.tq_decode_attn(c.kq, c.vq, q, tq.TQ_F16, 4, 1, 32, c.kc, c.kn, c.vc, c.vn, 0.0, out, None, 0)
    assert e.value.status == 3
    with pytest.raises(tq.TqError) as e:  # 4 query heads over 3 KV heads
        tq.tq_decode_attn(c.kq, c.vq, q, tq.TQ_F16, 4, 3, 32, c.kc, c.kn, c.vc, c.vn, 0.0, out, None, 0)
    assert e.value.status == 1
    v8 = tq.Quantizer(128, 32, 8, sv)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    with pytest.raises(tq.TqError) as e:  # 8-bit values are not an attention format
        tq.tq_decode_attn(c.kq, v8, q, tq.TQ_F16, 4, 1, 32, c.kc, c.kn, c.vc, c.vn, 0.0, out, ws, 1 << 20)
    assert e.value.status == 2


def test_attn_full_size_sampled():
    """head_dim 256, 4 KV heads, 16 query heads, 131072 tokens, 3-bit K and V: the full call on the GPU,
    the oracle on every KV head (all 16 query heads over all 131072 tokens)."""
    from synth.workloads import decode_cache

    w = decode_cache()
    c = Cache(w["k"][0], w["v"][0], 3, 3, w["signs_k"], w["signs_v"])
    del w["k"], w["v"]
    gpu = c.attend(w["q"])
    for g in range(c.H):
        orc, bound = c.oracle(w["q"], kv_heads=[g])
        _check(gpu[4 * g:4 * g + 4], orc, bound, f"131072 tokens, KV head {g}")


def test_attn_full_size_k8v4_sampled():
    """The same 131072-token cache with 8-bit keys and 4-bit values (the asymmetric allocation); the
    oracle on every KV head."""
    from synth.workloads import decode_cache

    w = decode_cache()
    c = Cache(w["k"][0], w["v"][0], 8, 4, w["signs_k"], w["signs_v"])
    del w["k"], w["v"]
    gpu = c.attend(w["q"])
    for g in range(c.H):
        orc, bound = c.oracle(w["q"], kv_heads=[g])
        _check(gpu[4 * g:4 * g + 4], orc, bound, f"131072 tokens, K8V4, KV head {g}")
