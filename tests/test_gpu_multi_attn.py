"""GPU parity of tq_multi_attn (several query tokens over one quantized cache, optionally causal)
against the oracle's multi_attention run on the GPU's own codes and norms.

The tolerance is the one derived for tq_decode_attn (see test_gpu_attn.py), evaluated per
(query token, head) row over the tokens that row sees.  KV heads with up to 16 rows run the decode
kernel; more rows run the prefill kernel in groups of 128 (both are covered below).
"""
import math

import numpy as np
import pytest

import synth
from oracle import Codebook, dequantize, multi_attention
from oracle.quantizer import code_to_index, unpack_codes
from test_gpu_attn import U16, Cache, _check, _data

torch = pytest.importorskip("torch")
import kv_cache_vector_amd as tq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu_multi(c: Cache, q, causal, scale=0.0):
    n_q, hq = q.shape[0], q.shape[1]
    qt = torch.from_numpy(np.ascontiguousarray(q)).to(DEV)
    qtype = tq.TQ_F32 if q.dtype == np.float32 else tq.TQ_F16
    out = torch.full((n_q * hq + 1, c.hd), -7.0, dtype=torch.float32, device=DEV)  # one guard row
    wsb = tq.tq_workspace_size(tq.TQ_OP_MULTI_ATTN, c.kq, n_q * hq, c.H, c.T)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    tq.tq_multi_attn(c.kq, c.vq, qt, qtype, n_q, hq, c.H, c.T, c.kc, c.kn, c.vc, c.vn, causal, scale, out, ws, wsb)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[n_q * hq] == -7.0), "output written past the last row"
    return o[:n_q * hq].reshape(n_q, hq, c.hd)


def oracle_multi(c: Cache, q, causal):
    """Oracle output and the per-row error bound of the decode kernel's arithmetic."""
    kc, kn, vc, vn = c.host()
    build = Codebook.build_beta if c.codebook == "beta" else Codebook.build
    kcb, vcb = build(c.kbits, 32), build(c.vbits, 32)
    q64 = q.astype(np.float64)
    out = multi_attention(q64, kc, kn, vc, vn, c.signs_k, c.signs_v, kcb, vcb, c.H, c.T, c.hd, causal=causal)
    H, T, hd, nb = c.H, c.T, c.hd, c.hd // 32
    n_q, hq = q.shape[0], q.shape[1]
    G = hq // H
    scale = 1.0 / math.sqrt(hd)
    k = dequantize(kc, kn, c.signs_k, kcb).reshape(H, T, hd)
    v = dequantize(vc, vn, c.signs_v, vcb).reshape(H, T, hd)
    cv = np.abs(vcb.unit_levels[code_to_index(unpack_codes(vc, c.vbits, 32), c.vbits)]).reshape(H, T, nb, 32)
    ck = kcb.unit_levels[code_to_index(unpack_codes(kc, c.kbits, 32), c.kbits)]
    ckn = np.linalg.norm(ck, axis=1).reshape(H, T, nb)
    knn = kn.astype(np.float64).reshape(H, T, nb)
    vnn = vn.astype(np.float64).reshape(H, T, nb)
    bound = np.zeros(out.shape)
    for i in range(n_q):
        t = T - n_q + i + 1 if causal else T
        for h in range(hq):
            g = h // G
            s = k[g, :t] @ q64[i, h] * scale
            p = np.exp(s - s.max())
            L = p.sum()
            qb = np.linalg.norm(q64[i, h].reshape(nb, 32), axis=1)
            eps = 4e-6 * scale * np.max((knn[g, :t] * ckn[g, :t]) @ qb) / math.sqrt(32) + 1e-6
            for b in range(nb):
                E = 2 * U16 * ((p * vnn[g, :t, b]) @ cv[g, :t, b]) + 2.0 ** -25 * cv[g, :t, b].sum(axis=0)
                vmax = np.abs(v[g, :t, 32 * b:32 * (b + 1)]).max()
                bound[i, h, 32 * b:32 * (b + 1)] = 1.25 * (np.linalg.norm(E) / (math.sqrt(32) * L) + 2 * eps * vmax)
    return out, bound + 1e-7


@pytest.mark.parametrize("hd,H,G,T,n_q,causal,kbits,vbits,qdt", [
    (128, 2, 4, 600, 4, True, 3, 3, np.float16),     # 16 rows per KV head: one row group
    (256, 1, 4, 300, 5, True, 4, 3, np.float32),     # 20 rows: a full and a partial row group
    (128, 2, 2, 1000, 9, False, 3, 4, np.float16),   # no mask, 18 rows per KV head
    (256, 4, 4, 200, 64, True, 3, 3, np.float16),    # a 64-token chunk: 16 row groups, masks crossing tiles
    (128, 1, 8, 130, 3, True, 8, 4, np.float16),     # 8-bit keys
    (128, 3, 1, 70, 70, True, 4, 4, np.float32),     # chunk as long as the cache: row 0 sees one token
    (256, 2, 4, 1500, 128, True, 3, 3, np.float16),  # 512 rows per KV head: four 128-row prefill groups
    (256, 1, 8, 700, 40, False, 8, 4, np.float32),   # 320 rows, a partial prefill group, 8-bit keys
])
def test_multi_attn_matrix(hd, H, G, T, n_q, causal, kbits, vbits, qdt):
    k, v, sk, sv = _data(hd + T + n_q, H, T, hd)
    c = Cache(k, v, kbits, vbits, sk, sv)
    q = synth.normal_f16(T + n_q, 6, n_q * H * G * hd).reshape(n_q, H * G, hd).astype(qdt)
    gpu = gpu_multi(c, q, causal)
    orc, bound = oracle_multi(c, q, causal)
    _check(gpu.reshape(-1, hd), orc.reshape(-1, hd), bound.reshape(-1, hd),
           f"hd={hd} H={H} G={G} T={T} n_q={n_q} causal={causal} K{kbits}V{vbits}")


def test_multi_attn_one_query_equals_decode():
    """n_q = 1 without a mask is the decode call, bit for bit (same kernels, same partials)."""
    k, v, sk, sv = _data(3, 2, 900, 256)
    c = Cache(k, v, 3, 3, sk, sv)
    q = synth.normal_f16(3, 6, 8 * 256).reshape(1, 8, 256)
    np.testing.assert_array_equal(gpu_multi(c, q, False)[0], c.attend(q[0]))


def test_multi_attn_rejects_bad_args():
    k, v, sk, sv = _data(2, 1, 32, 128)
    c = Cache(k, v, 3, 3, sk, sv)
    q = torch.zeros((40, 4, 128), dtype=torch.float16, device=DEV)
    out = torch.empty((40, 4, 128), dtype=torch.float32, device=DEV)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    with pytest.raises(tq.TqError) as e:  # a causal chunk longer than the cache
        tq.tq_multi_attn(c.kq, c.vq, q, tq.TQ_F16, 40, 4, 1, 32, c.kc, c.kn, c.vc, c.vn, True, 0.0, out, ws, 1 << 20)
    assert e.value.status == 1
    with pytest.raises(tq.TqError) as e:  # workspace too small
        tq.tq_multi_attn(c.kq, c.vq, q, tq.TQ_F16, 8, 4, 1, 32, c.kc, c.kn, c.vc, c.vn, True, 0.0, out, ws, 256)
    assert e.value.status == 3
    out.fill_(5.0)
    tq.tq_multi_attn(c.kq, c.vq, q, tq.TQ_F16, 0, 4, 1, 32, c.kc, c.kn, c.vc, c.vn, True, 0.0, out, None, 0)
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)
