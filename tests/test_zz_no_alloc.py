"""tq_decode_attn_noalloc (no workspace: the partials live in the library's static per-device scratch)
against tq_decode_attn with a caller workspace, through the C ABI.

Both run the same kernels with the same launch shape, so the outputs must be identical bit for bit.
Two calls in a row on one stream, the second with a smaller input (the scratch keeps the first
call's contents), then calls the scratch cannot hold, which must be rejected before any launch.
"""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
import kv_cache_vector_amd as tq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cache(seed, H, T, hd, kbits, vbits):
    k = synth.kv_tensor(seed, 1, H, 0, T, hd)[0].reshape(H * T, hd)
    v = synth.kv_tensor(seed, 1, H, 1, T, hd)[0].reshape(H * T, hd)
    kq = tq.Quantizer(hd, 32, kbits, synth.signs(seed, 2, 32))
    vq = tq.Quantizer(hd, 32, vbits, synth.signs(seed, 3, 32))
    units = H * T * hd // 32
    out = []
    for qz, x, b in ((kq, k, kbits), (vq, v, vbits)):
        codes = torch.empty(units * 4 * b, dtype=torch.uint8, device=DEV)
        norms = torch.empty(units, dtype=torch.float16, device=DEV)
        tq.tq_quantize(qz, torch.from_numpy(x).to(DEV), H * T, hd, codes, norms)
        out += [codes, norms]
    return kq, vq, out


def _both(kq, vq, planes, q, H, T):
    hq, hd = q.shape
    qt = torch.from_numpy(q).to(DEV)
    ref = torch.full((hq, hd), -3.0, dtype=torch.float32, device=DEV)
    wsb = tq.tq_workspace_size(tq.TQ_OP_DECODE_ATTN, kq, hq, H, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    tq.tq_decode_attn(kq, vq, qt, tq.TQ_F16, hq, H, T, *planes, 0.0, ref, ws, wsb)
    got = torch.full((hq, hd), -5.0, dtype=torch.float32, device=DEV)
    tq.tq_decode_attn_noalloc(kq, vq, qt, tq.TQ_F16, hq, H, T, *planes, 0.0, got)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy(), wsb


def test_noalloc_matches_workspace_call_twice():
    """The 131072-token, 4-KV-head, head_dim-256 turbo3 decode (16 query heads), then a smaller call
    (2 KV heads x 3000 tokens, head_dim 128, 8 query heads, 4-bit K / 3-bit V) on the same scratch."""
    kq, vq, planes = _cache(0, 4, 131072, 256, 3, 3)
    q = synth.normal_f16(0, 6, 16 * 256).reshape(16, 256)
    ref, got, wsb = _both(kq, vq, planes, q, 4, 131072)
    assert wsb <= 16 << 20
    assert np.all(np.isfinite(ref))
    np.testing.assert_array_equal(got, ref)
    del planes
    kq, vq, planes = _cache(5, 2, 3000, 128, 4, 3)
    q = synth.normal_f16(5, 6, 8 * 128).reshape(8, 128)
    ref2, got2, wsb2 = _both(kq, vq, planes, q, 2, 3000)
    assert wsb2 < wsb
    np.testing.assert_array_equal(got2, ref2)


def test_noalloc_rejects_oversize_and_bad_args():
    """Calls whose partials exceed the 16 MiB scratch, or with bad arguments, launch nothing and return
    an error; n_tokens = 0 leaves out untouched."""
    kq, vq, planes = _cache(1, 1, 64, 256, 3, 3)
    q = torch.zeros((16, 256), dtype=torch.float16, device=DEV)
    out = torch.full((16, 256), 9.0, dtype=torch.float32, device=DEV)
    with pytest.raises(tq.TqError) as e:  # 8.4 M tokens x 1 KV head x 16 query heads at head_dim 256
        tq.tq_decode_attn_noalloc(kq, vq, q, tq.TQ_F16, 16, 1, 8_400_000, *planes, 0.0, out)
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED and "scratch" in str(e.value)
    with pytest.raises(tq.TqError) as e:  # 16 query heads over 3 KV heads
        tq.tq_decode_attn_noalloc(kq, vq, q, tq.TQ_F16, 16, 3, 64, *planes, 0.0, out)
    assert e.value.status == tq.TQ_ERR_INVALID_ARG
    tq.tq_decode_attn_noalloc(kq, vq, q, tq.TQ_F16, 16, 1, 0, *planes, 0.0, out)
    torch.cuda.synchronize()
    assert torch.all(out == 9.0)
