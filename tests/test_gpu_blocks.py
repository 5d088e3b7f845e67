"""GPU parity of the fork's record format (TQ_BLOCKS) against the oracle, through the C ABI.

Records are 32-value blocks: the fp16 norm of the block's unit, then the
block's packed codes ([Fork] "GGML Types", "How it works").  The fork's own
layout is dt = 128 (128-value chunks, norm copied into each of the chunk's
four records); other unit lengths and bit widths use the same record rule.
Row counts make the last wave partial (its records are written one by one)
and cover several full waves (written as 16-byte chunks through LDS).
"""
import numpy as np
import pytest

import synth
from oracle import Codebook, dequantize_blocks, from_blocks, quantize, record_bytes, to_blocks
from tests.parity import assert_band_rate, check_codes, check_decoded_f16, check_decoded_f32, check_norms

torch = pytest.importorskip("torch")
import kv_cache_vector_amd as tq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _encode(qz, x_np, ld=None):
    n_rows, hd = x_np.shape
    ld = hd if ld is None else ld
    host = np.zeros((n_rows, ld), dtype=x_np.dtype)
    host[:, :hd] = x_np
    x = torch.from_numpy(host).to(DEV)
    n_rec = n_rows * hd // 32
    R = qz.record_bytes()
    buf = torch.full((n_rec * R + 64,), 0xA5, dtype=torch.uint8, device=DEV)  # guard bytes after the records
    tq.tq_quantize(qz, x, n_rows, ld, buf, None)
    torch.cuda.synchronize()
    out = buf.cpu().numpy()
    assert np.all(out[n_rec * R:] == 0xA5), "records written past the end"
    return out[:n_rec * R].reshape(n_rec, R)


def _decode(qz, records, n_rows, y_dtype, ld=None):
    hd = qz.cfg.head_dim
    ld = hd if ld is None else ld
    rec = torch.from_numpy(np.ascontiguousarray(records).reshape(-1)).to(DEV)
    y = torch.full((n_rows, ld), 1234.0, dtype=torch.float32 if y_dtype == tq.TQ_F32 else torch.float16, device=DEV)
    tq.tq_dequantize(qz, rec, None, None, None, n_rows, y, y_dtype, ld)
    torch.cuda.synchronize()
    out = y.cpu().numpy()
    if ld > hd:
        assert np.all(out[:, hd:] == 1234.0), "decode wrote outside the rows"
    return out[:, :hd]


def _case(x, dt, bits, seed, nc=False, ld=None, codebook="gaussian", band=True):
    n_rows, hd = x.shape
    signs = synth.signs(seed, 2, dt)
    x_dtype = tq.TQ_F32 if x.dtype == np.float32 else tq.TQ_F16
    qz = tq.Quantizer(hd, dt, bits, signs, flags=tq.TQ_BLOCKS | (tq.TQ_NORM_CORRECT if nc else 0), x_dtype=x_dtype,
                      codebook=codebook)
    cb = Codebook.build_beta(bits, dt) if codebook == "beta" else Codebook.build(bits, dt)
    rec = _encode(qz, x, ld)
    orc = quantize(x.astype(np.float64), signs, cb)
    codes, bn = from_blocks(rec, bits, dt)
    stats = check_codes(codes, orc, cb, bits, dt)
    if band:  # structured rows (zero units) sit on an edge by construction
        assert_band_rate(stats, cb)
    # every record of a unit carries the unit's norm
    for b in range(dt // 32):
        stats.update(check_norms(bn[:, b], orc["norms"]))
    np.testing.assert_array_equal(bn, np.repeat(bn[:, :1], dt // 32, axis=1))
    ref = dequantize_blocks(rec, signs, cb, nc=nc).reshape(n_rows, hd)
    norms_rows = bn[:, 0].astype(np.float64)
    for yt in (tq.TQ_F32, tq.TQ_F16):
        y = _decode(qz, rec, n_rows, yt, ld)
        yy, rr = y.reshape(-1, dt), ref.reshape(-1, dt)
        if yt == tq.TQ_F32:
            stats["decode_err"] = check_decoded_f32(yy, rr, norms_rows, dt)
        else:
            stats["f16_ulp_off"] = check_decoded_f16(yy, rr, norms_rows, dt)
    return stats, qz, rec, orc, signs, cb


@pytest.mark.parametrize("hd,bits", [(128, 3), (128, 4), (256, 3), (256, 4), (128, 1), (128, 2), (128, 8)])
def test_fork_layout_chunk128(hd, bits):
    """dt = 128: the fork's turbo layout (a 256 head is two chunks, each with its own norm)."""
    n_rows = 333  # 333 * hd/32 records: full waves plus a partial one
    x = synth.kv_tensor(hd + bits, 1, 1, 0, n_rows, hd).reshape(n_rows, hd)
    stats, *_ = _case(x, 128, bits, seed=hd + 7 * bits, nc=bits == 3)
    print(stats)


@pytest.mark.parametrize("dt,bits", [(32, 3), (32, 4), (64, 2), (256, 3), (32, 8)])
def test_records_other_units(dt, bits):
    hd, n_rows = 256, 201
    x = synth.kv_tensor(dt * bits, 1, 1, 1, n_rows, hd).reshape(n_rows, hd)
    stats, *_ = _case(x, dt, bits, seed=dt + bits)
    print(stats)


def test_records_f32_strided_beta():
    """fp32 rows with a padded stride, the Beta codebook the fork solves for (d = 128)."""
    hd, n_rows = 256, 150
    x = synth.normal_f32(12, 0, n_rows * hd).reshape(n_rows, hd) * 2.0
    stats, *_ = _case(x, 128, 3, seed=12, ld=hd + 8, codebook="beta")
    print(stats)


def test_records_decode_uses_each_copy():
    """Decode scales each block by the norm its own record carries (records edited on the host)."""
    n_rows = 70
    x = synth.kv_tensor(21, 1, 1, 0, n_rows, 128).reshape(n_rows, 128)
    _, qz, rec, orc, signs, cb = _case(x, 128, 4, seed=21)
    rec2 = rec.copy()
    rng = np.random.default_rng(21)
    scale = rng.uniform(0.5, 2.0, size=len(rec2)).astype(np.float16)
    new = (rec2[:, :2].copy().view("<f2")[:, 0] * scale).astype("<f2")
    rec2[:, :2] = new.view(np.uint8).reshape(-1, 2)
    y = _decode(qz, rec2, n_rows, tq.TQ_F32)
    ref = dequantize_blocks(rec2, signs, cb).reshape(n_rows, 128)
    bn = from_blocks(rec2, 4, 128)[1].astype(np.float64)
    err = np.abs(y.astype(np.float64) - ref).reshape(-1, 32) / np.maximum(bn.reshape(-1, 1), 1e-30)
    assert err.max() <= 1e-5


def test_records_edge_cases():
    """One row, zero rows inside a batch, a row count that fills exactly one wave."""
    for n_rows in (1, 16, 17):
        x = synth.kv_tensor(30 + n_rows, 1, 1, 0, n_rows, 128).reshape(n_rows, 128)
        x[n_rows // 2] = 0
        stats, qz, rec, *_ = _case(x, 128, 3, seed=30, band=False)
        assert np.all(from_blocks(rec, 3, 128)[1][n_rows // 2] == 0)
    qz = tq.Quantizer(128, 128, 3, np.ones(128), flags=tq.TQ_BLOCKS)
    buf = torch.full((64,), 7, dtype=torch.uint8, device=DEV)
    tq.tq_quantize(qz, torch.zeros((1, 128), dtype=torch.float16, device=DEV), 0, 128, buf, None)
    torch.cuda.synchronize()
    assert torch.all(buf == 7)


def test_records_full_size_sampled():
    """The fork-layout workload at full size (36 x 8 x 16384 vectors of 128, turbo3): 100000 sampled rows
    (12.8 M coordinates, in-band count held to the literal 1e-5 bound)."""
    from synth.workloads import qwen3_8b_kv_chunk128

    w = qwen3_8b_kv_chunk128()
    k = w["k"].reshape(-1, 128)
    rows = k.shape[0]
    qz = tq.Quantizer(128, 128, 3, w["signs_k"], flags=tq.TQ_BLOCKS, codebook="beta")
    xt = torch.from_numpy(k).to(DEV)
    rec = torch.empty(rows * 4 * 14, dtype=torch.uint8, device=DEV)
    tq.tq_quantize(qz, xt, rows, 128, rec, None)
    y = torch.empty((rows, 128), dtype=torch.float16, device=DEV)
    tq.tq_dequantize(qz, rec, None, None, None, rows, y, tq.TQ_F16, 128)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    sample = np.unique(np.concatenate([rng.choice(rows, 100000, replace=False), [0, rows - 1]]))
    r = rec.view(rows, 56)[torch.from_numpy(sample).to(DEV)].cpu().numpy().reshape(-1, 14)
    cb = Codebook.build_beta(3, 128)
    orc = quantize(k[sample].astype(np.float64), w["signs_k"], cb)
    codes, bn = from_blocks(r, 3, 128)
    stats = check_codes(codes, orc, cb, 3, 128)
    assert_band_rate(stats, cb, literal=True)
    check_norms(bn[:, 0], orc["norms"])
    ref = dequantize_blocks(r, w["signs_k"], cb)
    check_decoded_f16(y[torch.from_numpy(sample).to(DEV)].cpu().numpy(), ref, bn[:, 0], 128)
    print(stats)
