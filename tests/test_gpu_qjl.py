"""GPU parity of the QJL stage (encode with the residual sketch, dequantize with
the QJL correction) against the oracle, through the C ABI."""
import numpy as np
import pytest

import synth
from oracle import Codebook, code_to_index, dequantize, quantize, unpack_codes
from tests.parity import (BAND, assert_band_rate, assert_sign_band_rate, check_codes, check_decoded_f32,
                          check_norms, check_sign_bits, edge_distance)

torch = pytest.importorskip("torch")
import kv_cache_vector_amd as tq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _encode(keys, dt, bits, m, seed, nc=False, codebook="gaussian"):
    n = keys.shape[0]
    signs = synth.signs(seed, 2, dt)
    S = synth.gaussian_matrix(seed + 1, 0, m, dt)
    qz = tq.Quantizer(dt, dt, bits, signs, flags=tq.TQ_QJL | (tq.TQ_NORM_CORRECT if nc else 0), qjl_m=m,
                      codebook=codebook)
    params = torch.empty(tq.tq_qjl_params_size(m, dt), dtype=torch.uint8, device=DEV)
    tq.tq_qjl_prepare(qz, S, params)
    x = torch.from_numpy(keys).to(DEV)
    codes = torch.full((n * dt * bits // 8,), 0x5A, dtype=torch.uint8, device=DEV)
    norms = torch.empty(n, dtype=torch.float16, device=DEV)
    sbits = torch.full((n * m // 8,), 0x33, dtype=torch.uint8, device=DEV)
    rnorm = torch.empty(n, dtype=torch.float16, device=DEV)
    tq.tq_quantize(qz, x, n, dt, codes, norms, sbits, rnorm)
    torch.cuda.synchronize()
    return qz, signs, S, codes, norms, sbits, rnorm


@pytest.mark.parametrize("dt,m,bits,codebook", [(128, 128, 2, "gaussian"), (128, 64, 1, "gaussian"),
                                                 (64, 128, 3, "gaussian"), (64, 64, 2, "gaussian"),
                                                 (128, 96, 2, "gaussian"), (128, 32, 2, "gaussian"),
                                                 (128, 128, 3, "beta"),
                                                 (64, 64, 2, "beta"),
                                                 (32, 256, 2, "gaussian"),   # one lane per unit, 32 KiB of S~
                                                 (256, 64, 3, "gaussian"),   # eight lanes per unit, 64 KiB of S~
                                                 (256, 32, 4, "gaussian")])
def test_qjl_encode_decode(dt, m, bits, codebook):
    n = 1000  # several workgroups plus a ragged tail
    keys = synth.kv_tensor(dt + m + bits, 1, 1, 0, n, dt, n_outliers=0).reshape(n, dt)
    qz, signs, S, codes, norms, sbits, rnorm = _encode(keys, dt, bits, m, seed=dt + bits, codebook=codebook)
    cb = Codebook.build_beta(bits, dt) if codebook == "beta" else Codebook.build(bits, dt)
    orc = quantize(keys.astype(np.float64), signs, cb, S=S)
    codes_np, norms_np = codes.cpu().numpy(), norms.cpu().numpy()
    stats = check_codes(codes_np, orc, cb, bits, dt)
    assert_band_rate(stats, cb)
    check_norms(norms_np, orc["norms"])
    # sign bits and residual norms: compare units whose indices matched exactly
    same = np.all(unpack_codes(codes_np.reshape(n, -1), bits, dt) == unpack_codes(orc["codes"], bits, dt), axis=1)
    sb = sbits.cpu().numpy().reshape(n, m // 8)
    sub = {k: v[same] for k, v in orc.items()}
    st = check_sign_bits(sb[same], sub, m)
    assert_sign_band_rate(st)
    check_norms(rnorm.cpu().numpy()[same], orc["rho"][same])
    print(stats, st)
    # dequantize with the QJL correction (fp32 output), oracle on the GPU's own codes
    for nc in (False, True):
        qz.cfg.flags = tq.TQ_QJL | (tq.TQ_NORM_CORRECT if nc else 0)
        y = torch.empty((n, dt), dtype=torch.float32, device=DEV)
        tq.tq_dequantize(qz, codes, norms, sbits, rnorm, n, y, tq.TQ_F32, dt)
        torch.cuda.synchronize()
        ref = dequantize(codes_np.reshape(n, -1), norms_np, signs, cb, nc=nc, qjl_bits=sb, rho=rnorm.cpu().numpy(),
                         S=S)
        check_decoded_f32(y.cpu().numpy(), ref, norms_np, dt)


def test_qjl_keys_full_size_sampled():
    """65536 keys x 128 fp16, 2-bit MSE + 1-bit QJL, m = 128, S from seed 1: the whole set on the GPU and
    in the oracle (8.4 M coordinates and 8.4 M sign bits; in-band counts held to the literal 1e-5 bound)."""
    from synth.workloads import qjl_keys

    w = qjl_keys()
    keys = w["keys"]
    n, dt, bits, m = keys.shape[0], 128, 2, 128
    qz = tq.Quantizer(dt, dt, bits, w["signs"], flags=tq.TQ_QJL, qjl_m=m)
    params = torch.empty(tq.tq_qjl_params_size(m, dt), dtype=torch.uint8, device=DEV)
    tq.tq_qjl_prepare(qz, w["S"], params)
    x = torch.from_numpy(keys).to(DEV)
    codes = torch.empty(n * 32, dtype=torch.uint8, device=DEV)
    norms = torch.empty(n, dtype=torch.float16, device=DEV)
    sbits = torch.empty(n * 16, dtype=torch.uint8, device=DEV)
    rnorm = torch.empty(n, dtype=torch.float16, device=DEV)
    tq.tq_quantize(qz, x, n, dt, codes, norms, sbits, rnorm)
    torch.cuda.synchronize()
    cb = Codebook.build(bits, dt)
    orc = quantize(keys.astype(np.float64), w["signs"], cb, S=w["S"])
    c = codes.cpu().numpy().reshape(n, 32)
    st = check_codes(c, orc, cb, bits, dt)
    assert_band_rate(st, cb, literal=True)
    check_norms(norms.cpu().numpy(), orc["norms"])
    # sign bits of the keys whose codes match the oracle's (an in-band code flip changes the residual)
    same = np.all(unpack_codes(c, bits, dt) == unpack_codes(orc["codes"], bits, dt), axis=1)
    sb = check_sign_bits(sbits.cpu().numpy().reshape(n, 16)[same], {k: v[same] for k, v in orc.items()}, m)
    assert_sign_band_rate(sb, literal=True)
    check_norms(rnorm.cpu().numpy()[same], orc["rho"][same])
    print(st, sb)


@pytest.mark.parametrize("bits", [3, 4])
def test_qjl_encode_head128_f32_zero_keys(bits):
    """head_dim 128 with fp32 keys and fp32 norms at 3 and 4 bits, including all-zero keys: codes,
    norms, sign bits and residual norms against the oracle; zero keys store n = 0, the code just
    below zero for every coordinate, rho of the unit-less residual, and decode to zero."""
    dt, m, n = 128, 128, 333
    keys = synth.kv_tensor(bits + 40, 1, 1, 0, n, dt, n_outliers=2).reshape(n, dt).astype(np.float32)
    keys[[0, 17, 200, n - 1]] = 0.0
    signs = synth.signs(bits + 40, 2, dt)
    S = synth.gaussian_matrix(bits + 41, 0, m, dt)
    qz = tq.Quantizer(dt, dt, bits, signs, flags=tq.TQ_QJL, qjl_m=m, x_dtype=tq.TQ_F32, norm_dtype=tq.TQ_F32)
    params = torch.empty(tq.tq_qjl_params_size(m, dt), dtype=torch.uint8, device=DEV)
    tq.tq_qjl_prepare(qz, S, params)
    x = torch.from_numpy(keys).to(DEV)
    codes = torch.full((n * dt * bits // 8,), 0x5A, dtype=torch.uint8, device=DEV)
    norms = torch.full((n,), -1.0, dtype=torch.float32, device=DEV)
    sbits = torch.full((n * m // 8,), 0x33, dtype=torch.uint8, device=DEV)
    rnorm = torch.empty(n, dtype=torch.float16, device=DEV)
    tq.tq_quantize(qz, x, n, dt, codes, norms, sbits, rnorm)
    torch.cuda.synchronize()
    cb = Codebook.build(bits, dt)
    orc = quantize(keys.astype(np.float64), signs, cb, norm_dtype=np.float32, S=S)
    codes_np, norms_np = codes.cpu().numpy(), norms.cpu().numpy()
    check_codes(codes_np, orc, cb, bits, dt)
    check_norms(norms_np, orc["norms"])
    assert np.all(norms_np[[0, 17, 200, n - 1]] == 0.0)
    same = np.all(unpack_codes(codes_np.reshape(n, -1), bits, dt) == unpack_codes(orc["codes"], bits, dt), axis=1)
    assert same[[0, 17, 200, n - 1]].all(), "zero keys must take the code just below zero everywhere"
    sb = sbits.cpu().numpy().reshape(n, m // 8)
    check_sign_bits(sb[same], {k: v[same] for k, v in orc.items()}, m)
    check_norms(rnorm.cpu().numpy()[same], orc["rho"][same])
    y = torch.empty((n, dt), dtype=torch.float32, device=DEV)
    tq.tq_dequantize(qz, codes, norms, sbits, rnorm, n, y, tq.TQ_F32, dt)
    torch.cuda.synchronize()
    assert np.all(y.cpu().numpy()[[0, 17, 200, n - 1]] == 0.0)
