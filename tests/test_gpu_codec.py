"""GPU parity of tq_quantize / tq_dequantize (no QJL) against the oracle.

Every case runs the HIP path through the C ABI and the oracle on the same
seeded inputs; decode parity runs the oracle on the GPU's own codes and norms.
Sizes span several workgroups plus a ragged tail; the matrix covers every
transform length, bit width, input/norm dtype and output dtype.
"""
import math

import numpy as np
import pytest

import synth
from oracle import Codebook, dequantize, hadamard_matrix, quantize
from tests.parity import assert_band_rate, check_codes, check_decoded_f16, check_decoded_f32, check_norms

torch = pytest.importorskip("torch")
import kv_cache_vector_amd as tq  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run_encode(qz, x_np, ld=None):
    """Encode rows x_np [n_rows, head_dim] (float16/float32) on the GPU; returns (codes, norms) as numpy."""
    cfg = qz.cfg
    n_rows, hd = x_np.shape
    ld = hd if ld is None else ld
    host = np.zeros((n_rows, ld), dtype=x_np.dtype)
    host[:, :hd] = x_np
    x = torch.from_numpy(host).to(DEV)
    units = n_rows * qz.units_per_row
    codes = torch.full((units * qz.code_bytes(),), 0xA5, dtype=torch.uint8, device=DEV)
    norms = torch.full((units,), -7.0, dtype=torch.float32 if cfg.norm_dtype == tq.TQ_F32 else torch.float16,
                       device=DEV)
    tq.tq_quantize(qz, x, n_rows, ld, codes, norms)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), norms.cpu().numpy()


def _run_decode(qz, codes_np, norms_np, n_rows, y_dtype, ld=None):
    hd = qz.cfg.head_dim
    ld = hd if ld is None else ld
    codes = torch.from_numpy(codes_np).to(DEV)
    norms = torch.from_numpy(norms_np).to(DEV)
    y = torch.full((n_rows, ld), 1234.0, dtype=torch.float32 if y_dtype == tq.TQ_F32 else torch.float16, device=DEV)
    tq.tq_dequantize(qz, codes, norms, None, None, n_rows, y, y_dtype, ld)
    torch.cuda.synchronize()
    out = y.cpu().numpy()
    if ld > hd:
        assert np.all(out[:, hd:] == 1234.0), "decode wrote outside the rows"
    return out[:, :hd]


def _roundtrip(x_np, dt, bits, seed, x_dtype, norm_dtype, nc=False, ld=None, y_dtypes=(tq.TQ_F32, tq.TQ_F16),
               codebook="gaussian"):
    n_rows, hd = x_np.shape
    signs = synth.signs(seed, 2, dt)
    qz = tq.Quantizer(hd, dt, bits, signs, flags=tq.TQ_NORM_CORRECT if nc else 0, x_dtype=x_dtype,
                      norm_dtype=norm_dtype, codebook=codebook)
    cb = Codebook.build_beta(bits, dt) if codebook == "beta" else Codebook.build(bits, dt)
    codes, norms = _run_encode(qz, x_np, ld)
    orc = quantize(x_np.astype(np.float64), signs, cb, norm_dtype=np.float32 if norm_dtype == tq.TQ_F32 else np.float16)
    stats = check_codes(codes, orc, cb, bits, dt)
    assert_band_rate(stats, cb)
    stats.update(check_norms(norms, orc["norms"]))
    ref = dequantize(codes.reshape(-1, dt * bits // 8), norms, signs, cb, nc=nc)
    for yt in y_dtypes:
        # the output rows keep the input's padding where that is a legal pitch for their element size
        # (a multiple of 16 bytes); fp16 rows otherwise take the next multiple of 8 elements
        ld_y = None if ld is None else (ld if yt == tq.TQ_F32 or ld % 8 == 0 else (ld + 7) // 8 * 8)
        y = _run_decode(qz, codes, norms, n_rows, yt, ld_y)
        if yt == tq.TQ_F32:
            stats["decode_err"] = check_decoded_f32(y, ref, norms, dt)
        else:
            stats["f16_ulp_off"] = check_decoded_f16(y, ref, norms, dt)
    return stats, codes, norms, orc


@pytest.mark.parametrize("dt", [32, 64, 128, 256])
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_matrix_f16(dt, bits):
    hd = max(dt, 128)
    n_rows = 333  # several workgroups of groups plus a ragged tail
    x = synth.kv_tensor(dt + bits, 1, 1, 0, n_rows, hd).reshape(n_rows, hd)
    stats, *_ = _roundtrip(x, dt, bits, seed=dt * 10 + bits, x_dtype=tq.TQ_F16, norm_dtype=tq.TQ_F16)
    print(stats)


@pytest.mark.parametrize("pad", [4, 8])
@pytest.mark.parametrize("dt", [32, 128])
@pytest.mark.parametrize("bits", [2, 3, 8])
def test_matrix_f32_strided(dt, bits, pad):
    """fp32 rows with a padded stride: pad 4 makes the row pitch 16 mod 32 bytes (1040 B), pad 8 a
    multiple of 32; encode reads and decode writes the rows in place."""
    hd, n_rows = 256, 129
    x = synth.normal_f32(7, 0, n_rows * hd).reshape(n_rows, hd) * 3.0
    stats, *_ = _roundtrip(x, dt, bits, seed=5, x_dtype=tq.TQ_F32, norm_dtype=tq.TQ_F32, ld=hd + pad)
    print(stats)


@pytest.mark.parametrize("pad", [8, 16])
@pytest.mark.parametrize("dt", [32, 64, 128])
@pytest.mark.parametrize("bits", [3, 4, 8])
def test_matrix_f16_strided(dt, bits, pad):
    """fp16 rows with a padded stride (row pitch hd + 8 or hd + 16 elements): the strided forms of the
    block-32 MFMA encode and decode (dt = 32, 3 and 4 bits; 8-bit decode takes the generic kernel) and
    of the generic kernels (dt = 64, 128), fp16 and fp32 output rows of the same stride."""
    hd, n_rows = 128, 333
    x = synth.kv_tensor(dt + bits + pad, 1, 1, 1, n_rows, hd).reshape(n_rows, hd)
    stats, *_ = _roundtrip(x, dt, bits, seed=dt + pad, x_dtype=tq.TQ_F16, norm_dtype=tq.TQ_F16, ld=hd + pad)
    print(stats)


@pytest.mark.parametrize("dt", [32, 128])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_beta_codebook(dt, bits):
    """Codebook solved for the exact marginal (tq_codebook_init_beta): the same kernels, other centroids."""
    hd, n_rows = 256, 301
    x = synth.kv_tensor(100 + dt + bits, 1, 1, 0, n_rows, hd).reshape(n_rows, hd)
    stats, *_ = _roundtrip(x, dt, bits, seed=3 * dt + bits, x_dtype=tq.TQ_F16, norm_dtype=tq.TQ_F16,
                           nc=bits == 3, codebook="beta")
    print(stats)


@pytest.mark.parametrize("dt,nc", [(32, True), (32, False), (128, True)])
def test_eight_bit_keys(dt, nc):
    """8-bit keys ([Scratch] §10, k8v4): block-32 and whole-vector units on a Qwen3-8B-shaped slice,
    with and without norm correction."""
    from synth.workloads import qwen3_8b_kv

    w = qwen3_8b_kv(layers=1, heads=2, tokens=700)
    x = w["k"].reshape(-1, 128)
    stats, codes, norms, orc = _roundtrip(x, dt, 8, seed=8, x_dtype=tq.TQ_F16, norm_dtype=tq.TQ_F16, nc=nc)
    # 255 cell edges put about 1e-4 of the coordinates inside the 1e-6 band (the 8-bit bar of
    # assert_band_rate, applied in _roundtrip); the codes that actually differ there stay rare
    print(stats)


def test_vectors_fp32_config_and_mse():
    """4096 x 128 fp32 N(0,1), 3 bits, one fp32 norm per vector; MSE of the unit vectors ~ 0.034."""
    from synth.workloads import vectors_fp32

    w = vectors_fp32()
    x = w["x"]
    qz = tq.Quantizer(128, 128, 3, w["signs"], x_dtype=tq.TQ_F32, norm_dtype=tq.TQ_F32)
    cb = Codebook.build(3, 128)
    codes, norms = _run_encode(qz, x)
    orc = quantize(x.astype(np.float64), w["signs"], cb, norm_dtype=np.float32)
    assert_band_rate(check_codes(codes, orc, cb, 3, 128), cb)
    check_norms(norms, orc["norms"])
    y = _run_decode(qz, codes, norms, len(x), tq.TQ_F32)
    ref = dequantize(codes.reshape(-1, 48), norms, w["signs"], cb)
    check_decoded_f32(y, ref, norms, 128)
    u = x.astype(np.float64) / np.linalg.norm(x.astype(np.float64), axis=1, keepdims=True)
    mse = np.mean(np.sum((u - y.astype(np.float64) / norms[:, None]) ** 2, axis=1))
    assert mse == pytest.approx(0.034, abs=0.001)


def test_norm_correction_llama_shape():
    """head_dim 64, 4 bits, per-vector norm + norm correction (small slice of the Llama-3.2-1B-shaped cache)."""
    from synth.workloads import llama_1b_kv

    w = llama_1b_kv(layers=2, heads=8, tokens=300)
    for half, s in (("k", "signs_k"), ("v", "signs_v")):
        x = w[half].reshape(-1, 64)
        stats, codes, norms, _ = _roundtrip(x, 64, 4, seed=0, x_dtype=tq.TQ_F16, norm_dtype=tq.TQ_F16, nc=True)
        qz = tq.Quantizer(64, 64, 4, w[s], flags=tq.TQ_NORM_CORRECT)
        y = _run_decode(qz, codes, norms, len(x), tq.TQ_F32)
        lengths = np.linalg.norm(y.astype(np.float64), axis=1)
        np.testing.assert_allclose(lengths, norms.astype(np.float64), rtol=2e-6)


@pytest.mark.parametrize("bits", [3, 4])
def test_block32_qwen_shape(bits):
    """Block-32 layout on a slice of the Qwen3-8B-shaped cache (outlier channels)."""
    from synth.workloads import qwen3_8b_kv

    w = qwen3_8b_kv(layers=2, heads=2, tokens=1000)
    for half, s in (("k", "signs_k"), ("v", "signs_v")):
        x = w[half].reshape(-1, 128)
        stats, *_ = _roundtrip(x, 32, bits, seed=0, x_dtype=tq.TQ_F16, norm_dtype=tq.TQ_F16)
        print(half, stats)


def test_edge_cases():
    hd, dt = 128, 32
    x = np.zeros((70, hd), dtype=np.float16)
    x[1] = 1.0  # all-equal
    x[2, 0] = 1.0  # one-hot
    x[3] = np.float16(6.0e-8)  # subnormal magnitude
    x[4] = np.float16(2000.0)  # large entries (norm 2.3e4, still a finite fp16)
    x[5, ::2] = -2.5
    x[6] = synth.normal_f16(1, 0, hd)
    x[7:] = synth.normal_f16(2, 0, 63 * hd).reshape(63, hd)
    for bits in (1, 2, 3, 4, 8):
        signs = synth.signs(9, 2, dt)
        qz = tq.Quantizer(hd, dt, bits, signs)
        cb = Codebook.build(bits, dt)
        codes, norms = _run_encode(qz, x)
        orc = quantize(x.astype(np.float64), signs, cb)
        # structured rows hit cell edges exactly: only neighbouring cells are accepted there
        check_codes(codes, orc, cb, bits, dt)
        check_norms(norms, orc["norms"])
        # a zero row stores norm 0 and decodes to zeros
        assert np.all(norms[:4] == 0)
        y = _run_decode(qz, codes, norms, len(x), tq.TQ_F32)
        assert np.all(y[0] == 0)
        ref = dequantize(codes.reshape(-1, dt * bits // 8), norms, signs, cb)
        check_decoded_f32(y, ref, norms, dt)


def test_empty_input_is_noop():
    qz = tq.Quantizer(128, 32, 3, np.ones(32))
    codes = torch.full((16,), 7, dtype=torch.uint8, device=DEV)
    norms = torch.zeros(4, dtype=torch.float16, device=DEV)
    x = torch.zeros((1, 128), dtype=torch.float16, device=DEV)
    tq.tq_quantize(qz, x, 0, 128, codes, norms)
    torch.cuda.synchronize()
    assert torch.all(codes == 7)


def test_deterministic_repeat():
    from synth.workloads import qwen3_8b_kv

    w = qwen3_8b_kv(layers=1, heads=2, tokens=2048)
    x = torch.from_numpy(w["k"].reshape(-1, 128)).to(DEV)
    qz = tq.Quantizer(128, 32, 3, w["signs_k"])
    n = x.shape[0]
    outs = []
    for _ in range(2):
        codes = torch.empty(n * 4 * 12, dtype=torch.uint8, device=DEV)
        norms = torch.empty(n * 4, dtype=torch.float16, device=DEV)
        tq.tq_quantize(qz, x, n, 128, codes, norms)
        outs.append((codes.clone(), norms.clone()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])



@pytest.mark.parametrize("bits,dt,records", [(b, dt, rec) for b in (2, 3, 4, 8)
                                              for dt, rec in ((32, False), (128, False), (128, True))
                                              if not (rec and b == 8)])  # records hold 1-4 bit codes
@pytest.mark.parametrize("pad", [0, 8])
def test_lone_waves_repeat(bits, dt, records, pad):
    """Regression test for missing wait states in hand-written instruction sequences (a VALU-written
    SGPR read too soon, an M0 write before an LDS-direct load, an MFMA result read before it is
    ready): such a read picks up a stale value only when nothing else runs between the two
    instructions, i.e. when a wave has its SIMD to itself.  64 rows = 256 groups = one workgroup of
    four waves on an otherwise idle GPU; the encode is repeated 64 times and every repeat must give
    the same bytes, and the first must match the oracle outside the edge band."""
    hd, n_rows = 128, 64
    x_np = synth.kv_tensor(7 * bits + dt + pad, 1, 1, 1, n_rows, hd).reshape(n_rows, hd)
    signs = synth.signs(bits + dt, 2, dt)
    flags = tq.TQ_BLOCKS if records else 0
    qz = tq.Quantizer(hd, dt, bits, signs, flags=flags, x_dtype=tq.TQ_F16, norm_dtype=tq.TQ_F16,
                      codebook="beta" if records else "gaussian")
    ld = hd + pad
    host = np.zeros((n_rows, ld), dtype=np.float16)
    host[:, :hd] = x_np
    x = torch.from_numpy(host).to(DEV)
    units = n_rows * qz.units_per_row
    nbytes = n_rows * (hd // 32) * qz.record_bytes() if records else units * qz.code_bytes()
    outs = []
    for _ in range(64):
        codes = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV)
        norms = None if records else torch.full((units,), -7.0, dtype=torch.float16, device=DEV)
        tq.tq_quantize(qz, x, n_rows, ld, codes, norms)
        outs.append((codes, norms))
    torch.cuda.synchronize()
    for codes, norms in outs[1:]:
        assert torch.equal(codes, outs[0][0])
        if norms is not None:
            assert torch.equal(norms, outs[0][1])
    if not records:
        cb = Codebook.build(bits, dt)
        orc = quantize(x_np.astype(np.float64), signs, cb, norm_dtype=np.float16)
        stats = check_codes(outs[0][0].cpu().numpy(), orc, cb, bits, dt)
        assert_band_rate(stats, cb)
        stats.update(check_norms(outs[0][1].cpu().numpy(), orc["norms"]))


def test_graph_capture_codec():
    """Encode and decode captured in a HIP graph: several replays, with eager work in between, give the
    bytes of an eager call.  The 3-bit block-32 encode with fp32 norms and strided rows is launched
    here for the first time inside the capture, where it runs without the residency padding."""
    hd, n_rows, ld = 128, 1000, 136
    x_np = synth.kv_tensor(91, 1, 1, 1, n_rows, hd).reshape(n_rows, hd)
    host = np.zeros((n_rows, ld), dtype=np.float16)
    host[:, :hd] = x_np
    x = torch.from_numpy(host).to(DEV)
    qz = tq.Quantizer(hd, 32, 3, synth.signs(91, 2, 32), norm_dtype=tq.TQ_F32)
    units = n_rows * qz.units_per_row
    codes = torch.zeros(units * qz.code_bytes(), dtype=torch.uint8, device=DEV)
    norms = torch.zeros(units, dtype=torch.float32, device=DEV)
    y = torch.zeros((n_rows, hd), dtype=torch.float16, device=DEV)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        tq.tq_quantize(qz, x, n_rows, ld, codes, norms, stream=stream)
        tq.tq_dequantize(qz, codes, norms, None, None, n_rows, y, tq.TQ_F16, hd, stream=stream)
    torch.cuda.synchronize()
    ref_codes = torch.empty_like(codes)
    ref_norms = torch.empty_like(norms)
    ref_y = torch.empty_like(y)
    tq.tq_quantize(qz, x, n_rows, ld, ref_codes, ref_norms)
    tq.tq_dequantize(qz, ref_codes, ref_norms, None, None, n_rows, ref_y, tq.TQ_F16, hd)
    torch.cuda.synchronize()
    for _ in range(3):
        codes.zero_()
        norms.zero_()
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(codes, ref_codes) and torch.equal(norms, ref_norms) and torch.equal(y, ref_y)
        tq.tq_quantize(qz, x, n_rows, ld, ref_codes, ref_norms)  # eager work between the replays
        torch.cuda.synchronize()

def _bucket_targets(cb, rng):
    """Rotated coordinates (sqrt(dt) y) on the 4- and 8-bit encoders' bucket-table grid: the bin of |y|/n is
    the rounded or truncated product |y| kb with 1.6 bins per narrowest cell, so every bin centre, bin edge
    and the points a quarter bin either side are taken, out past the top cell edge, with random signs."""
    h = 1 << (cb.bits - 1)
    pos = np.asarray(cb.unit_bounds, dtype=np.float64)[h:]
    w = min(pos[0], float(np.diff(pos).min()))
    bs = float(np.float32(1.6 / w))
    top = int(math.ceil(pos[-1] * bs)) + 3
    grid = np.arange(0.0, top, 0.25) / bs
    return grid * rng.choice([-1.0, 1.0], size=grid.size)


def _units_with(targets, dt, rng):
    """Units z (rows of dt values with sum z^2 = dt) that carry the targets, at most dt/2 per unit and a
    sum of squares up to 3/4 dt, the other coordinates equal in magnitude and filling the rest."""
    units, cur = [], []
    for t in rng.permutation(targets):
        if len(cur) == dt // 2 or sum(v * v for v in cur) + t * t > 0.75 * dt:
            units.append(cur)
            cur = []
        cur.append(t)
    units.append(cur)
    out = np.empty((len(units), dt))
    for i, u in enumerate(units):
        rest = dt - len(u)
        f = math.sqrt((dt - sum(v * v for v in u)) / rest)
        row = np.concatenate([u, f * rng.choice([-1.0, 1.0], size=rest)])
        out[i] = rng.permutation(row)
    return out


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("dt,x_dtype", [(32, tq.TQ_F16), (128, tq.TQ_F16), (32, tq.TQ_F32)])
def test_bucket_table_bins(bits, dt, x_dtype):
    """The 4- and 8-bit encoders find a code's magnitude from a table entry chosen by the bin of |y|/n; inputs
    whose rotated coordinates sit on that bin grid (centres, edges, quarter points) would show an entry off by
    one as a code mismatch away from every cell edge.  Each unit is x = D H z / sqrt(dt) (H orthonormal), so
    that the oracle's sqrt(dt) y is z itself (checked here on the CPU first)."""
    rng = np.random.default_rng(100 + bits + dt)
    cb = Codebook.build(bits, dt)
    signs = synth.signs(7, 2, dt)
    z = np.concatenate([_units_with(_bucket_targets(cb, rng), dt, rng) for _ in range(3)])
    x = (z @ hadamard_matrix(dt).T) / math.sqrt(dt) * signs.astype(np.float64)
    hd = 128
    pad_units = (-len(z)) % (hd // dt)
    x = np.concatenate([x, x[:pad_units]]).reshape(-1, hd)
    x_np = x.astype(np.float16 if x_dtype == tq.TQ_F16 else np.float32)
    orc = quantize(x_np.astype(np.float64), signs, cb, norm_dtype=np.float16)
    if x_dtype == tq.TQ_F32:
        assert np.allclose(orc["y_unit"][:len(z)], z, atol=1e-5), "construction: sqrt(dt) y is not z"
    qz = tq.Quantizer(hd, dt, bits, signs, x_dtype=x_dtype)
    codes, _ = _run_encode(qz, x_np)
    check_codes(codes, orc, cb, bits, dt)  # targets at 0, or within 1e-6 of an edge after fp16 rounding, are in band


@pytest.fixture(scope="module")
def qwen_full():
    from synth.workloads import qwen3_8b_kv

    return qwen3_8b_kv()


@pytest.mark.parametrize("kbits,vbits", [(3, 3), (4, 4), (8, 4)])
def test_block32_full_size_sampled(qwen_full, kbits, vbits):
    """The Qwen3-8B-shaped cache at full size (36 x 8 x 16384 x 128, K and V fp16) in block-32
    planes, each half encoded and decoded by one call as the step timing launches it (turbo3,
    turbo4, and 8-bit keys with 4-bit values): codes, norms and decoded rows of 100000 sampled rows
    (the first and last row among them) against the oracle.  The sample holds 12.8 M coordinates
    per half, so the in-band count is held to the literal bound (1e-5 of the coordinates at 3 and 4
    bits, where about 3.5e-6 and 6.7e-6 are expected)."""
    w = qwen_full
    rows = w["k"].shape[0] * w["k"].shape[1] * w["k"].shape[2]
    rng = np.random.default_rng(11 + kbits)
    sample = np.unique(np.concatenate([rng.choice(rows, 100000, replace=False), [0, rows - 1]]))
    sidx = torch.from_numpy(sample).to(DEV)
    for half, s, bits in (("k", "signs_k", kbits), ("v", "signs_v", vbits)):
        x_np = w[half].reshape(rows, 128)
        qz = tq.Quantizer(128, 32, bits, w[s])
        x = torch.from_numpy(x_np).to(DEV)
        rb = 4 * 4 * bits  # code bytes of one row: four 32-value groups
        codes = torch.empty(rows * rb, dtype=torch.uint8, device=DEV)
        norms = torch.empty(rows * 4, dtype=torch.float16, device=DEV)
        tq.tq_quantize(qz, x, rows, 128, codes, norms)
        del x
        y = torch.empty((rows, 128), dtype=torch.float16, device=DEV)
        tq.tq_dequantize(qz, codes, norms, None, None, rows, y, tq.TQ_F16, 128)
        torch.cuda.synchronize()
        c = codes.view(rows, rb)[sidx].cpu().numpy()
        n = norms.view(rows, 4)[sidx].cpu().numpy().reshape(-1)
        ys = y[sidx].cpu().numpy()
        del codes, norms, y
        cb = Codebook.build(bits, 32)
        orc = quantize(x_np[sample].astype(np.float64), w[s], cb)
        stats = check_codes(c, orc, cb, bits, 32)
        stats.update(check_norms(n, orc["norms"]))
        ref = dequantize(c.reshape(-1, 4 * bits), n, w[s], cb)
        stats["f16_ulp_off"] = check_decoded_f16(ys, ref, n, 32)
        print(half, bits, stats)
        assert_band_rate(stats, cb, literal=True)


@pytest.mark.parametrize("bits,dt", [(3, 32), (4, 32), (4, 64)])
def test_grid_threshold_ragged(bits, dt):
    """A launch just over four workgroups per compute unit, where the codec grids switch to two groups
    per lane: 4 x CUs x 256 + 148 groups, so the grid of 4 x CUs workgroups leaves a ragged second
    iteration of 148 groups.  Codes, norms and decoded rows of the last 600 rows and 20000 others
    against the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    hd = 128
    rows = cus * 256 + 37  # 4 groups per row
    x_np = synth.normal_f16(11 + bits, dt, rows * hd).reshape(rows, hd)
    signs = synth.signs(13, 2, dt)
    qz = tq.Quantizer(hd, dt, bits, signs)
    cb = Codebook.build(bits, dt)
    x = torch.from_numpy(x_np).to(DEV)
    units = rows * (hd // dt)
    codes = torch.empty(units * qz.code_bytes(), dtype=torch.uint8, device=DEV)
    norms = torch.empty(units, dtype=torch.float16, device=DEV)
    tq.tq_quantize(qz, x, rows, hd, codes, norms)
    y = torch.empty((rows, hd), dtype=torch.float32, device=DEV)
    tq.tq_dequantize(qz, codes, norms, None, None, rows, y, tq.TQ_F32, hd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(bits + dt)
    sample = np.unique(np.concatenate([rng.choice(rows - 600, 20000, replace=False), np.arange(rows - 600, rows)]))
    upr = hd // dt
    usample = (sample[:, None] * upr + np.arange(upr)[None, :]).reshape(-1)
    c = codes.view(units, -1).cpu().numpy()[usample]
    n = norms.cpu().numpy()[usample]
    ys = y.cpu().numpy()[sample]
    orc = quantize(x_np[sample].astype(np.float64), signs, cb)
    stats = check_codes(c, orc, cb, bits, dt)
    stats.update(check_norms(n, orc["norms"]))
    ref = dequantize(c, n, signs, cb)
    check_decoded_f32(ys, ref.reshape(len(sample), hd), n, dt)
    assert_band_rate(stats, cb)


def test_llama_full_size_sampled():
    """The Llama-3.2-1B-shaped cache at full size (16 x 8 x 2048 vectors of 64 per half, fp16),
    4 bits with a per-vector norm and norm correction, one call per half: codes, norms and
    decoded rows of 200000 of the 262144 rows of each half against the oracle (12.8 M coordinates,
    in-band count held to the literal 1e-5 bound)."""
    from synth.workloads import llama_1b_kv

    w = llama_1b_kv()
    rows = w["k"].shape[0] * w["k"].shape[1] * w["k"].shape[2]
    rng = np.random.default_rng(5)
    sample = np.unique(np.concatenate([rng.choice(rows, 200000, replace=False), [0, rows - 1]]))
    sidx = torch.from_numpy(sample).to(DEV)
    cb = Codebook.build(4, 64)
    for half, s in (("k", "signs_k"), ("v", "signs_v")):
        x_np = w[half].reshape(rows, 64)
        qz = tq.Quantizer(64, 64, 4, w[s], flags=tq.TQ_NORM_CORRECT)
        x = torch.from_numpy(x_np).to(DEV)
        codes = torch.empty(rows * 32, dtype=torch.uint8, device=DEV)
        norms = torch.empty(rows, dtype=torch.float16, device=DEV)
        tq.tq_quantize(qz, x, rows, 64, codes, norms)
        y = torch.empty((rows, 64), dtype=torch.float32, device=DEV)
        tq.tq_dequantize(qz, codes, norms, None, None, rows, y, tq.TQ_F32, 64)
        torch.cuda.synchronize()
        c = codes.view(rows, 32)[sidx].cpu().numpy()
        n = norms[sidx].cpu().numpy()
        ys = y[sidx].cpu().numpy()
        orc = quantize(x_np[sample].astype(np.float64), w[s], cb)
        stats = check_codes(c, orc, cb, 4, 64)
        stats.update(check_norms(n, orc["norms"]))
        ref = dequantize(c, n, w[s], cb, nc=True)
        stats["decode_err"] = check_decoded_f32(ys, ref, n, 64)
        print(half, stats)
        assert_band_rate(stats, cb, literal=True)
