"""GPU parity of tq_qjl_scores against the oracle's QJL estimator.

Keys are encoded on the GPU (tq_quantize with TQ_QJL); the oracle then scores
the GPU's own codes, norms, sign bits and residual norms, so the comparison
isolates the scoring kernels.  Tolerance: |score_gpu - score_orc| <= 1e-4 *
n_j * ||q_i|| (the Cauchy-Schwarz scale of the score; a pointwise relative
error is undefined for scores near zero).  The pointwise relative error
|score_gpu - score_orc| / |score_orc| is reported beside it, as a distribution
over the scores with |score_orc| >= 1e-3 n_j ||q_i||, with its largest value
among the scores well away from zero (|score_orc| >= 0.1 n_j ||q_i||, about a
quarter of the scores of random pairs in 128 dimensions).
"""
import numpy as np
import pytest

import synth
from oracle import Codebook, qjl_scores

torch = pytest.importorskip("torch")
import kv_cache_vector_amd as tq  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-4


class Keys:
    def __init__(self, keys, dt, bits, m, signs, S, codebook="gaussian"):
        n = keys.shape[0]
        self.n, self.dt, self.bits, self.m = n, dt, bits, m
        self.signs, self.S, self.codebook = signs, S, codebook
        self.qz = tq.Quantizer(dt, dt, bits, signs, flags=tq.TQ_QJL, qjl_m=m, codebook=codebook)
        self.params = torch.empty(tq.tq_qjl_params_size(m, dt), dtype=torch.uint8, device=DEV)
        tq.tq_qjl_prepare(self.qz, S, self.params)
        x = torch.from_numpy(keys).to(DEV)
        self.codes = torch.empty(n * dt * bits // 8, dtype=torch.uint8, device=DEV)
        self.norms = torch.empty(n, dtype=torch.float16, device=DEV)
        self.sbits = torch.empty(n * m // 8, dtype=torch.uint8, device=DEV)
        self.rnorm = torch.empty(n, dtype=torch.float16, device=DEV)
        tq.tq_quantize(self.qz, x, n, dt, self.codes, self.norms, self.sbits, self.rnorm)

    def scores(self, q_np, ld_s=None):
        nq = q_np.shape[0]
        qt = torch.from_numpy(q_np).to(DEV)
        qtype = tq.TQ_F32 if q_np.dtype == np.float32 else tq.TQ_F16
        ld_s = self.n if ld_s is None else ld_s
        out = torch.full((nq, ld_s), -99.0, dtype=torch.float32, device=DEV)
        wsb = tq.tq_workspace_size(tq.TQ_OP_QJL_SCORES, self.qz, nq, self.n)
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        tq.tq_qjl_scores(self.qz, qt, qtype, nq, self.dt, self.codes, self.norms, self.sbits, self.rnorm, self.n, out,
                         ld_s, ws, wsb)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        if ld_s > self.n:
            assert np.all(o[:, self.n:] == -99.0), "scores written outside the rows"
        return o[:, :self.n]

    def host(self):
        n = self.n
        return (self.codes.cpu().numpy().reshape(n, -1), self.norms.cpu().numpy(),
                self.sbits.cpu().numpy().reshape(n, -1), self.rnorm.cpu().numpy())

    def oracle(self, q_np, rows=None, cols=None):
        codes, norms, sb, rn = self.host()
        cols = np.arange(self.n) if cols is None else cols
        q = q_np if rows is None else q_np[rows]
        cb = Codebook.build_beta(self.bits, self.dt) if self.codebook == "beta" else Codebook.build(self.bits, self.dt)
        return qjl_scores(q.astype(np.float64), codes[cols], norms[cols], sb[cols], rn[cols], self.signs, cb, self.S)


def pointwise(err, orc, scale):
    """Distribution of the pointwise relative error over the scores with |orc| >= 1e-3 of their
    Cauchy-Schwarz scale: quantiles, the largest value, and the largest among |orc| >= 0.1 scale."""
    a = np.abs(orc)
    sel = a >= 1e-3 * scale
    rel = err[sel] / a[sel]
    far = a >= 0.1 * scale
    q = np.quantile(rel, [0.5, 0.99, 0.999]) if rel.size else [0.0, 0.0, 0.0]
    return {"scores": int(sel.sum()), "median": float(q[0]), "p99": float(q[1]), "p999": float(q[2]),
            "max": float(rel.max(initial=0.0)),
            "max_far_from_zero": float((err[far] / a[far]).max(initial=0.0)), "far_from_zero": int(far.sum())}


def _check(gpu, orc, q, norms):
    scale = np.linalg.norm(q.astype(np.float64), axis=1)[:, None] * norms.astype(np.float64)[None, :]
    err = np.abs(gpu.astype(np.float64) - orc)
    bound = TOL * scale + 1e-30
    worst = float(np.max(err / np.maximum(scale, 1e-30)))
    assert np.all(err <= bound), f"score error {worst:.3g} of n*||q|| exceeds {TOL}"
    print(f"worst error {worst:.3g} of n*||q||; pointwise relative error: {pointwise(err, orc, scale)}")
    return worst


@pytest.mark.parametrize("bits,dt,m,qdt", [(2, 128, 128, np.float16), (1, 128, 128, np.float32),
                                           (3, 128, 64, np.float16), (2, 64, 128, np.float32),
                                           (3, 64, 64, np.float16)])
def test_scores_matrix(bits, dt, m, qdt):
    n_k, n_q = 1000, 70  # ragged against the 32-query blocks and the 128/256-key tiles
    keys = synth.kv_tensor(bits + dt, 1, 1, 0, n_k, dt, n_outliers=0).reshape(n_k, dt)
    signs = synth.signs(bits, 2, dt)
    S = synth.gaussian_matrix(bits + 1, 0, m, dt)
    K = Keys(keys, dt, bits, m, signs, S)
    q = synth.normal_f16(bits, 6, n_q * dt).reshape(n_q, dt).astype(qdt)
    gpu = K.scores(q, ld_s=n_k + 7)
    orc = K.oracle(q)
    worst = _check(gpu, orc, q, K.host()[1][None, :][0])
    print(f"bits={bits} dt={dt} m={m}: worst error {worst:.2e} of n*||q||")


@pytest.mark.parametrize("bits,dt", [(2, 128), (3, 64)])
def test_scores_beta_codebook(bits, dt):
    """Keys encoded with the exact-marginal codebook: QJL residuals and scores use its centroids."""
    n_k, n_q, m = 700, 40, 128
    keys = synth.kv_tensor(90 + bits, 1, 1, 0, n_k, dt, n_outliers=0).reshape(n_k, dt)
    signs = synth.signs(91, 2, dt)
    S = synth.gaussian_matrix(92, 0, m, dt)
    K = Keys(keys, dt, bits, m, signs, S, codebook="beta")
    q = synth.normal_f16(93, 6, n_q * dt).reshape(n_q, dt)
    gpu = K.scores(q)
    orc = K.oracle(q)
    worst = _check(gpu, orc, q, K.host()[1])
    print(f"beta bits={bits} dt={dt}: worst error {worst:.2e} of n*||q||")


@pytest.mark.parametrize("n_k,n_q", [(1000, 70), (4100, 200), (4100, 3000)])
def test_scores_dense_rows_ragged(n_k, n_q):
    """ld_s == n_k (buffer stores where a whole key tile and query block fit, element stores on the
    ragged key tile and query block): every score of the matrix against the oracle.  At 4100 x 3000
    each workgroup streams several query blocks through its ring, the last chunk a shorter one."""
    bits, dt, m = 2, 128, 128
    keys = synth.kv_tensor(77, 1, 1, 0, n_k, dt, n_outliers=0).reshape(n_k, dt)
    signs = synth.signs(78, 2, dt)
    S = synth.gaussian_matrix(79, 0, m, dt)
    K = Keys(keys, dt, bits, m, signs, S)
    q = synth.normal_f16(80, 6, n_q * dt).reshape(n_q, dt)
    gpu = K.scores(q)
    orc = K.oracle(q)
    worst = _check(gpu, orc, q, K.host()[1])
    print(f"n_k={n_k} n_q={n_q}: worst error {worst:.2e} of n*||q||")


def test_scores_wide_rows():
    """Rows of 2^24 + 3 floats: the byte offsets within a query block no longer fit 32 bits, so every
    tile takes the element-store path.  Every score against the oracle; the padding is untouched."""
    n_k, n_q, bits, dt, m = 300, 40, 2, 128, 128
    ld_s = (1 << 24) + 3
    keys = synth.kv_tensor(81, 1, 1, 0, n_k, dt, n_outliers=0).reshape(n_k, dt)
    K = Keys(keys, dt, bits, m, synth.signs(82, 2, dt), synth.gaussian_matrix(83, 0, m, dt))
    q = synth.normal_f16(84, 6, n_q * dt).reshape(n_q, dt)
    out = torch.full((n_q, ld_s), -99.0, dtype=torch.float32, device=DEV)
    wsb = tq.tq_workspace_size(tq.TQ_OP_QJL_SCORES, K.qz, n_q, n_k)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    tq.tq_qjl_scores(K.qz, torch.from_numpy(q).to(DEV), tq.TQ_F16, n_q, dt, K.codes, K.norms, K.sbits, K.rnorm,
                     n_k, out, ld_s, ws, wsb)
    torch.cuda.synchronize()
    assert bool((out[:, n_k:n_k + 4096] == -99.0).all()) and bool((out[:, -4096:] == -99.0).all())
    gpu = out[:, :n_k].cpu().numpy()
    del out
    worst = _check(gpu, K.oracle(q), q, K.host()[1])
    print(f"ld_s=2^24+3: worst error {worst:.2e} of n*||q||")


def test_scores_full_size_sampled():
    """4096 queries x 65536 keys x 128, 2-bit + QJL (m = 128): the full score matrix on the GPU,
    the oracle on 48 sampled queries x 4096 sampled keys."""
    from synth.workloads import qjl_keys

    w = qjl_keys()
    K = Keys(w["keys"], 128, 2, 128, w["signs"], w["S"])
    gpu = K.scores(w["q"])
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(w["q"].shape[0], 48, replace=False))
    cols = np.sort(rng.choice(K.n, 4096, replace=False))
    orc = K.oracle(w["q"], rows, cols)
    worst = _check(gpu[np.ix_(rows, cols)], orc, w["q"][rows], K.host()[1][cols])
    print(f"full-size sample worst error {worst:.2e} of n*||q||")


@pytest.mark.parametrize("total_bits", [2, 3, 4])
@pytest.mark.parametrize("n_k", [512, 2048, 8192])
def test_needle_retrieval(total_bits, n_k):
    """A key planted near the query among random keys is the top-1 score (total_bits = MSE bits + 1 QJL bit)."""
    dt = m = 128
    rng = np.random.default_rng(total_bits * 100000 + n_k)
    keys = synth.normal_f16(total_bits, 0, n_k * dt).reshape(n_k, dt).astype(np.float32)
    q = synth.normal_f16(total_bits, 6, dt).reshape(1, dt).astype(np.float32)
    needle = int(rng.integers(n_k))
    keys[needle] = q[0] + 0.3 * rng.standard_normal(dt)
    keys = keys.astype(np.float16)
    K = Keys(keys, dt, total_bits - 1, m, synth.signs(total_bits, 2, dt), synth.gaussian_matrix(1, 0, m, dt))
    gpu = K.scores(q.astype(np.float16))
    assert int(np.argmax(gpu[0])) == needle
