#!/usr/bin/env python3
"""Throughput of the TurboQuant KV-cache quantizer hot path on one MI355X.

Workload (one step): encode then decode the whole Qwen3-8B-shaped KV cache,
36 layers x 8 KV heads x 16384 tokens x head_dim 128, K and V fp16
(synthetic: N(0,1) entries times per-channel log-normal scales, 2 outlier
channels per head at 10x), in the block-32 layout (one fp16 norm per 32
values) at 3 bits (3.5 bits per value).  Inputs are resident in HBM before
the timed region; each step runs tq_quantize(K), tq_quantize(V),
tq_dequantize(K), tq_dequantize(V) through the C ABI.

Prints one JSON line.  `value` is fp16 KV GB/s encoded+decoded: fp16 bytes
read by the encodes plus fp16 bytes written by the decodes, per second.

The same cache is also run in the fork's production layout (128-value
chunks, the chunk norm copied into each 14/18-byte 32-value record, Beta
codebook for d = 128), reported as `fork_layout`, and with 8-bit keys and
4-bit values (block-32), reported as `k8v4` (neither is part of `value`).

More workloads are timed and reported beside it (not part of `value`):
  vectors_fp32  4096 vectors x 128 fp32, 3 bits, one fp32 norm per vector
        (whole-vector units): device time per encode and decode call;
  llama_1b      the Llama-3.2-1B-shaped cache, 16 layers x 8 KV heads x 2048
        tokens x head_dim 64 per half, fp16, 4 bits with a per-vector norm and
        norm correction: the same four-launch step, flushed and warm (the
        cache fits the 256 MB last-level cache);
  qjl   65536 keys x 128 fp16 encoded at 2 bits + the 1-bit QJL residual
        (dense Gaussian S, m = 128), then scored against 4096 queries
        (32 heads x 128 tokens): keys/s and scores/s;
  attn  single-token decode attention over a 131072-token cache, head_dim
        256, 4 KV heads, 16 query heads, 3-bit block-32 K and V (and, as
        attn.k8v4, 8-bit K with 4-bit V): time per call and compressed bytes
        read per second, with the cache warm in the last-level cache and with
        it flushed before each call.

`cpu_baseline` times the CPU oracle (unchanged, float64 numpy) on the host:
encode + decode of whole layers of the same cache in worker processes, one
per core of this GPU's CPU share and then a single one, and the oracle's QJL
scores and decode attention on the other two workloads.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
LAYERS, KV_HEADS, TOKENS, HEAD_DIM, DT = 36, 8, 16384, 128, 32
SAMPLE_ROWS = 4096  # head vectors of the oracle's sample (layer 0, head 0 K)
CODEBOOK = "gaussian"  # set from --codebook


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(units: int, bits: int) -> dict:
    fp16 = units * DT * 2
    codes = units * DT * bits // 8
    norms = units * 2
    return {"fp16": fp16, "compressed": codes + norms, "per_launch": fp16 + codes + norms}


def make_cache(tq, torch, dev):
    import synth
    from synth import workloads

    rows = LAYERS * KV_HEADS * TOKENS
    t0 = time.time()
    w = workloads.qwen3_8b_kv()
    log(f"generated K/V ({2 * rows * HEAD_DIM * 2 / 2**30:.2f} GiB fp16) in {time.time() - t0:.1f}s")
    k = torch.from_numpy(w["k"].reshape(rows, HEAD_DIM)).to(dev)
    v = torch.from_numpy(w["v"].reshape(rows, HEAD_DIM)).to(dev)
    del w["k"], w["v"]
    return k, v, w["signs_k"], w["signs_v"], rows


class Codec:
    """K and V encode/decode buffers for the cache: block-32 units in two planes (codes, fp16 norms),
    or with records=True the fork's 32-value records over dt-long chunks (norms inside the records)."""

    def __init__(self, tq, torch, dev, rows, bits, signs_k, signs_v, dt=DT, records=False, codebook=None,
                 vbits=None):
        vbits = vbits or bits  # V may take fewer bits than K (8-bit keys with 4-bit values)
        self.tq, self.rows, self.bits, self.vbits = tq, rows, bits, vbits
        flags = tq.TQ_BLOCKS if records else 0
        cbk = codebook or CODEBOOK
        self.qk = tq.Quantizer(HEAD_DIM, dt, bits, signs_k, flags=flags, codebook=cbk)
        self.qv = tq.Quantizer(HEAD_DIM, dt, vbits, signs_v, flags=flags, codebook=cbk)
        groups = rows * HEAD_DIM // 32
        self.units = groups  # 32-value groups (the unit of the byte accounting)
        if records:
            self.ck = torch.empty(groups * (2 + 4 * bits), dtype=torch.uint8, device=dev)
            self.cv = torch.empty(groups * (2 + 4 * vbits), dtype=torch.uint8, device=dev)
            self.nk = self.nv = None
        else:
            units = rows * HEAD_DIM // dt
            self.ck = torch.empty(units * dt * bits // 8, dtype=torch.uint8, device=dev)
            self.cv = torch.empty(units * dt * vbits // 8, dtype=torch.uint8, device=dev)
            self.nk = torch.empty(units, dtype=torch.float16, device=dev)
            self.nv = torch.empty(units, dtype=torch.float16, device=dev)

    def outputs(self):
        return [t for t in (self.ck, self.cv, self.nk, self.nv) if t is not None]

    def launches(self, k, v, ok, ov):
        """The step's four launches: quantize K, quantize V, dequantize K, dequantize V."""
        tq = self.tq
        return [lambda: tq.tq_quantize(self.qk, k, self.rows, HEAD_DIM, self.ck, self.nk),
                lambda: tq.tq_quantize(self.qv, v, self.rows, HEAD_DIM, self.cv, self.nv),
                lambda: tq.tq_dequantize(self.qk, self.ck, self.nk, None, None, self.rows, ok, tq.TQ_F16, HEAD_DIM),
                lambda: tq.tq_dequantize(self.qv, self.cv, self.nv, None, None, self.rows, ov, tq.TQ_F16, HEAD_DIM)]


def time_steps(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def capture_step(torch, step, outputs):
    """Capture one step (its four launches) in a HIP graph.  The graph runs the same kernels on the
    same buffers; its replays are checked against an eager step, with eager work in between, before
    they are timed.  Returns None (eager timing) if a replay differs."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    for _ in range(3):
        for t in outputs:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(ref, outputs)):
            log("graph replay differs from the eager step; timing eager launches")
            return None
        step()
        torch.cuda.synchronize()
    return graph


def per_kernel_ms(torch, codec, k, v, ok, ov, reps, split=False):
    """Average duration (ms) of one encode launch and one decode launch inside the step sequence
    (quantize K, quantize V, dequantize K, dequantize V, so every launch streams from HBM as in the
    step), from HIP events recorded between the launches on the stream they run on (torch's
    current stream).  One untimed step first keeps the GPU busy, so host launch latency is not
    timed; each interval also holds the launch gap before its kernel."""
    launches = codec.launches(k, v, ok, ov)
    torch.cuda.synchronize()
    for f in launches:
        f()
    ev = []
    for _ in range(reps):
        for f in launches:
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            ev.append(e)
            f()
    end = torch.cuda.Event(enable_timing=True)
    end.record()
    ev.append(end)
    torch.cuda.synchronize()
    d = [ev[i].elapsed_time(ev[i + 1]) for i in range(len(ev) - 1)]
    if split:  # K encode, V encode, K decode, V decode separately
        return tuple(sum(d[i] for i in range(len(d)) if i % 4 == j) / reps for j in range(4))
    enc = [d[i] for i in range(len(d)) if i % 4 in (0, 1)]
    dec = [d[i] for i in range(len(d)) if i % 4 in (2, 3)]
    return sum(enc) / len(enc), sum(dec) / len(dec)


def launch_avg_ms(torch, launches, outputs, reps):
    """Average duration (ms) of one launch of a kernel: its K and V launches (as in the step) captured
    back to back in a HIP graph, the replays timed between two HIP events on the launch stream, divided
    by the number of launches.  Every launch streams from HBM (K and V alternate), and no event packet
    sits between the kernels, so each launch is charged only the ordinary gap to the next one."""
    def run():
        for f in launches:
            f()

    graph = capture_step(torch, run, outputs)
    fn = graph.replay if graph is not None else run
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * len(launches))


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "codec_qwen3_8b_hbm_traffic.txt")


def measured_traffic(tag: str):
    """HBM bytes per launch of the encode/decode kernel `tag` (e.g. 'decode_turbo3') from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None if the kernel source changed since it was taken."""
    import hashlib

    try:
        fields = dict(line.split(": ", 1) for line in open(TRAFFIC_PROFILE).read().splitlines()
                      if ": " in line and not line.startswith("#"))
    except OSError:
        return None
    src = os.path.join(ROOT, "kv_cache_vector_amd", "csrc", "tq_codec.hip")
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != fields.get("codec_source_sha256"):
        return None
    v = fields.get(f"{tag}_traffic_bytes")
    return int(v) if v else None


# ---- CPU oracle baseline ---------------------------------------------------------------------------------
# The oracle as it stands, split over rows (or queries, or KV heads) across worker processes started fresh
# (spawn) with one BLAS thread each; inputs reach the workers through shared memory and are generated
# before the timed region.  Only this leg of the bench runs the oracle.

_SHM = {}


def _cpu_worker_init():
    import numpy  # noqa: F401  (imported before the timed region)

    import oracle  # noqa: F401


def _shm_view(name, shape, dtype):
    from multiprocessing import shared_memory

    import numpy as np

    if name not in _SHM:
        _SHM[name] = shared_memory.SharedMemory(name=name)
    return np.ndarray(shape, dtype=dtype, buffer=_SHM[name].buf)


def _cpu_codec_task(t):
    """Encode + decode rows [r0, r1) of the shared fp16 array with the oracle; returns seconds spent."""
    import numpy as np

    import synth
    from oracle import Codebook, dequantize, quantize

    name, shape, r0, r1, bits, dt = t
    x = np.array(_shm_view(name, shape, np.float16)[r0:r1], dtype=np.float64)
    cb = Codebook.build(bits, dt)
    signs = synth.signs(0, synth.STREAM_SIGNS_K, dt)
    t0 = time.perf_counter()
    q = quantize(x, signs, cb)
    dequantize(q["codes"], q["norms"], signs, cb)
    return time.perf_counter() - t0


def _cpu_scores_task(t):
    """The oracle's QJL scores of queries [q0, q1) against every key; returns seconds spent."""
    import numpy as np

    from oracle import qjl_scores

    (qn, qs), (cn, cs), (nn, ns), (bn, bs), (rn, rs), q0, q1, signs, cb, S = t
    q = np.array(_shm_view(qn, qs, np.float16)[q0:q1])
    args = [np.array(_shm_view(n_, s_, dt_)) for (n_, s_), dt_ in
            (((cn, cs), np.uint8), ((nn, ns), np.float16), ((bn, bs), np.uint8), ((rn, rs), np.float16))]
    t0 = time.perf_counter()
    qjl_scores(q.astype(np.float64), args[0], args[1], args[2], args[3], signs, cb, S)
    return time.perf_counter() - t0


def _cpu_attn_task(t):
    """The oracle's decode attention of one KV head (its query heads over every token); returns seconds."""
    import numpy as np

    from oracle import decode_attention

    q, kc, kn, vc, vn, sk, sv, kcb, vcb, T, hd = t
    t0 = time.perf_counter()
    decode_attention(q, kc, kn, vc, vn, sk, sv, kcb, vcb, 1, T, hd)
    return time.perf_counter() - t0


def _cpu_share() -> int:
    """Worker processes: the CPUs this process may run on, at most 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _timed_map(pool, fn, tasks):
    t0 = time.perf_counter()
    busy = pool.map(fn, tasks, chunksize=1)
    return time.perf_counter() - t0, sum(busy)


def cpu_baseline(bits: int, layers: int = 4, x_rows=None, gpu_codes=None, gpu_norms=None) -> dict:
    """The float64 oracle on the host, timed on `layers` whole layers of the Qwen3-8B-shaped cache (K and V,
    fp16): encode + decode split over rows across one worker per core of this GPU's CPU share, and again
    in one worker; the same fp16-bytes-per-second unit as `value`.  Then the oracle's QJL scores (65536
    keys, 4096 queries; one core on a 1/16 strided sample of the queries) and its decode attention (131072
    tokens, per KV head).  With the GPU's codes and norms of layer 0 / head 0 K's first rows, also the parity
    counts of that sample: coordinates within 1e-6 (unit-variance scale, i.e. 1e-6/sqrt(d) for the
    N(0, 1/d) cells) of a cell edge, codes that differ from the oracle's, those outside that band, and
    norms that differ."""
    import multiprocessing as mp
    from multiprocessing import shared_memory

    import numpy as np

    import synth
    from synth import workloads

    n_cores = _cpu_share()
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"  # one BLAS thread per worker (the spawned workers inherit this)
    ctx = mp.get_context("spawn")
    shms = []

    def share(a):
        m = shared_memory.SharedMemory(create=True, size=max(1, a.nbytes))
        np.ndarray(a.shape, dtype=a.dtype, buffer=m.buf)[...] = a
        shms.append(m)
        return m.name, a.shape

    out = {"unit": "GB/s", "cores": n_cores, "kind": "oracle"}
    try:
        # --- encode + decode of whole layers -------------------------------------------------------------
        rows_half = layers * KV_HEADS * TOKENS
        kv = workloads.qwen3_8b_kv(layers=layers)
        x = np.concatenate([kv["k"].reshape(rows_half, HEAD_DIM), kv["v"].reshape(rows_half, HEAD_DIM)])
        del kv
        name, shape = share(x)
        rows = x.shape[0]
        del x
        chunk = 4096
        tasks = [(name, shape, r, min(rows, r + chunk), bits, DT) for r in range(0, rows, chunk)]
        fp16_bytes = rows * HEAD_DIM * 2 * 2  # encoded in + decoded out
        with ctx.Pool(n_cores, initializer=_cpu_worker_init) as pool:
            pool.map(_cpu_codec_task, tasks[:n_cores], chunksize=1)  # every worker up and warm
            wall_n, busy_n = _timed_map(pool, _cpu_codec_task, tasks)
        with ctx.Pool(1, initializer=_cpu_worker_init) as pool:
            pool.map(_cpu_codec_task, tasks[:1])
            wall_1, busy_1 = _timed_map(pool, _cpu_codec_task, tasks)
        out["value"] = fp16_bytes / wall_n / 1e9
        out["sample"] = (f"layers 0-{layers - 1} of the cache, K and V ({rows} head vectors, {rows * HEAD_DIM // DT} "
                         f"blocks), encode+decode at {bits} bits: {wall_n:.2f} s on {n_cores} worker processes "
                         f"({busy_n:.1f} s of worker time), {wall_1:.2f} s on one")
        out["single_core"] = {"value": fp16_bytes / wall_1 / 1e9, "unit": "GB/s", "cores": 1,
                              "blocks_per_s": round(rows * HEAD_DIM // DT / wall_1)}
        out["blocks_per_s"] = round(rows * HEAD_DIM // DT / wall_n)
        log(f"cpu oracle codec: {out['value']:.3f} GB/s on {n_cores} cores, "
            f"{out['single_core']['value']:.3f} GB/s on one")

        # --- QJL scores ----------------------------------------------------------------------------------
        from oracle import Codebook, quantize

        w = workloads.qjl_keys()
        cbq = Codebook.build(2, 128)
        enc = quantize(w["keys"].astype(np.float64), w["signs"], cbq, S=w["S"])
        qsh = share(w["q"])
        parts = [share(enc["codes"]), share(enc["norms"]), share(enc["qjl_bits"]), share(enc["rho"])]
        nq, nk = w["q"].shape[0], w["keys"].shape[0]
        blk = 128
        sc_tasks = [(qsh, *parts, q0, min(nq, q0 + blk), w["signs"], cbq, w["S"]) for q0 in range(0, nq, blk)]
        with ctx.Pool(n_cores, initializer=_cpu_worker_init) as pool:
            pool.map(_cpu_scores_task, sc_tasks[:n_cores], chunksize=1)
            wall_sn, _ = _timed_map(pool, _cpu_scores_task, sc_tasks)
        one = [(qsh, *parts, q0, q0 + 16, w["signs"], cbq, w["S"]) for q0 in range(0, nq, 512)]
        with ctx.Pool(1, initializer=_cpu_worker_init) as pool:
            pool.map(_cpu_scores_task, one[:1])
            wall_s1, _ = _timed_map(pool, _cpu_scores_task, one)
        out["qjl_scores"] = {"scores_per_s": round(nq * nk / wall_sn), "cores": n_cores,
                             "scores_per_s_single_core": round(16 * len(one) * nk / wall_s1),
                             "sample": f"{nq} queries x {nk} keys on {n_cores} cores ({wall_sn:.2f} s); "
                                       f"{16 * len(one)} queries (16 of every 512) x {nk} keys on one ({wall_s1:.2f} s)"}
        log(f"cpu oracle scores: {out['qjl_scores']['scores_per_s']:.3g} scores/s on {n_cores} cores")

        # --- decode attention ----------------------------------------------------------------------------
        c = workloads.decode_cache()
        H, T, hd = c["k"].shape[1], c["k"].shape[2], c["k"].shape[3]
        cba = Codebook.build(3, 32)
        G = c["q"].shape[0] // H
        at_tasks = []
        for g in range(H):
            ek = quantize(c["k"][0, g].astype(np.float64), c["signs_k"], cba)
            ev = quantize(c["v"][0, g].astype(np.float64), c["signs_v"], cba)
            at_tasks.append((c["q"][g * G:(g + 1) * G].astype(np.float64), ek["codes"], ek["norms"], ev["codes"],
                             ev["norms"], c["signs_k"], c["signs_v"], cba, cba, T, hd))
        with ctx.Pool(min(n_cores, H), initializer=_cpu_worker_init) as pool:
            wall_an, _ = _timed_map(pool, _cpu_attn_task, at_tasks)
        with ctx.Pool(1, initializer=_cpu_worker_init) as pool:
            wall_a1, _ = _timed_map(pool, _cpu_attn_task, at_tasks[:1])
        out["attn"] = {"us_per_call": round(wall_an * 1e6), "cores": min(n_cores, H),
                       "kv_head_tokens_per_s": round(H * T / wall_an),
                       "kv_head_tokens_per_s_single_core": round(T / wall_a1),
                       "sample": f"the whole call ({H} KV heads x {T} tokens, {c['q'].shape[0]} query heads, one "
                                 f"worker per KV head) in {wall_an:.2f} s; one KV head on one core in {wall_a1:.2f} s"}
        log(f"cpu oracle attention: {wall_an:.2f} s per call on {min(n_cores, H)} cores")
    finally:
        for m in shms:
            m.close()
            m.unlink()

    if gpu_codes is not None and x_rows is not None:
        from oracle import Codebook, code_to_index, quantize, unpack_codes

        cb = Codebook.build(bits, DT)
        signs = synth.signs(0, synth.STREAM_SIGNS_K, DT)
        q = quantize(np.asarray(x_rows, dtype=np.float64), signs, cb)
        g = code_to_index(unpack_codes(np.asarray(gpu_codes).reshape(-1, DT * bits // 8), bits, DT), bits)
        o = code_to_index(unpack_codes(q["codes"], bits, DT), bits)
        edges = np.asarray(cb.unit_bounds)
        i = np.searchsorted(edges, q["y_unit"])
        dist = np.minimum(np.abs(q["y_unit"] - edges[np.clip(i - 1, 0, len(edges) - 1)]),
                          np.abs(q["y_unit"] - edges[np.clip(i, 0, len(edges) - 1)]))
        near, diff = dist < 1e-6, g != o
        nd = np.asarray(gpu_norms).astype(np.float16).view(np.uint16) != q["norms"].astype(np.float16).view(np.uint16)
        out["parity"] = {"rows": len(x_rows), "coords": int(g.size), "near_edge": int(near.sum()),
                         "code_mismatch": int(diff.sum()), "code_mismatch_off_edge": int((diff & ~near).sum()),
                         "norm_mismatch": int(nd.sum())}
    return out


def run_k8v4(tq, torch, dev, rows, k, v, ok, ov, signs_k, signs_v, args):
    """The cache with 8-bit keys and 4-bit values (block-32): the same four-launch step."""
    codec = Codec(tq, torch, dev, rows, 8, signs_k, signs_v, vbits=4)
    launches = codec.launches(k, v, ok, ov)

    def step():
        for f in launches:
            f()

    graph = None if args.no_graph else capture_step(torch, step, codec.outputs() + [ok, ov])
    ms = time_steps(torch, graph.replay if graph is not None else step, args.steps, args.warmup)
    del graph
    ek, ev, dk, dv = per_kernel_ms(torch, codec, k, v, ok, ov, max(5, args.steps // 2), split=True)
    b8, b4 = algorithmic_bytes(codec.units, 8), algorithmic_bytes(codec.units, 4)
    out = {"workload": "same cache, 8-bit keys and 4-bit values, block-32 (fp16 norm per 32 values)",
           "step_ms": round(ms, 4), "GBs": round(2 * 2 * b8["fp16"] / (ms * 1e-3) / 1e9, 1),
           "encode_k8_ms": round(ek, 4), "encode_k8_GBs": round(b8["per_launch"] / ek / 1e6, 1),
           "decode_k8_ms": round(dk, 4), "decode_k8_GBs": round(b8["per_launch"] / dk / 1e6, 1),
           "encode_k8_frac": round(b8["per_launch"] / ek / 1e6 / HBM_PEAK_GBS, 4),
           "decode_k8_frac": round(b8["per_launch"] / dk / 1e6 / HBM_PEAK_GBS, 4),
           "encode_v4_ms": round(ev, 4), "decode_v4_ms": round(dv, 4),
           "encode_v4_frac": round(b4["per_launch"] / ev / 1e6 / HBM_PEAK_GBS, 4),
           "decode_v4_frac": round(b4["per_launch"] / dv / 1e6 / HBM_PEAK_GBS, 4)}
    log(f"k8v4: step {ms:.3f} ms, K encode {ek:.3f} ms ({out['encode_k8_GBs']} GB/s), K decode {dk:.3f} ms "
        f"({out['decode_k8_GBs']} GB/s), V encode {ev:.3f} ms, V decode {dv:.3f} ms")
    del codec
    torch.cuda.empty_cache()
    return out


def event_ms(torch, fn, reps, before=None):
    """Median and minimum duration (ms) of fn() from HIP events on the current stream;
    before() runs untimed ahead of each repetition (it must keep the GPU busy, e.g. a cache
    flush, so that the host's launch latency is not timed)."""
    ts = []
    for _ in range(reps):
        if before is not None:
            before()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts.sort()
    return ts[len(ts) // 2], ts[0]


def batch_ms(torch, fn, reps):
    """Average duration (ms) of fn() over `reps` back-to-back calls between two HIP events on the
    current stream; one untimed call first keeps the GPU busy while the timed calls are queued."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def graph_ms(torch, fn, outputs, reps, calls=1):
    """Average device duration (ms) of one fn() call from `reps` replays of a HIP graph holding
    `calls` calls back to back, between two HIP events (the host cost of the Python call is not
    timed; several calls per graph spread a replay's launch latency, which is comparable to a kernel
    of ~20 us, over them).  The replay is checked against an eager call first; falls back to
    back-to-back eager calls if it differs."""
    def many():
        for _ in range(calls):
            fn()

    graph = capture_step(torch, many, outputs)
    if graph is None:
        return batch_ms(torch, fn, reps)
    torch.cuda.synchronize()
    graph.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * calls)


def bench_vectors_fp32(tq, torch, dev, reps):
    """4096 random vectors x 128 fp32 (N(0,1), seed 0), 3 bits, whole-vector units with one fp32 norm each:
    encode and decode of the whole set, device time per call from HIP-graph replays (the set is 2 MiB
    and stays in L2, so this is a latency figure)."""
    from synth import workloads

    w = workloads.vectors_fp32()
    n, d, bits = w["x"].shape[0], w["x"].shape[1], 3
    qz = tq.Quantizer(d, d, bits, w["signs"], x_dtype=tq.TQ_F32, norm_dtype=tq.TQ_F32, codebook=CODEBOOK)
    x = torch.from_numpy(w["x"]).to(dev)
    codes = torch.empty(n * d * bits // 8, dtype=torch.uint8, device=dev)
    norms = torch.empty(n, dtype=torch.float32, device=dev)
    y = torch.empty((n, d), dtype=torch.float32, device=dev)

    def enc():
        tq.tq_quantize(qz, x, n, d, codes, norms)

    def dec():
        tq.tq_dequantize(qz, codes, norms, None, None, n, y, tq.TQ_F32, d)

    enc()
    dec()
    enc_ms = graph_ms(torch, enc, [codes, norms], reps, calls=10)
    dec_ms = graph_ms(torch, dec, [y], reps, calls=10)
    nbytes = n * (4 * d + d * bits // 8 + 4)  # fp32 vectors + codes + fp32 norms, per direction
    out = {"workload": "4096 vectors x 128 fp32 N(0,1), 3 bits, whole-vector units, fp32 norm per vector",
           "encode_us": round(enc_ms * 1e3, 2), "decode_us": round(dec_ms * 1e3, 2),
           "encode_vectors_per_s": round(n / (enc_ms * 1e-3)), "decode_vectors_per_s": round(n / (dec_ms * 1e-3)),
           "bytes_per_direction": nbytes, "encode_GBs": round(nbytes / (enc_ms * 1e-3) / 1e9, 1),
           "decode_GBs": round(nbytes / (dec_ms * 1e-3) / 1e9, 1)}
    log(f"vectors fp32: encode {enc_ms * 1e3:.2f} us, decode {dec_ms * 1e3:.2f} us per 4096 vectors")
    return out


def bench_llama(tq, torch, dev, reps, flush):
    """The Llama-3.2-1B-shaped cache (16 layers x 8 KV heads x 2048 tokens x head_dim 64 per half, fp16),
    4 bits, one fp16 norm per head vector and norm correction: the four-launch step (quantize K, V,
    dequantize K, V to fp16) timed warm (graph replays back to back; the 170 MB working set stays in the
    last-level cache) and flushed (a 1 GiB read before each step); per-launch times from events between
    the launches of warm steps and of single flushed launches."""
    from synth import workloads

    w = workloads.llama_1b_kv()
    L, H, T, d = w["k"].shape
    rows, bits = L * H * T, 4
    qk = tq.Quantizer(d, d, bits, w["signs_k"], flags=tq.TQ_NORM_CORRECT, codebook=CODEBOOK)
    qv = tq.Quantizer(d, d, bits, w["signs_v"], flags=tq.TQ_NORM_CORRECT, codebook=CODEBOOK)
    k = torch.from_numpy(w["k"].reshape(rows, d)).to(dev)
    v = torch.from_numpy(w["v"].reshape(rows, d)).to(dev)
    ck = torch.empty(rows * d * bits // 8, dtype=torch.uint8, device=dev)
    cv = torch.empty_like(ck)
    nk = torch.empty(rows, dtype=torch.float16, device=dev)
    nv = torch.empty_like(nk)
    ok, ov = torch.empty_like(k), torch.empty_like(v)
    launches = [lambda: tq.tq_quantize(qk, k, rows, d, ck, nk), lambda: tq.tq_quantize(qv, v, rows, d, cv, nv),
                lambda: tq.tq_dequantize(qk, ck, nk, None, None, rows, ok, tq.TQ_F16, d),
                lambda: tq.tq_dequantize(qv, cv, nv, None, None, rows, ov, tq.TQ_F16, d)]

    def step():
        for f in launches:
            f()

    step()
    graph = capture_step(torch, step, [ck, cv, nk, nv, ok, ov])
    run = graph.replay if graph is not None else step
    warm_ms = time_steps(torch, run, reps, 3)
    cold_ms, _ = event_ms(torch, run, reps, before=lambda: flush.sum())
    del graph
    # per launch, warm: events between the launches of back-to-back steps
    torch.cuda.synchronize()
    step()
    ev = []
    for _ in range(reps):
        for f in launches:
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            ev.append(e)
            f()
    ev.append(torch.cuda.Event(enable_timing=True))
    ev[-1].record()
    torch.cuda.synchronize()
    dd = [ev[i].elapsed_time(ev[i + 1]) for i in range(len(ev) - 1)]
    enc_w = sum(dd[i] for i in range(len(dd)) if i % 4 in (0, 1)) / (2 * reps)
    dec_w = sum(dd[i] for i in range(len(dd)) if i % 4 in (2, 3)) / (2 * reps)
    # per launch, flushed
    enc_c, _ = event_ms(torch, launches[0], reps, before=lambda: flush.sum())
    dec_c, _ = event_ms(torch, launches[2], reps, before=lambda: flush.sum())
    per_launch = rows * (2 * d + d * bits // 8 + 2)  # one half: fp16 rows + codes + fp16 norms
    fp16_step = 2 * 2 * rows * d * 2
    res = {"workload": "Llama-3.2-1B-shaped KV, 16 x 8 x 2048 x 64 per half, fp16, 4 bits, per-vector norm + "
                       "norm correction",
           "step_ms_warm": round(warm_ms, 4), "step_ms_flushed": round(cold_ms, 4),
           "GBs_warm": round(fp16_step / (warm_ms * 1e-3) / 1e9, 1),
           "GBs_flushed": round(fp16_step / (cold_ms * 1e-3) / 1e9, 1),
           "algorithmic_bytes_per_launch": per_launch,
           "encode_us_warm": round(enc_w * 1e3, 2), "decode_us_warm": round(dec_w * 1e3, 2),
           "encode_us_flushed": round(enc_c * 1e3, 2), "decode_us_flushed": round(dec_c * 1e3, 2),
           "encode_frac_flushed": round(per_launch / (enc_c * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "decode_frac_flushed": round(per_launch / (dec_c * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "encode_frac_warm": round(per_launch / (enc_w * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "decode_frac_warm": round(per_launch / (dec_w * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "vectors_per_s_flushed": round(2 * 2 * rows / (cold_ms * 1e-3)),
           "vectors_per_s_warm": round(2 * 2 * rows / (warm_ms * 1e-3))}
    log(f"llama-1b 4-bit nc: step {cold_ms * 1e3:.1f} us flushed / {warm_ms * 1e3:.1f} us warm; encode "
        f"{enc_c * 1e3:.1f} / {enc_w * 1e3:.1f} us, decode {dec_c * 1e3:.1f} / {dec_w * 1e3:.1f} us (flushed / warm)")
    return res


def bench_qjl(tq, torch, dev, reps):
    """QJL workload: encode 65536 keys (2-bit MSE + QJL, m = 128), score 4096 queries against them."""
    from synth import workloads

    w = workloads.qjl_keys()
    n, d, m, bits = w["keys"].shape[0], 128, 128, 2
    nq = w["q"].shape[0]
    qz = tq.Quantizer(d, d, bits, w["signs"], flags=tq.TQ_QJL, qjl_m=m, codebook=CODEBOOK)
    params = torch.empty(tq.tq_qjl_params_size(m, d), dtype=torch.uint8, device=dev)
    tq.tq_qjl_prepare(qz, w["S"], params)
    x = torch.from_numpy(w["keys"]).to(dev)
    q = torch.from_numpy(w["q"]).to(dev)
    codes = torch.empty(n * d * bits // 8, dtype=torch.uint8, device=dev)
    norms = torch.empty(n, dtype=torch.float16, device=dev)
    sbits = torch.empty(n * m // 8, dtype=torch.uint8, device=dev)
    rnorm = torch.empty(n, dtype=torch.float16, device=dev)
    scores = torch.empty((nq, n), dtype=torch.float32, device=dev)
    wsb = tq.tq_workspace_size(tq.TQ_OP_QJL_SCORES, qz, nq, n)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def enc():
        tq.tq_quantize(qz, x, n, d, codes, norms, sbits, rnorm)

    def score():
        tq.tq_qjl_scores(qz, q, tq.TQ_F16, nq, d, codes, norms, sbits, rnorm, n, scores, n, ws, wsb)

    for _ in range(2):
        enc()
        score()
    # device time per call from graph replays of several calls (the kernels are far shorter than the host
    # cost of a call)
    enc_ms = graph_ms(torch, enc, [codes, norms, sbits, rnorm], reps, calls=10)
    sc_ms = graph_ms(torch, score, [scores], reps, calls=4)
    key_bytes = n * (d * 2 + d * bits // 8 + 2 + m // 8 + 2)  # fp16 key in; codes, norm, signs, rho out
    n_scores = nq * n
    # int8 MFMA work of the scoring kernel: per score, hi and lo limbs of the rotated query against
    # 2^(b-1) ternary centroid planes, and of the projected query against the sign plane
    macs = n_scores * 2 * ((1 << (bits - 1)) * d + m)
    out = {"workload": "65536 keys x 128 fp16, 2-bit + QJL m=128; 4096 queries",
           "encode_ms": round(enc_ms, 4), "keys_per_s": round(n / (enc_ms * 1e-3)),
           "encode_GBs": round(key_bytes / (enc_ms * 1e-3) / 1e9, 1),
           "scores_ms": round(sc_ms, 4),
           "scores_per_s": round(n_scores / (sc_ms * 1e-3)),
           "scores_write_GBs": round(4 * n_scores / (sc_ms * 1e-3) / 1e9, 1),
           "scores_int8_mfma_TOPS": round(2 * macs / (sc_ms * 1e-3) / 1e12, 1),
           "scores_int8_mfma_frac": round(2 * macs / (sc_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)}
    log(f"qjl: encode {enc_ms:.4f} ms ({out['keys_per_s']:.3g} keys/s), scores {sc_ms:.4f} ms "
        f"({out['scores_per_s']:.3g} scores/s, {out['scores_write_GBs']} GB/s written)")
    return out


def bench_multi(tq, torch, dev, reps, w, kq, vq, plane, H, T, hd, hq, flush):
    """Several query tokens over the same cache: causal chunks of n_q tokens at the end of it (a
    prefill chunk or a batch of draft tokens), n_q x 16 query rows."""
    import synth

    out = {}
    for n_q in (4, 16, 64):
        q = torch.from_numpy(synth.normal_f16(7, 6, n_q * hq * hd).reshape(n_q, hq, hd)).to(dev)
        o = torch.empty((n_q, hq, hd), dtype=torch.float32, device=dev)
        wsb = tq.tq_workspace_size(tq.TQ_OP_MULTI_ATTN, kq, n_q * hq, H, T)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

        def call():
            tq.tq_multi_attn(kq, vq, q, tq.TQ_F16, n_q, hq, H, T, plane["k"][0], plane["k"][1], plane["v"][0],
                             plane["v"][1], True, 0.0, o, ws, wsb)

        call()
        ms, _ = event_ms(torch, call, max(5, reps // 2), before=lambda: flush.sum())
        rows = n_q * hq
        out[f"n_q{n_q}"] = {"us_flushed": round(ms * 1e3, 2), "query_rows": rows,
                            "row_tokens_per_s": round(rows * T / (ms * 1e-3)),
                            "us_per_query_token": round(ms * 1e3 / n_q, 3)}
        log(f"multi-query attention, causal chunk of {n_q} tokens: {ms * 1e3:.1f} us flushed "
            f"({ms * 1e3 / n_q:.2f} us per query token)")
    return out


def bench_attn(tq, torch, dev, reps, kbits=3, vbits=3):
    """Decode attention: 16 query heads over a 131072-token, 4-KV-head, head_dim-256 cache, K and V in
    the block-32 layout (turbo3 by default; kbits=8, vbits=4 is the asymmetric 8-bit-key cache)."""
    from synth import workloads

    w = workloads.decode_cache()
    H, T, hd = w["k"].shape[1], w["k"].shape[2], w["k"].shape[3]
    hq = w["q"].shape[0]
    rows = H * T
    kq = tq.Quantizer(hd, 32, kbits, w["signs_k"], codebook=CODEBOOK)
    vq = tq.Quantizer(hd, 32, vbits, w["signs_v"], codebook=CODEBOOK)
    units = rows * hd // 32
    plane = {}
    for name, qz, b in (("k", kq, kbits), ("v", vq, vbits)):
        x = torch.from_numpy(w[name].reshape(rows, hd)).to(dev)
        plane[name] = (torch.empty(units * 4 * b, dtype=torch.uint8, device=dev),
                       torch.empty(units, dtype=torch.float16, device=dev))
        tq.tq_quantize(qz, x, rows, hd, plane[name][0], plane[name][1])
        del x
    q = torch.from_numpy(w["q"]).to(dev)
    out = torch.empty((hq, hd), dtype=torch.float32, device=dev)
    wsb = tq.tq_workspace_size(tq.TQ_OP_DECODE_ATTN, kq, hq, H, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    # cold-cache runs are preceded by a read of 1 GiB (evicts L2 and the 256 MB MALL without leaving
    # dirty lines whose write-back would land inside the timed kernel)
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)

    def attn():
        tq.tq_decode_attn(kq, vq, q, tq.TQ_F16, hq, H, T, plane["k"][0], plane["k"][1], plane["v"][0],
                          plane["v"][1], 0.0, out, ws, wsb)

    for _ in range(3):
        attn()
    multi = {}
    if kbits == 3 and vbits == 3:
        multi = bench_multi(tq, torch, dev, reps, w, kq, vq, plane, H, T, hd, hq, flush)
    warm_ms = batch_ms(torch, attn, reps)
    cold_ms, cold_min = event_ms(torch, attn, reps, before=lambda: flush.sum())
    nbytes = units * (4 * kbits + 2 + 4 * vbits + 2)  # K and V codes and norms
    fmt = "turbo3 K/V" if kbits == vbits == 3 else f"{kbits}-bit K, {vbits}-bit V"
    res = {"workload": f"decode attention, head_dim 256, 4 KV heads, 16 query heads, 131072 tokens, {fmt}",
           "us_flushed": round(cold_ms * 1e3, 2), "us_warm": round(warm_ms * 1e3, 2),
           "us_min_flushed": round(cold_min * 1e3, 2), "compressed_bytes": nbytes,
           "GBs_flushed": round(nbytes / (cold_ms * 1e-3) / 1e9, 1),
           "GBs_warm": round(nbytes / (warm_ms * 1e-3) / 1e9, 1),
           "frac_hbm_flushed": round(nbytes / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "tokens_per_s_flushed": round(H * T / (cold_ms * 1e-3))}
    if multi:
        res["multi_query"] = multi
    log(f"attn K{kbits}V{vbits}: {cold_ms * 1e3:.1f} us flushed ({res['GBs_flushed']} GB/s), "
        f"{warm_ms * 1e3:.1f} us warm")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a captured step")
    ap.add_argument("--only", choices=("all", "codec", "qjl", "attn", "llama", "vectors"), default="all",
                    help="run one workload (for profiling runs); the JSON line needs 'all'")
    ap.add_argument("--codebook", choices=("gaussian", "beta"), default="gaussian",
                    help="Lloyd-Max codebook for N(0,1/d) (default) or for the exact Beta marginal")
    args = ap.parse_args()
    global CODEBOOK
    CODEBOOK = args.codebook
    if args.gpus != 1:
        print("bench.py measures one GPU: this quantizer's hot path has no cross-GPU step, so a run over "
              "several GPUs would only repeat the one-GPU figure per GPU (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_vector_amd as tq

    tq.lib()
    dev = torch.device("cuda:0")
    reps = max(5, args.steps)
    if args.only in ("qjl", "attn"):
        (bench_qjl if args.only == "qjl" else bench_attn)(tq, torch, dev, reps)
        return
    if args.only == "vectors":
        bench_vectors_fp32(tq, torch, dev, reps)
        return
    if args.only == "llama":
        bench_llama(tq, torch, dev, reps, torch.zeros(1 << 28, dtype=torch.float32, device=dev))
        return
    k, v, signs_k, signs_v, rows = make_cache(tq, torch, dev)
    ok, ov = torch.empty_like(k), torch.empty_like(v)

    # streaming-copy reference on the same buffers (read 1.125 GiB + write 1.125 GiB)
    copy_ms = time_steps(torch, lambda: ok.copy_(k), 10, 2)
    copy_gbs = 2 * k.numel() * 2 / (copy_ms * 1e-3) / 1e9
    log(f"device copy of one half-cache: {copy_ms:.3f} ms ({copy_gbs:.0f} GB/s read+write)")

    def run_codec(bits, tag, sk, sv, keep=None, **kw):
        codec = Codec(tq, torch, dev, rows, bits, sk, sv, **kw)
        launches = codec.launches(k, v, ok, ov)

        def step():
            for f in launches:
                f()

        graph = None if args.no_graph else capture_step(torch, step, codec.outputs() + [ok, ov])
        ms = time_steps(torch, graph.replay if graph is not None else step, args.steps, args.warmup)
        graphed = graph is not None
        del graph
        # per launch: K and V launches of one kernel back to back (the roofline's launch duration), and
        # for reference the same launches timed with events between the step's four launches
        enc_ms = launch_avg_ms(torch, launches[:2], codec.outputs(), max(5, args.steps // 2))
        dec_ms = launch_avg_ms(torch, launches[2:], [ok, ov], max(5, args.steps // 2))
        enc_split, dec_split = per_kernel_ms(torch, codec, k, v, ok, ov, max(5, args.steps // 2))
        if keep is not None:  # the K codes and norms of the first rows, for the oracle's sample
            keep["codes"] = codec.ck[:SAMPLE_ROWS * HEAD_DIM // DT * DT * bits // 8].cpu().numpy()
            keep["norms"] = codec.nk[:SAMPLE_ROWS * HEAD_DIM // DT].cpu().numpy()
            keep["x"] = k[:SAMPLE_ROWS].cpu().numpy()
        ab = algorithmic_bytes(codec.units, bits)
        log(f"{tag} {bits}-bit: step {ms:.3f} ms, encode {enc_ms:.3f} ms ({ab['per_launch'] / enc_ms / 1e6:.0f} GB/s), "
            f"decode {dec_ms:.3f} ms ({ab['per_launch'] / dec_ms / 1e6:.0f} GB/s)")
        del codec
        torch.cuda.empty_cache()
        return {"ms": ms, "enc_ms": enc_ms, "dec_ms": dec_ms, "bytes": ab, "units": ab["fp16"] // 64,
                "graphed": graphed, "enc_split_ms": enc_split, "dec_split_ms": dec_split}

    kept = {}
    results = {bits: run_codec(bits, "block-32", signs_k, signs_v, keep=kept if bits == 3 else None)
               for bits in (3, 4)}
    # the fork's production layout: 128-value chunks, norm copied into 14/18-byte records, Beta codebook
    import synth

    sk128, sv128 = synth.signs(0, synth.STREAM_SIGNS_K, 128), synth.signs(0, synth.STREAM_SIGNS_V, 128)
    fork = {bits: run_codec(bits, "fork records", sk128, sv128, dt=128, records=True, codebook="beta")
            for bits in (3, 4)}
    k8v4 = run_k8v4(tq, torch, dev, rows, k, v, ok, ov, signs_k, signs_v, args)

    if args.only == "codec":
        return
    del k, v, ok, ov
    torch.cuda.empty_cache()
    vectors = bench_vectors_fp32(tq, torch, dev, reps)
    llama = bench_llama(tq, torch, dev, reps, torch.zeros(1 << 28, dtype=torch.float32, device=dev))
    torch.cuda.empty_cache()
    qjl = bench_qjl(tq, torch, dev, reps)
    torch.cuda.empty_cache()
    attn = bench_attn(tq, torch, dev, reps)
    torch.cuda.empty_cache()
    attn["k8v4"] = bench_attn(tq, torch, dev, reps, kbits=8, vbits=4)
    torch.cuda.empty_cache()

    r = results[3]
    fp16_bytes_step = 2 * 2 * r["bytes"]["fp16"]  # K and V, encoded and decoded
    value = fp16_bytes_step / (r["ms"] * 1e-3) / 1e9
    dom = "decode" if r["dec_ms"] >= r["enc_ms"] else "encode"
    dom_ms = max(r["dec_ms"], r["enc_ms"])
    achieved = r["bytes"]["per_launch"] / (dom_ms * 1e-3) / 1e9
    traffic = measured_traffic(f"{dom}_turbo3")
    r4 = results[4]
    out = {
        "metric": "fp16 KV GB/s encoded+decoded (fraction of HBM peak); QJL scores/sec",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "qwen3_8b_kv_block32_turbo3", "layers": LAYERS, "kv_heads": KV_HEADS,
                   "tokens": TOKENS, "head_dim": HEAD_DIM, "block": DT, "bits": 3, "kv_dtype": "f16",
                   "codebook": CODEBOOK,
                   "step": "quantize K, quantize V, dequantize K, dequantize V",
                   "launch": "hip graph of the step's four launches" if results[3]["graphed"] else "eager launches"},
        "roofline": {"bound": "hbm", "kernel": f"{dom} (turbo3, one half-cache per launch)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": r["bytes"]["per_launch"], "avg_launch_ms": round(dom_ms, 4),
                     "launch_timing": "K and V launches back to back in a HIP graph, replays between HIP events",
                     "avg_launch_ms_events_between_step_launches": round(
                         r["dec_split_ms"] if dom == "decode" else r["enc_split_ms"], 4)},
        "fraction_of_hbm_peak": round((2 * 2 * r["bytes"]["per_launch"]) / (r["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "encode": {"turbo3_GBs": round(r["bytes"]["per_launch"] / r["enc_ms"] / 1e6, 1),
                   "turbo4_GBs": round(r4["bytes"]["per_launch"] / r4["enc_ms"] / 1e6, 1),
                   "turbo3_frac": round(r["bytes"]["per_launch"] / r["enc_ms"] / 1e6 / HBM_PEAK_GBS, 4),
                   "turbo4_frac": round(r4["bytes"]["per_launch"] / r4["enc_ms"] / 1e6 / HBM_PEAK_GBS, 4),
                   "turbo3_blocks_per_s": round(r["units"] / (r["enc_ms"] * 1e-3)),
                   "turbo4_blocks_per_s": round(r4["units"] / (r4["enc_ms"] * 1e-3)),
                   "turbo3_ms": round(r["enc_ms"], 4), "turbo4_ms": round(r4["enc_ms"], 4),
                   "turbo3_ms_events_in_step": round(r["enc_split_ms"], 4),
                   "turbo4_ms_events_in_step": round(r4["enc_split_ms"], 4)},
        "decode": {"turbo3_GBs": round(r["bytes"]["per_launch"] / r["dec_ms"] / 1e6, 1),
                   "turbo4_GBs": round(r4["bytes"]["per_launch"] / r4["dec_ms"] / 1e6, 1),
                   "turbo3_frac": round(r["bytes"]["per_launch"] / r["dec_ms"] / 1e6 / HBM_PEAK_GBS, 4),
                   "turbo4_frac": round(r4["bytes"]["per_launch"] / r4["dec_ms"] / 1e6 / HBM_PEAK_GBS, 4),
                   "turbo3_blocks_per_s": round(r["units"] / (r["dec_ms"] * 1e-3)),
                   "turbo4_blocks_per_s": round(r4["units"] / (r4["dec_ms"] * 1e-3)),
                   "turbo3_ms": round(r["dec_ms"], 4), "turbo4_ms": round(r4["dec_ms"], 4),
                   "turbo3_ms_events_in_step": round(r["dec_split_ms"], 4),
                   "turbo4_ms_events_in_step": round(r4["dec_split_ms"], 4)},
        "turbo4_value": round(2 * 2 * r4["bytes"]["fp16"] / (r4["ms"] * 1e-3) / 1e9, 1),
        "fork_layout": {
            "workload": "same cache as 128-value chunks stored as the fork's records (fp16 chunk norm in each "
                        "32-value record + packed codes: 14 B turbo3, 18 B turbo4), Beta codebook for d=128",
            **{f"turbo{b}": {"GBs": round(2 * 2 * fork[b]["bytes"]["fp16"] / (fork[b]["ms"] * 1e-3) / 1e9, 1),
                             "step_ms": round(fork[b]["ms"], 4),
                             "encode_ms": round(fork[b]["enc_ms"], 4), "decode_ms": round(fork[b]["dec_ms"], 4),
                             "encode_GBs": round(fork[b]["bytes"]["per_launch"] / fork[b]["enc_ms"] / 1e6, 1),
                             "decode_GBs": round(fork[b]["bytes"]["per_launch"] / fork[b]["dec_ms"] / 1e6, 1),
                             "encode_frac": round(fork[b]["bytes"]["per_launch"] / fork[b]["enc_ms"] / 1e6
                                                  / HBM_PEAK_GBS, 4),
                             "decode_frac": round(fork[b]["bytes"]["per_launch"] / fork[b]["dec_ms"] / 1e6
                                                  / HBM_PEAK_GBS, 4)}
               for b in (3, 4)}},
        "k8v4": k8v4,
        "copy_reference_GBs": round(copy_gbs, 1),
        "vectors_fp32": vectors,
        "llama_1b": llama,
        "qjl": qjl,
        "attn": attn,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(3, x_rows=kept.get("x"), gpu_codes=kept.get("codes"),
                                           gpu_norms=kept.get("norms"))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
