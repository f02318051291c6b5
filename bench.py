"""Benchmark of the QJL KV-cache hot path on one MI355X.

One step = the serving step of one layer: quantize the newly generated token's key (1-bit JL sketch
+ fp16 norms + outlier sketch) and value (token-wise 2-bit) of every sequence into slot N-1 of the
cache, then decode attention of every query head over all N cached tokens (query projection,
estimator scores, online softmax, value aggregation, split merge).  The cache of the first N-1
tokens is built by the library's own prefill quantization before timing; inputs are resident in HBM.

The headline workload is the largest single-GPU decode (Llama-3.1-70B shape: B=16, 64 query / 8 KV
heads, N=131072); the Llama-2-7B and Llama-3-8B decode shapes are reported beside it, each with its own
roofline, and the prefill quantize stream (65536 tokens x 8 KV heads) after them.

Prints ONE JSON line.  value = keys scored per second = B * Hq * N / step time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import seeded_inputs as si  # noqa: E402

METRIC = "decode keys scored/sec (QJL attention) + % of MI355X HBM peak; quantize tok/s"
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0     # MI355X dense bf16
BYTES_PER_TOKEN_HEAD = 104          # 64 B signs + 4 B norms + 32 B codes + 4 B (min, step)
DECODE_SOURCES = [os.path.join(ROOT, "bit_kv_cache_qjl_amd", "csrc", f) for f in
                  ("qjl_decode.hip", "qjl_decode_mfma.hip", "qjl_decode_common.h", "qjl_common.h")]
DECODE_KERNEL = "decode_mfma"          # name prefix of the matrix-core decode kernels (counter records)
DECODE_KERNEL_VECTOR = "decode_kernel"  # the vector-unit (byte-table) decode


def mfma_decode_kernel(w: si.Workload) -> str:
    """The matrix-core decode kernel a workload runs: eight waves over two row groups of four query
    heads when a KV head has more than four (2-bit codes), else four waves."""
    return "decode_mfma8_kernel" if (w.g > 4 and w.nbits == 2) else "decode_mfma_kernel"
HEADLINE = "llama31_70b_gqa_decode"
DECODE_WORKLOADS = ("llama31_70b_gqa_decode", "llama2_7b_decode", "llama3_8b_gqa_decode")
PATHS = {"auto": 0, "mfma": 1, "valu": 2}
# the arithmetic each decode path computes in (bf16 keys, queries and JL matrices in; fp32 accumulation)
DTYPE = {"mfma": "bf16 in; 1-bit keys x fp6e2m3x4 query, 2-bit values x fp8e4m3x3 weights on f8f6f4 MFMA; fp32 acc",
         "valu": "bf16 in; 1-bit keys x fp32 byte tables, 2-bit values x fp16 weights (v_dot2); fp32 acc"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_{}_traffic.json")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per decode launch from committed rocprofv3 counters, if they match this source."""
    path = TRAFFIC_FILE.format(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("decode_source_sha256_16") != source_hash(DECODE_SOURCES):
        return None
    return t.get("bytes_per_launch")


KERNELS = ("decode", "append_project", "quantize_keys", "quantize_values", "query_project", "combine")
CALIB_BYTES = 1 << 30               # plain copy kernel used to scale FETCH_SIZE / WRITE_SIZE
MALL_BYTES = 256 << 20              # MI355X last-level (Infinity) cache
QUANT_CALLS = 25                    # back-to-back calls per prefill quantize figure
QUANT_WARM_S = 0.040                # each quantize stream first runs this long on its own kernel (>= 8 calls):
                                    # its first tens of launches ride the GPU's clock transient


def _counter_rows(path: str):
    import csv
    with open(path) as f:
        for row in csv.DictReader(f):
            yield row


def _per_dispatch(path: str, counter: str, name_part: str) -> list[float]:
    """Counter value (KiB) of every dispatch whose kernel name contains name_part."""
    acc: dict[str, float] = {}
    for row in _counter_rows(path):
        if row.get("Counter_Name") != counter or name_part not in row.get("Kernel_Name", ""):
            continue
        key = row.get("Dispatch_Id") or row.get("Correlation_Id")
        acc[key] = acc.get(key, 0.0) + float(row["Counter_Value"])
    return list(acc.values())


def write_traffic(fetch_csv: str, write_csv: str, workload: str) -> int:
    """HBM bytes per decode launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the decode kernel,
    each scaled by what the same counter reads for the plain copy of CALIB_BYTES bytes."""
    import statistics
    copy_f = _per_dispatch(fetch_csv, "FETCH_SIZE", "copyBuffer")      # the runtime's device-to-device blit
    copy_w = _per_dispatch(write_csv, "WRITE_SIZE", "copyBuffer")
    big_f = max(copy_f)
    big_w = max(copy_w)
    kf = CALIB_BYTES / (big_f * 1024.0)
    kw = CALIB_BYTES / (big_w * 1024.0)
    dec_f = statistics.mean(_per_dispatch(fetch_csv, "FETCH_SIZE", DECODE_KERNEL))
    dec_w = statistics.mean(_per_dispatch(write_csv, "WRITE_SIZE", DECODE_KERNEL))
    w = si.WORKLOADS[workload]
    rec = {"workload": workload, "kernel": mfma_decode_kernel(si.WORKLOADS[workload]),
           "decode_source_sha256_16": source_hash(DECODE_SOURCES),
           "fetch_kib_per_launch": dec_f, "write_kib_per_launch": dec_w,
           "copy_fetch_kib": big_f, "copy_write_kib": big_w, "copy_bytes": CALIB_BYTES,
           "read_scale": kf, "write_scale": kw,
           "bytes_per_launch": dec_f * 1024.0 * kf + dec_w * 1024.0 * kw,
           "algorithmic_bytes": float(BYTES_PER_TOKEN_HEAD) * w.B * w.Hkv * w.N}
    out = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))
    return 0


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([1] + [int(i.get("num_threads", 1)) for i in threadpool_info()])
    except Exception:  # pragma: no cover
        return 1


def _quality(s_est, s_exact, o_qjl, o_keys_only, o_exact) -> dict:
    """Estimator quality of sampled heads against unquantized attention (reporting only)."""
    s_est, s_exact = np.concatenate(s_est), np.concatenate(s_exact)
    cos = lambda a, b: float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))  # noqa: E731
    c_all = [cos(a, b) for a, b in zip(o_qjl, o_exact)]
    c_keys = [cos(a, b) for a, b in zip(o_keys_only, o_exact)]
    rmse = float(np.sqrt(np.mean((s_est - s_exact) ** 2)))
    return {"score_rmse": rmse, "score_rmse_rel": rmse / float(np.sqrt(np.mean(s_exact ** 2))),
            "score_corr": float(np.corrcoef(s_est, s_exact)[0, 1]),
            "output_cosine_mean": float(np.mean(c_all)), "output_cosine_min": float(np.min(c_all)),
            "output_cosine_keys_only_mean": float(np.mean(c_keys)), "heads": len(c_all), "keys": int(s_est.size)}


def _unit_quality(w: si.Workload, oidx, S_in, S_out, Q, b: int, h: int, kq=None, vhat=None, k=None, v=None):
    """Quality terms of one (sequence, KV head): estimator scores against <q, k>, and the decode output
    (1-bit keys + quantized values; 1-bit keys + exact values) against exact attention."""
    import oracle
    k = si.key_slice(w, b, h, oidx) if k is None else k
    v = si.value_slice(w, b, h) if v is None else v
    if kq is None:
        kq = oracle.quantize_key_vectors(k, S_in, S_out, oidx[h])
        codes, meta = oracle.quantize_value_vectors(v, w.nbits)
        vhat = oracle.dequantize_value_vectors(codes, meta)
    sm = 1.0 / math.sqrt(w.d)
    out = ([], [], [], [], [])
    for i in range(w.g):
        q = Q[b, h * w.g + i]
        sq_in, sq_out = oracle.project_query(q, S_in, S_out, oidx[h])
        s = oracle.estimator_scores(sq_in, sq_out, kq["bits"], kq["norms"])
        out[0].append(s)
        out[1].append(np.asarray(k, np.float64) @ np.asarray(q, np.float64))
        out[2].append(oracle.attend(s, vhat, sm))
        out[3].append(oracle.attend(s, v, sm))
        out[4].append(oracle.exact_attention(q, k, v, sm))
    return out


def cpu_baseline(w: si.Workload, budget_s: float) -> tuple[dict, dict]:
    """The oracle, as it stands, on a bounded sample of the same workload: whole (sequence, KV head)
    units (quantize their keys and values, then decode every query head of the unit), until the
    time budget is spent.  The estimator quality of those units is computed afterwards (untimed)."""
    import oracle
    oidx = si.outlier_channels(w)
    S_in, S_out = si.jl_matrices(w)
    Q = si.queries(w)
    g = w.g
    done = []
    elapsed = 0.0
    for b, h in [(b, h) for b in range(w.B) for h in range(w.Hkv)]:
        k = si.key_slice(w, b, h, oidx)
        v = si.value_slice(w, b, h)
        t0 = time.perf_counter()
        kq = oracle.quantize_key_vectors(k, S_in, S_out, oidx[h])
        codes, meta = oracle.quantize_value_vectors(v, w.nbits)
        vhat = oracle.dequantize_value_vectors(codes, meta)
        for i in range(g):
            sq_in, sq_out = oracle.project_query(Q[b, h * g + i], S_in, S_out, oidx[h])
            s = oracle.estimator_scores(sq_in, sq_out, kq["bits"], kq["norms"])
            oracle.attend(s, vhat, 1.0 / math.sqrt(w.d))
        elapsed += time.perf_counter() - t0
        done.append((b, h, k, v, kq, vhat))
        if elapsed >= budget_s and len(done) >= 2:
            break
    keys = len(done) * g * w.N
    terms = ([], [], [], [], [])
    for b, h, k, v, kq, vhat in done[:2]:
        for acc, part in zip(terms, _unit_quality(w, oidx, S_in, S_out, Q, b, h, kq, vhat, k, v)):
            acc.extend(part)
    base = {"value": keys / elapsed, "unit": "keys/s", "cores": _blas_threads(), "kind": "oracle",
            "host_cores": len(os.sched_getaffinity(0)), "host_cpu_count": os.cpu_count(),
            "sample": f"{len(done)} of {w.B * w.Hkv} (sequence, KV head) units of {w.name} "
                      f"(key + value quantization and decode of all {g} query heads over N={w.N}), "
                      f"{elapsed:.1f} s of oracle time; numpy fp64 with {_blas_threads()} BLAS threads for the "
                      "matrix products, the rest on one core"}
    return base, {w.name: {"units": [(b, h) for b, h, *_ in done[:2]], **_quality(*terms)}}


def estimator_quality(w: si.Workload, unit=(0, 0)) -> dict:
    """Quality of one sampled (sequence, KV head) unit of a workload (reporting only)."""
    oidx = si.outlier_channels(w)
    S_in, S_out = si.jl_matrices(w)
    Q = si.queries(w)
    terms = _unit_quality(w, oidx, S_in, S_out, Q, *unit)
    return {"units": [list(unit)], **_quality(*terms)}


def _timer_run(qjl, torch, names, run_one, steps: int) -> dict:
    """HIP-event durations (recorded by the library on each launch's stream) over `steps` calls."""
    qjl.timer_enable(True)
    for k in names:
        qjl.timer_read(k)
    for _ in range(steps):
        run_one()
    torch.cuda.synchronize()
    res = {k: qjl.timer_read(k) for k in names}
    qjl.timer_enable(False)
    return res


def _region_ms(torch, run_one, steps: int) -> tuple:
    """Mean duration of one call over `steps` back-to-back calls: HIP events on the launch stream (torch's
    current stream, which the binding launches on) bracket the whole run, so the figure is the rate a
    stream of such calls sustains (the key quantizer's launches slow down over a run as the clock drops
    under matrix-core load).  Returns (event ms, host wall-clock ms) per call of the same run."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        run_one()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    return e0.elapsed_time(e1) / steps, wall


def _warm(torch, run_one, min_calls: int) -> int:
    """Back-to-back calls of one stream until QUANT_WARM_S of its work has run (at least min_calls)."""
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while n < min_calls or time.perf_counter() - t0 < QUANT_WARM_S:
        for _ in range(8):
            run_one()
        n += 8
        torch.cuda.synchronize()
    return n


def bench_quantize(qjl, torch, steps: int) -> dict:
    """Prefill quantize stream: 65536 tokens x 8 KV heads, m = m_out = 512 (keys), 2-bit values.  Each
    call takes the next of several input and output copies, so that no call finds its inputs (134 MB
    of keys or values) or its outputs in the 256 MiB last-level cache."""
    w = si.WORKLOADS["prefill_quantize_64k"]
    oidx = si.outlier_channels(w)
    S_in, S_out = si.jl_matrices(w)
    K0 = torch.from_numpy(si.keys(w, oidx)).cuda().to(torch.bfloat16)
    Si = torch.from_numpy(S_in).cuda().to(torch.bfloat16)
    So = torch.from_numpy(S_out).cuda().to(torch.bfloat16)
    od = torch.from_numpy(oidx).cuda()
    in_bytes = K0.numel() * K0.element_size()
    copies = max(2, math.ceil(2 * MALL_BYTES / in_bytes))
    Ks = [K0] + [K0.clone() for _ in range(copies - 1)]
    caches = [qjl.alloc_cache(w.B, w.Hkv, w.N, w.m, w.m_out, w.nbits) for _ in range(copies)]
    turn = [0]

    def keys_once():
        i = turn[0] % copies
        turn[0] += 1
        qjl.quantize_keys(Ks[i], Si, So, od, caches[i].bits, caches[i].norms)
    _warm(torch, keys_once, 2 * copies)
    kern_ms, wall_ms = _region_ms(torch, keys_once, steps)
    kern_s = kern_ms / 1e3
    # outlier-channel selection over the same keys (one read of K, two launches)
    ws = torch.empty(qjl.lib.qjl_select_outliers_workspace_size(w.B, w.N, w.Hkv, w.d), dtype=torch.uint8, device="cuda")
    sel = torch.empty((w.Hkv, w.n_out), dtype=torch.int32, device="cuda")

    def select_once():
        i = turn[0] % copies
        turn[0] += 1
        qjl.select_outliers(Ks[i], w.n_out, sel, workspace=ws)
    _warm(torch, select_once, 2 * copies)
    sel_s = _region_ms(torch, select_once, steps)[0] / 1e3
    sel_bytes = float(in_bytes)
    del Ks, K0
    # token-wise value codes of the same prefill: V [1, 65536, 8, 128] bf16 -> 2-bit code tiles + (min, step)
    V0 = torch.from_numpy(si.values(w)).cuda().to(torch.bfloat16)
    Vs = [V0] + [V0.clone() for _ in range(copies - 1)]

    def values_once():
        i = turn[0] % copies
        turn[0] += 1
        qjl.quantize_values(Vs[i], w.nbits, caches[i].codes, caches[i].meta)
    _warm(torch, values_once, 2 * copies)
    val_s = _region_ms(torch, values_once, steps)[0] / 1e3
    del Vs, V0
    # per token and KV head: d bf16 values read, d b / 8 code bytes and the fp16 (min, step) pair written
    val_bytes = float(w.B * w.N * w.Hkv * (2 * w.d + w.d * w.nbits // 8 + 4))
    tokens = w.B * w.N
    flops = 2.0 * w.d * w.m * tokens * w.Hkv          # inlier (d - n_out) m + outlier n_out m_out = d m MACs
    return {"workload": f"{w.name}: B={w.B} T={w.N} Hkv={w.Hkv} d={w.d} m=m_out={w.m} n_out={w.n_out}",
            "input_copies": copies, "tok_per_s": tokens / kern_s, "key_vectors_per_s": tokens * w.Hkv / kern_s,
            "kernel_ms": kern_s * 1e3, "wall_ms_per_call": wall_ms,
            "mfma": {"bound": "mfma", "achieved": flops / kern_s / 1e12, "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": flops / kern_s / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                     "flops_per_launch": flops},
            "select_outliers": {"kernel_ms": sel_s * 1e3, "bound": "hbm", "achieved": sel_bytes / sel_s / 1e9,
                                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": sel_bytes / sel_s / 1e9 / HBM_PEAK_GBS,
                                "bytes_per_launch": sel_bytes},
            "quantize_values": {"kernel_ms": val_s * 1e3, "tok_per_s": tokens / val_s, "bits": w.nbits, "bound": "hbm",
                                "achieved": val_bytes / val_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": val_bytes / val_s / 1e9 / HBM_PEAK_GBS, "bytes_per_launch": val_bytes}}


def bench_decode(qjl, torch, w: si.Workload, args, path: str) -> dict:
    """Time the serving step of one decode workload; returns its keys/s, step time and roofline."""
    N = w.N
    # algorithmic bytes per cached token and KV head: sign words, two fp16 norms, codes, fp16 (min, step)
    bytes_per_token_head = (w.m + w.m_out) // 8 + 4 + w.d * w.nbits // 8 + 4
    log(f"bench: {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={N} ({path} decode); generating inputs")
    oidx = si.outlier_channels(w)
    S_in_np, S_out_np = si.jl_matrices(w)
    K = torch.from_numpy(si.keys(w, oidx)).cuda().to(torch.bfloat16)
    V = torch.from_numpy(si.values(w)).cuda().to(torch.bfloat16)
    Q = torch.from_numpy(si.queries(w)).cuda().to(torch.bfloat16)
    S_in = torch.from_numpy(S_in_np).cuda().to(torch.bfloat16)
    S_out = torch.from_numpy(S_out_np).cuda().to(torch.bfloat16)
    od = torch.from_numpy(oidx).cuda()
    cache_bytes = bytes_per_token_head * w.B * w.Hkv * N
    copies = args.cache_copies or max(1, math.ceil(3 * MALL_BYTES / cache_bytes))
    caches = []
    for _ in range(copies):
        cache = qjl.alloc_cache(w.B, w.Hkv, N, w.m, w.m_out, w.nbits)
        qjl.quantize_keys(K[:, : N - 1], S_in, S_out, od, cache.bits, cache.norms, t0=0)
        qjl.quantize_values(V[:, : N - 1], w.nbits, cache.codes, cache.meta, t0=0)
        caches.append(cache)
    log(f"bench: {copies} cache cop{'y' if copies == 1 else 'ies'} of {cache_bytes / 1e6:.0f} MB (steps rotate)")
    k_new, v_new = K[:, N - 1:].clone(), V[:, N - 1:].clone()
    del K, V
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    ws = torch.empty(qjl.decode_workspace_size(w.B, w.Hq, w.Hkv, N, w.m, w.m_out, args.nsplit), dtype=torch.uint8,
                     device="cuda")
    if args.calibration_copy:
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()
    pid = PATHS[path]
    turn = [0]

    def step():
        cache = caches[turn[0] % copies]
        turn[0] += 1
        if args.separate_calls:
            qjl.quantize_keys(k_new, S_in, S_out, od, cache.bits, cache.norms, t0=N - 1)
            qjl.quantize_values(v_new, w.nbits, cache.codes, cache.meta, t0=N - 1)
            qjl.decode_attention(Q, S_in, S_out, od, cache.bits, cache.norms, N, out, codes=cache.codes,
                                 meta=cache.meta, nbits=w.nbits, nsplit=args.nsplit, workspace=ws, path=pid)
        else:
            qjl.decode_step(Q, k_new, v_new, S_in, S_out, od, cache, N, out, nsplit=args.nsplit, workspace=ws, path=pid)

    log(f"bench: warmup {args.warmup}, timed {args.steps}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def timed(run_one) -> float:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            run_one()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps * 1e3

    ms_eager = timed(step)
    graph_ok = None
    ms_per_step = ms_eager
    if args.graph:
        # the same launches captured once and replayed (no host launch overhead per kernel); a replay
        # must reproduce the eager step bit for bit before it is timed
        ref_out = out.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for _ in range(copies):             # one graph per cache copy, replayed in rotation
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
            graphs.append(g)
        turn_g = [0]

        def replay():
            graphs[turn_g[0] % copies].replay()
            turn_g[0] += 1
        for _ in range(3 * copies):
            out.zero_()
            torch.cuda.synchronize()
            replay()
            torch.cuda.synchronize()
            graph_ok = bool(torch.equal(out, ref_out))
            if not graph_ok:
                break
        if graph_ok:
            for _ in range(args.warmup):
                replay()
            ms_per_step = timed(replay)
        else:
            log("bench: graph replay differs from the eager step; reporting eager timing")
    # per-kernel durations: HIP events the library records around each launch on its stream, over
    # another args.steps eager steps of the same rotation
    kernels = _timer_run(qjl, torch, KERNELS, step, args.steps)
    keys_scored = w.B * w.Hq * N
    value = keys_scored / (ms_per_step / 1e3)
    n_dec, ms_dec = kernels["decode"]
    dec_s = ms_dec / 1e3 / max(n_dec, 1)
    bytes_alg = float(bytes_per_token_head) * w.B * w.Hkv * N
    achieved = bytes_alg / dec_s / 1e9
    log(f"bench: {w.name} kernel ms/launch " + ", ".join(f"{k}={v[1] / max(v[0], 1):.4f}" for k, v in kernels.items()))
    mfma_kernel = path != "valu"
    return {
        "value": value, "unit": "keys/s", "ms_per_step": ms_per_step,
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "N": N, "m": w.m,
                   "m_out": w.m_out, "n_out": w.n_out, "outlier_scale": w.outlier_scale, "value_bits": w.nbits,
                   "decode_path": path,
                   "step": "append 1 token per sequence (key sketch + value codes) + decode attention over N",
                   "entry_points": ("qjl_quantize_keys + qjl_quantize_values + qjl_decode_attention"
                                    if args.separate_calls or path == "valu" else "qjl_decode_step")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     # counters are taken for the 2-bit matrix-core decode
                     "traffic": measured_traffic(w.name) if (w.nbits == 2 and mfma_kernel) else None,
                     "kernel": mfma_decode_kernel(w) if mfma_kernel else DECODE_KERNEL_VECTOR, "kernel_ms": dec_s * 1e3,
                     "launches_timed": n_dec, "algorithmic_bytes": bytes_alg,
                     "bytes_per_token_kv_head": bytes_per_token_head},
        "kernel_ms_per_launch": {k: v[1] / max(v[0], 1) for k, v in kernels.items()},
        "step_timing": {"mode": "hip_graph_replay" if (graph_ok and args.graph) else "eager",
                        "ms_per_step_eager": ms_eager, "graph_replay_matches_eager": graph_ok,
                        "cache_copies": copies, "cache_bytes": cache_bytes,
                        "nsplit": args.nsplit or "library choice"},
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # decode steps: the first tens of back-to-back launches ride the GPU's clock transient (they slow down,
    # then settle), so the default warm-up runs past it and the timed steps see the sustained rate
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=HEADLINE, choices=list(DECODE_WORKLOADS))
    ap.add_argument("--extra-workloads", default=None,
                    help="comma-separated decode workloads reported beside the headline (default: the other two; "
                         "'' for none)")
    ap.add_argument("--decode-path", default="auto", choices=list(PATHS),
                    help="decode kernels: auto (matrix cores where the shape allows), mfma (matrix cores), valu "
                         "(vector units, byte tables)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work (0 = skip)")
    ap.add_argument("--no-quantize", action="store_true", help="skip the prefill quantize measurement")
    ap.add_argument("--graph", action="store_true",
                    help="time the step captured once in a HIP graph and replayed (after checking that a replay "
                         "reproduces the eager result) instead of eager launches")
    ap.add_argument("--cache-copies", type=int, default=0,
                    help="independent caches the steps rotate through (0: enough that consecutive steps never "
                         f"find their cache in the {MALL_BYTES >> 20} MiB last-level cache)")
    ap.add_argument("--value-bits", type=int, default=0, choices=[0, 2, 3, 4],
                    help="token-wise value code width (0: the workload's, 2 bits)")
    ap.add_argument("--nsplit", type=int, default=0,
                    help="context chunks per (sequence, KV head) of the decode (0: the library's choice)")
    ap.add_argument("--separate-calls", action="store_true",
                    help="run the step as three calls (quantize keys, quantize values, decode attention) instead "
                         "of the one decode-step call")
    ap.add_argument("--quantize-only", action="store_true", help="only the prefill quantize measurement (profiling)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help=f"run one plain {CALIB_BYTES >> 20} MiB device copy first (the reference kernel that "
                         "scales the HBM byte counters of a --pmc profile)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a --calibration-copy "
                         "run into the traffic record under profiles/, then exit")
    args = ap.parse_args()
    if args.traffic_from:
        return write_traffic(*args.traffic_from, args.workload)
    if args.gpus != 1:
        print(f"bench.py: the library and this benchmark run on one GPU only (asked for --gpus {args.gpus}); "
              "sharding decode by (sequence, KV head) across GPUs is not implemented", file=sys.stderr)
        return 2

    import torch
    import bit_kv_cache_qjl_amd as qjl

    if args.quantize_only:
        print(json.dumps(bench_quantize(qjl, torch, args.steps)), flush=True)
        return 0

    extras = ([x for x in DECODE_WORKLOADS if x != args.workload] if args.extra_workloads is None
              else [x for x in args.extra_workloads.split(",") if x])
    for x in extras:
        if x not in DECODE_WORKLOADS:
            raise SystemExit(f"bench.py: unknown workload {x!r}")

    def workload(name):
        w = si.WORKLOADS[name]
        return w.scaled(nbits=args.value_bits) if args.value_bits else w

    path = args.decode_path
    kpath = "valu" if path == "valu" else "mfma"
    head = bench_decode(qjl, torch, workload(args.workload), args, path)
    torch.cuda.empty_cache()
    result = {
        "metric": METRIC, "value": head["value"], "unit": "keys/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE[kpath], "data": "synthetic",
        "config": head["config"], "roofline": head["roofline"],
        "kernel_ms_per_launch": head["kernel_ms_per_launch"], "step_timing": head["step_timing"],
    }
    if extras:
        result["other_decode_workloads"] = {}
        for x in extras:
            r = bench_decode(qjl, torch, workload(x), args, path)
            torch.cuda.empty_cache()
            result["other_decode_workloads"][x] = {k: r[k] for k in ("value", "unit", "ms_per_step", "roofline",
                                                                     "kernel_ms_per_launch", "step_timing")}
    if not args.no_quantize:
        log("bench: prefill quantize stream")
        result["quantize"] = bench_quantize(qjl, torch, QUANT_CALLS)
    if args.cpu_budget > 0:
        log(f"bench: oracle on the host (~{args.cpu_budget:.0f} s), then estimator quality")
        base, quality = cpu_baseline(workload(args.workload), args.cpu_budget)
        for x in extras:
            quality[x] = estimator_quality(workload(x))
        result["cpu_baseline"] = base
        result["estimator_quality"] = {"reference": "unquantized attention (exact <q, k> and fp32 values) on the "
                                                    "same sampled units", **quality}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
