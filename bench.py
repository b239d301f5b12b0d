#!/usr/bin/env python3
"""CSA decode benchmark on one MI355X: query-tokens/s and achieved HBM GB/s.

A step is one pass of the decode hot path over one batch.  For the CSA workloads the
indexer scores every compressed entry of each query's sequence, keeps the top-512, and
attends over those entries plus the 128-row sliding window (csa_decode, FULL mode);
the CSA2 stack adds five Reuse layers that attend with the same indices over their own
caches.  The CSA2 Reindex stack is the hierarchical indexer: the Full layer selects a
1024-row pool, and each of six layers re-ranks the pool with its own indexer query to
512 rows (csa_reindex_topk; the Full layer with its own query) and attends over them in
its own cache.  The HCA workload attends densely over every row (hca_decode).  The default
workload is the 1M-token context with mixed FP8/BF16 shared-KV rows and FP4 indexer
keys, B = 4 query tokens.  Inputs are synthetic and seed-generated, and resident in HBM
before timing starts; R replicas of every cache (>= 1 GiB in all) rotate across steps so
that the 256 MB Infinity Cache cannot serve a step from the previous one.

Timing: the K timed steps are captured as one hipGraph (torch.cuda.CUDAGraph over the
library's own launches; step i runs on replica i % R), replayed once untimed and once
between HIP events on the current stream.  `protocol` adds the R-step graph (all
replicas) replayed 50 times.  Output: one JSON line.  `roofline` reports the dominant
kernel (the indexer scan, csa_select_scan; for HCA the whole hca_decode): K back-to-back
launches captured and timed the same way, on the stream they run on, as algorithmic GB/s
against 8 TB/s, as algorithmic TFLOP/s against the 2.5 PFLOP/s of dense fp16/bf16 MFMA
(`mfma`), and against the rate a plain streaming read reaches on the same GPU
(`read_probe`).  `cpu_baseline`
times the CPU oracle on a bounded sample of the same workload, on one thread and on
every host core.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "CSA decode query-tokens/s + achieved HBM GB/s, top-512 @1M ctx, 1 GPU"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16 matrix cores (the scan's and attention's MFMA types)
MALL_BYTES = 1 << 30

WORKLOADS = {
    # kind, B, N_c, window, H_q, H_I, top_k, kv format, indexer format, seed, layers
    # (csa: layer 0 runs the indexer, layers 1.. reuse its top-k over their own caches)
    "csa_mixed_1m": dict(kind="csa", B=4, n_c=262144, window=128, hq=64, hi=64, top_k=512,
                         kv="mixed", idx="fp4", seed=4, context=1 << 20, layers=1),
    "csa_fp4h_mixed_1m": dict(kind="csa", B=4, n_c=262144, window=128, hq=64, hi=64, top_k=512,
                              kv="mixed", idx="fp4h", seed=7, context=1 << 20, layers=1),
    "csa_bf16_131k": dict(kind="csa", B=32, n_c=32768, window=128, hq=64, hi=64, top_k=512,
                          kv="bf16", idx="bf16", seed=2, context=131072, layers=1),
    "csa2_stack_fp4_1m": dict(kind="csa", B=8, n_c=262144, window=128, hq=64, hi=64, top_k=512,
                              kv="fp4", idx="fp4", seed=5, context=1 << 20, layers=6),
    "csa2_reindex_fp4_1m": dict(kind="csa2r", B=8, n_c=262144, window=128, hq=64, hi=64,
                                top_k=512, pool=1024, kv="fp4", idx="fp4", seed=5,
                                context=1 << 20, layers=6),
    "hca_bf16_1m": dict(kind="hca", B=16, n_c=8192, window=128, hq=64, hi=0, top_k=0, kv="bf16",
                        idx=None, seed=3, context=1 << 20, layers=1),
}
# HBM traffic of the dominant kernel (the indexer scan) at the default workload, from
# rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs scaled as the summary derives.  Valid only
# while the kernel sources hash to the recorded value.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_scan_csa_mixed_1m_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "compressed_sparse_kv_csa_amd", "csrc", f)
                  for f in ("indexer.hip", "topk_select.h", "csakv_device.h", "csakv_launch.h")]

KV_ROW_BYTES = {"bf16": 1024, "mixed": 576, "fp4": 256 + 32}
IDX_ROW_BYTES = {"bf16": 256, "fp4": 64 + 8, "fp4h": 64 + 8}


def algorithmic_bytes(w: dict) -> dict:
    """Bytes the method itself moves per step (no workspace, re-reads or padding)."""
    B, n_c, k = w["B"], w["n_c"], w["top_k"]
    if w["kind"] == "hca":
        attn = B * ((n_c + w["window"]) * KV_ROW_BYTES[w["kv"]] + 2 * w["hq"] * 512 * 2)
        return {"scan": 0, "indexer": 0, "attention": attn, "step": attn}
    rows = min(k, n_c) + w["window"]
    q_i = w["hi"] * 128 * 2 + w["hi"] * 4
    attn = B * (rows * KV_ROW_BYTES[w["kv"]] + 2 * w["hq"] * 512 * 2)
    if w["kind"] == "csa2r":  # pool select, then per layer: re-rank the pool and attend
        P = w["pool"]
        scan = B * (n_c * IDX_ROW_BYTES[w["idx"]] + q_i)
        idx = B * (n_c * IDX_ROW_BYTES[w["idx"]] + q_i + P * 4)
        reindex = B * (P * IDX_ROW_BYTES[w["idx"]] + q_i + P * 4 + k * 4)
        return {"scan": scan, "indexer": idx, "attention": attn,
                "step": idx + w["layers"] * (reindex + attn + B * k * 4)}
    scan = B * (n_c * IDX_ROW_BYTES[w["idx"]] + q_i)      # the scan reads keys, q_I and w
    idx = scan + B * k * 4                                  # the merge writes topk
    reuse = (w["layers"] - 1) * (attn + B * k * 4)
    return {"scan": scan, "indexer": idx, "attention": attn, "step": idx + attn + reuse}


def algorithmic_flops(w: dict) -> int:
    """Flops of the dominant timed unit: the indexer scan's contraction 2·H_I·128·N_c per
    query, or for HCA the whole attention, 4·H_q·512·rows per query."""
    if w["kind"] == "hca":
        return w["B"] * 4 * w["hq"] * 512 * (w["n_c"] + w["window"])
    return w["B"] * 2 * w["hi"] * 128 * w["n_c"]


READ_PROBE = "row sums of a 2 GiB float32 buffer (torch.sum over rows of 4096), best of 5"


def read_probe_gbps(reps: int = 5, nbytes: int = 2 << 30) -> float:
    """Achieved HBM read bandwidth of a plain streaming read (the row sums of a 2 GiB float32
    buffer viewed as rows of 4096 values; 512 KB written), GB/s, best of `reps` timed
    passes after one untimed pass: the rate a simple read-only kernel reaches on this GPU,
    beside the 8 TB/s specification.  (A full reduction to one value reads more slowly.)"""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda").view(-1, 4096)
    x.sum(dim=1)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        x.sum(dim=1)
        t1.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (t0.elapsed_time(t1) * 1e-3) / 1e9)
    del x
    torch.cuda.empty_cache()
    return best


def build_inputs(w: dict, replicas: int):
    import torch
    import compressed_sparse_kv_csa_amd as ck
    import seedgen

    dev = "cuda"
    T = seedgen.TID
    B, n_c, W = w["B"], w["n_c"], w["window"]
    rows = W + n_c
    kv_fmt = {"bf16": ck.KV_BF16, "mixed": ck.KV_FP8_MIXED, "fp4": ck.KV_FP4}[w["kv"]]

    def kv_cache(layer):
        kv16 = seedgen.kv_rows_bf16(w["seed"], seedgen.tid(T.KV, layer), (B, rows, 512), dev)
        if w["kv"] == "mixed":
            codes = torch.empty((B, rows, 576), dtype=torch.uint8, device=dev)
            ck.kv_quantize_fp8(kv16, B * rows, 512, 448, codes)
            return codes, None
        if w["kv"] == "fp4":
            codes = torch.empty((B, rows, 256), dtype=torch.uint8, device=dev)
            scales = torch.empty((B, rows, 32), dtype=torch.uint8, device=dev)
            ck.kv_quantize_fp4(kv16, B * rows, 512, codes, scales)
            return codes, scales
        return kv16, None

    # One set of caches, generated and quantised on the GPU, then copied per replica.
    kvs = [kv_cache(layer) for layer in range(w["layers"])]
    k_codes = k_scales = None
    if w["kind"] in ("csa", "csa2r"):
        keys16 = seedgen.bf16_normal(w["seed"], seedgen.tid(T.IDX_KEYS), (B, n_c, 128), dev)
        if w["idx"] in ("fp4", "fp4h"):
            k_codes = torch.empty((B, n_c, 64), dtype=torch.uint8, device=dev)
            k_scales = torch.empty((B, n_c, 8), dtype=torch.uint8, device=dev)
            if w["idx"] == "fp4h":
                ck.idx_quantize_fp4_hadamard(keys16, B * n_c, k_codes, k_scales)
            else:
                ck.kv_quantize_fp4(keys16, B * n_c, 128, k_codes, k_scales)
            del keys16
        else:
            k_codes = keys16
    torch.cuda.synchronize()
    reps = []
    for r in range(replicas):
        def cp(t):
            return None if t is None else (t if r == 0 else t.clone())
        rep = {"kv": [], "q": [], "out": []}
        s = w["seed"] * 1000 + r  # distinct queries per replica (their own top-k rows)
        for layer, (codes, scales) in enumerate(kvs):
            c, sc = cp(codes), cp(scales)
            rep["kv"].append(ck.cache(kv_fmt, c, rows, rows, sc))
            rep.setdefault("keep", []).append((c, sc))
            rep["q"].append(seedgen.bf16_normal(s, seedgen.tid(T.Q, layer), (B, w["hq"], 512), dev))
            rep["out"].append(torch.empty((B, w["hq"], 512), dtype=torch.bfloat16, device=dev))
        if w["kind"] == "csa":
            idx_fmt = {"bf16": ck.IDX_BF16, "fp4": ck.IDX_FP4, "fp4h": ck.IDX_FP4_HADAMARD}[w["idx"]]
            rep["kc"], rep["ks"] = cp(k_codes), cp(k_scales)
            rep["idx"] = ck.cache(idx_fmt, rep["kc"], n_c, n_c, rep["ks"])
            rep["qi"] = seedgen.bf16_normal(s, seedgen.tid(T.Q_IDX), (B, w["hi"], 128), dev)
            rep["w"] = seedgen.uniform01(s, seedgen.tid(T.W_IDX), (B, w["hi"]), dev)
            rep["topk"] = torch.empty((B, w["top_k"]), dtype=torch.int32, device=dev)
        if w["kind"] == "csa2r":
            idx_fmt = {"bf16": ck.IDX_BF16, "fp4": ck.IDX_FP4, "fp4h": ck.IDX_FP4_HADAMARD}[w["idx"]]
            rep["kc"], rep["ks"] = cp(k_codes), cp(k_scales)
            rep["idx"] = ck.cache(idx_fmt, rep["kc"], n_c, n_c, rep["ks"])
            rep["qi"] = [seedgen.bf16_normal(s, seedgen.tid(T.Q_IDX, layer), (B, w["hi"], 128), dev)
                         for layer in range(w["layers"])]
            rep["w"] = [seedgen.uniform01(s, seedgen.tid(T.W_IDX, layer), (B, w["hi"]), dev)
                        for layer in range(w["layers"])]
            rep["pool"] = torch.empty((B, w["pool"]), dtype=torch.int32, device=dev)
            rep["topk"] = torch.empty((B, w["top_k"]), dtype=torch.int32, device=dev)
        reps.append(rep)
    torch.cuda.synchronize()
    return reps


def run_gpu(w: dict, steps: int, warmup: int, replicas: int | None):
    import torch
    import compressed_sparse_kv_csa_amd as ck

    nbytes = algorithmic_bytes(w)
    R = replicas or max(2, math.ceil(MALL_BYTES / nbytes["step"]))
    reps = build_inputs(w, R)
    B, scale = w["B"], 1.0 / math.sqrt(512)
    if w["kind"] == "hca":
        rows = w["n_c"] + w["window"]
        ws_bytes = ck.hca_decode_workspace_bytes(B, w["hq"], rows)
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")

        def step(i, sh):
            r = reps[i % R]
            ck.hca_decode(B, w["hq"], scale, r["kv"][0], r["q"][0], r["out"][0], ws, ws_bytes, stream=sh)

        stage, stage_bytes, stage_name = step, nbytes["attention"], "hca_decode (attention + combine)"
        whole, whole_bytes, whole_name = None, None, None
    elif w["kind"] == "csa2r":
        P = w["pool"]
        p_pool = ck.CsaParams(B, w["hq"], w["hi"], P, w["window"], ck.MODE_FULL, scale, 0)
        p_rx = ck.CsaParams(B, 0, w["hi"], w["top_k"], 0, ck.MODE_REINDEX, 1.0, 0)
        p_reuse = ck.CsaParams(B, w["hq"], 0, w["top_k"], w["window"], ck.MODE_REUSE, scale, 0)
        ws_bytes = max(ck.csa_select_topk_workspace_bytes(p_pool, w["n_c"]),
                       ck.csa_decode_workspace_bytes(p_reuse, w["n_c"]))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        rx_bytes = ck.csa_reindex_topk_workspace_bytes(p_rx, P)
        rx_ws = torch.empty(rx_bytes, dtype=torch.uint8, device="cuda")

        def step(i, sh):
            r = reps[i % R]
            ck.csa_select_topk(p_pool, r["idx"], r["qi"][0], r["w"][0], r["pool"], ws, ws_bytes,
                               stream=sh)
            for layer in range(w["layers"]):
                ck.csa_reindex_topk(p_rx, r["idx"], r["qi"][layer], r["w"][layer], r["pool"], P,
                                    r["topk"], rx_ws, rx_bytes, stream=sh)
                ck.csa_decode(p_reuse, r["kv"][layer], None, r["q"][layer], None, None, r["topk"],
                              r["out"][layer], ws, ws_bytes, stream=sh)

        def stage(i, sh):
            r = reps[i % R]
            ck.csa_select_scan(p_pool, r["idx"], r["qi"][0], r["w"][0], ws, ws_bytes, stream=sh)

        def whole(i, sh):
            r = reps[i % R]
            ck.csa_select_topk(p_pool, r["idx"], r["qi"][0], r["w"][0], r["pool"], ws, ws_bytes,
                               stream=sh)

        stage_bytes, stage_name = nbytes["scan"], "indexer_scan_kernel (csa_select_scan, 1024-row pool)"
        whole_bytes, whole_name = nbytes["indexer"], "indexer stage: scan + merge (csa_select_topk)"
    else:
        p = ck.CsaParams(B, w["hq"], w["hi"], w["top_k"], w["window"], ck.MODE_FULL, scale, 0)
        p_reuse = ck.CsaParams(B, w["hq"], 0, w["top_k"], w["window"], ck.MODE_REUSE, scale, 0)
        ws_bytes = ck.csa_decode_workspace_bytes(p, w["n_c"])
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

        def step(i, sh):
            r = reps[i % R]
            ck.csa_decode(p, r["kv"][0], r["idx"], r["q"][0], r["qi"], r["w"], r["topk"], r["out"][0],
                          ws, ws_bytes, stream=sh)
            for layer in range(1, w["layers"]):
                ck.csa_decode(p_reuse, r["kv"][layer], None, r["q"][layer], None, None, r["topk"],
                              r["out"][layer], ws, ws_bytes, stream=sh)

        def stage(i, sh):
            r = reps[i % R]
            ck.csa_select_scan(p, r["idx"], r["qi"], r["w"], ws, ws_bytes, stream=sh)

        def whole(i, sh):
            r = reps[i % R]
            ck.csa_select_topk(p, r["idx"], r["qi"], r["w"], r["topk"], ws, ws_bytes, stream=sh)

        stage_bytes, stage_name = nbytes["scan"], "indexer_scan_kernel (csa_select_scan)"
        whole_bytes, whole_name = nbytes["indexer"], "indexer stage: scan + merge (csa_select_topk)"

    cur = torch.cuda.current_stream

    def timed(fn, n):
        """HIP-event time of fn(i) for i < n on the current stream, ms per call."""
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(cur())
        for i in range(n):
            fn(i)
        t1.record(cur())
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n

    side = torch.cuda.Stream()

    def capture(fn, n):
        """One graph holding fn(0) .. fn(n - 1), launched on the capture stream."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(n):
                fn(i, cur().cuda_stream)
        return g

    def graph_ms(fn, n):
        """ms per call of fn over n calls captured in one graph: one untimed replay, then
        one replay bracketed by HIP events on the current stream."""
        g = capture(fn, n)
        g.replay()
        return timed(lambda i: g.replay(), 1) / n

    # Eager warmup (every replica at least once) and an eager timing for reference.
    for i in range(max(warmup, R)):
        step(i, cur().cuda_stream)
    torch.cuda.synchronize()
    eager_ms = timed(lambda i: step(i, cur().cuda_stream), steps)
    # The K timed steps: one graph of steps 0 .. K-1 (step i on replica i % R).
    ms = graph_ms(step, steps)
    # Protocol: one graph of all R replicas' steps, replayed M >= 50 times.
    g_all = capture(step, R)
    g_all.replay()
    M = 50
    proto_ms = timed(lambda i: g_all.replay(), M) / R
    # The dominant kernel (and its whole stage): K back-to-back launches in one graph.
    stage_ms = graph_ms(stage, steps)
    whole_ms = graph_ms(whole, steps) if whole is not None else None
    return dict(ms=ms, eager_ms=eager_ms, stage_ms=stage_ms, stage_bytes=stage_bytes,
                stage_name=stage_name, whole_ms=whole_ms, whole_bytes=whole_bytes,
                whole_name=whole_name, replicas=R, bytes=nbytes, proto_ms=proto_ms,
                proto_replays=M)


def kernel_sources_sha256() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """Bytes per launch from the committed counter summary, or None if stale or absent."""
    if workload != "csa_mixed_1m" or not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    with open(TRAFFIC_FILE) as f:
        for ln in f:
            if ":" in ln:
                k, v = ln.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


CPU_SAMPLE_SECONDS = 8.0  # each leg of the oracle's sample repeats until it has run this long


def timed_passes(one_pass):
    """Run one_pass until CPU_SAMPLE_SECONDS have elapsed (at least once): (passes, seconds)."""
    n, t0 = 0, time.perf_counter()
    while True:
        one_pass()
        n += 1
        dt = time.perf_counter() - t0
        if dt >= CPU_SAMPLE_SECONDS:
            return n, dt


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def two_legs(one_pass, queries):
    """The oracle's sample timed on one thread, then on every host core (numpy's BLAS
    threads): (rates, passes, seconds, threads of the second leg)."""
    from threadpoolctl import threadpool_info, threadpool_limits
    with threadpool_limits(limits=1):
        p1, d1 = timed_passes(one_pass)
    pn, dn = timed_passes(one_pass)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return (queries * pn / dn, queries * p1 / d1), (pn, p1), (dn, d1), threads


def cpu_record(rates, passes, secs, threads, sample):
    return {"value": round(rates[0], 4), "unit": "query-tokens/s", "cores": int(threads),
            "kind": "oracle", "single_thread_value": round(rates[1], 4),
            "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model(),
            "sample": f"{sample}; {passes[1]} pass(es) in {secs[1]:.1f} s on 1 thread, {passes[0]} in "
                      f"{secs[0]:.1f} s on {threads} threads; numpy fp64"}


def run_cpu_baseline(w: dict, queries: int):
    """The oracle, untuned, on `queries` query tokens of the same workload (seed, shapes)."""
    import numpy as np
    import torch
    import seedgen
    from oracle import decode as OD, formats as OF
    T = seedgen.TID
    n_c, W, k, B = w["n_c"], w["window"], w["top_k"], w["B"]
    dev = "cuda" if torch.cuda.is_available() else "cpu"
    s = w["seed"] * 1000           # replica 0's queries
    scale = 1.0 / math.sqrt(512)

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def encode(row_bits):
        if w["kv"] == "mixed":
            return OF.mixed_quantize(row_bits)
        if w["kv"] == "fp4":
            return OF.fp4_quantize(OF.bf16_bits_to_f64(row_bits))
        return row_bits

    def decode(enc):
        if w["kv"] == "mixed":
            return OF.mixed_dequantize(enc)
        if w["kv"] == "fp4":
            return OF.fp4_dequantize(*enc)
        return OF.bf16_bits_to_f64(enc)

    qs = [seedgen.bf16_normal(s, seedgen.tid(T.Q, layer), (B, w["hq"], 512), dev)[:queries]
          .float().cpu().double().numpy() for layer in range(w["layers"])]

    # Untimed preparation by the oracle's own encoders: every indexer key, and the KV rows
    # the decode reads (window + the oracle's own top-k, in every layer).
    if w["kind"] == "hca":
        kv_all = seedgen.kv_rows_bf16(w["seed"], seedgen.tid(T.KV), (B, W + n_c, 512), dev)
        encs = [encode(bits(kv_all[b])) for b in range(queries)]
        del kv_all
        def one_pass():
            for b in range(queries):
                OD.hca_decode_one(qs[0][b], decode(encs[b]), scale)
        sample = (f"{queries} of the {B} query tokens of one step (same seeds and shapes): dense "
                  f"attention over {W + n_c} {w['kv']} rows each")
        return cpu_record(*two_legs(one_pass, queries), sample)

    if w["kind"] == "csa2r":
        return cpu_baseline_reindex(w, queries, qs, bits, encode, decode)

    qi = seedgen.bf16_normal(s, seedgen.tid(T.Q_IDX), (B, w["hi"], 128), dev)[:queries]
    wv = seedgen.uniform01(s, seedgen.tid(T.W_IDX), (B, w["hi"]), dev)[:queries]
    if w["idx"] == "fp4h":  # the queries as the indexer scores them: rotated, FP4, decoded
        qi = OF.fp4_dequantize(*OF.fp4h_quantize(bits(qi)))
    else:
        qi = qi.float().cpu().double().numpy()
    wv = wv.cpu().double().numpy()
    keys = bits(seedgen.bf16_normal(w["seed"], seedgen.tid(T.IDX_KEYS), (B, n_c, 128), dev)[:queries])
    fp4 = w["idx"] in ("fp4", "fp4h")

    def key_codec(b):
        if w["idx"] == "fp4h":
            return OF.fp4h_quantize(keys[b])
        return OF.fp4_quantize(OF.bf16_bits_to_f64(keys[b])) if fp4 else keys[b]

    key_enc, sels = [], []
    for b in range(queries):
        kc = key_codec(b)
        kd = OF.fp4_dequantize(*kc) if fp4 else OF.bf16_bits_to_f64(kc)
        key_enc.append(kc)
        sels.append(OD.topk_indices(OD.indexer_scores(qi[b], wv[b], kd), k))
    rows_enc = [[None] * queries for _ in range(w["layers"])]
    for layer in range(w["layers"]):
        kv_all = seedgen.kv_rows_bf16(w["seed"], seedgen.tid(T.KV, layer), (B, W + n_c, 512), dev)
        for b in range(queries):
            need = np.concatenate([np.arange(W), W + sels[b][sels[b] >= 0]])
            rows_enc[layer][b] = encode(bits(kv_all[b, torch.from_numpy(need).to(kv_all.device)]))
        del kv_all

    def one_pass():
        for b in range(queries):
            kd = OF.fp4_dequantize(*key_enc[b]) if fp4 else OF.bf16_bits_to_f64(key_enc[b])
            OD.topk_indices(OD.indexer_scores(qi[b], wv[b], kd), k)
            for layer in range(w["layers"]):
                OD.attention(qs[layer][b], decode(rows_enc[layer][b]), scale)
    layers = f" in each of {w['layers']} layers" if w["layers"] > 1 else ""
    sample = (f"{queries} of the {B} query tokens of one step (same seeds and shapes): "
              f"{n_c} {w['idx']} indexer keys each, then {W}+{k} {w['kv']} rows{layers}")
    return cpu_record(*two_legs(one_pass, queries), sample)


def cpu_baseline_reindex(w, queries, qs, bits, encode, decode):
    """The oracle on the CSA2 Reindex stack: the Full layer's pool, then per layer the
    re-ranked top-k and the attention over it (same seeds and shapes as the GPU run)."""
    import numpy as np
    import torch
    import seedgen
    from oracle import decode as OD, formats as OF
    T = seedgen.TID
    n_c, W, k, B, P = w["n_c"], w["window"], w["top_k"], w["B"], w["pool"]
    dev = "cuda" if torch.cuda.is_available() else "cpu"
    s = w["seed"] * 1000
    scale = 1.0 / math.sqrt(512)
    qi = [seedgen.bf16_normal(s, seedgen.tid(T.Q_IDX, layer), (B, w["hi"], 128), dev)[:queries]
          .float().cpu().double().numpy() for layer in range(w["layers"])]
    wv = [seedgen.uniform01(s, seedgen.tid(T.W_IDX, layer), (B, w["hi"]), dev)[:queries]
          .cpu().double().numpy() for layer in range(w["layers"])]
    keys = bits(seedgen.bf16_normal(w["seed"], seedgen.tid(T.IDX_KEYS), (B, n_c, 128), dev)[:queries])
    kds = [OF.fp4_dequantize(*OF.fp4_quantize(OF.bf16_bits_to_f64(keys[b]))) for b in range(queries)]
    # Untimed: the rows each layer reads, encoded by the oracle's own encoders.
    rows_enc = [[None] * queries for _ in range(w["layers"])]
    for b in range(queries):
        pool = OD.topk_indices(OD.indexer_scores(qi[0][b], wv[0][b], kds[b]), P)
        for layer in range(w["layers"]):
            sel = OD.reindex_topk(qi[layer][b], wv[layer][b], kds[b], pool, k)
            kv_all = seedgen.kv_rows_bf16(w["seed"], seedgen.tid(T.KV, layer), (B, W + n_c, 512), dev)
            need = np.concatenate([np.arange(W), W + sel[sel >= 0]])
            rows_enc[layer][b] = encode(bits(kv_all[b, torch.from_numpy(need).to(kv_all.device)]))
            del kv_all
    def one_pass():
        for b in range(queries):
            pool = OD.topk_indices(OD.indexer_scores(qi[0][b], wv[0][b], kds[b]), P)
            for layer in range(w["layers"]):
                OD.reindex_topk(qi[layer][b], wv[layer][b], kds[b], pool, k)
                OD.attention(qs[layer][b], decode(rows_enc[layer][b]), scale)
    sample = (f"{queries} of the {B} query tokens of one step (same seeds and shapes): "
              f"{n_c} {w['idx']} indexer keys -> a {P}-row pool, then in each of "
              f"{w['layers']} layers the pool re-ranked to {k} and {W}+{k} {w['kv']} rows")
    return cpu_record(*two_legs(one_pass, queries), sample)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="csa_mixed_1m", choices=sorted(WORKLOADS))
    ap.add_argument("--replicas", type=int, default=None)
    ap.add_argument("--cpu-queries", type=int, default=None,
                    help="query tokens in the oracle sample (default: one step's batch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the streaming read-bandwidth probe (for counter-collection runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (HIP device) to run.", file=sys.stderr)
        sys.exit(1)
    w = WORKLOADS[args.workload]
    g = run_gpu(w, args.steps, args.warmup, args.replicas)
    B = w["B"]
    tok_s = B / (g["ms"] * 1e-3)
    step_gbps = g["bytes"]["step"] / (g["ms"] * 1e-3) / 1e9
    stage_gbps = g["stage_bytes"] / (g["stage_ms"] * 1e-3) / 1e9
    whole_gbps = (g["whole_bytes"] / (g["whole_ms"] * 1e-3) / 1e9) if g["whole_ms"] else None
    probe = None if args.no_read_probe else read_probe_gbps()
    stage_tflops = algorithmic_flops(w) / (g["stage_ms"] * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(w, args.cpu_queries or B)
    line = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(g["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "context_tokens": w["context"],
                   "n_compressed": w["n_c"], "top_k": w["top_k"], "window": w["window"],
                   "q_heads": w["hq"], "idx_heads": w["hi"], "kv_format": w["kv"],
                   "idx_format": w["idx"], "layers": w["layers"], "replicas": g["replicas"],
                   **({"pool": w["pool"]} if "pool" in w else {})},
        "hbm_gbps": round(step_gbps, 1),
        "algorithmic_bytes_per_step": g["bytes"]["step"],
        "timing": {"k_steps_in_one_graph": True, "eager_ms_per_step": round(g["eager_ms"], 5)},
        "protocol": {"replicas": g["replicas"], "replays": g["proto_replays"],
                     "ms_per_step": round(g["proto_ms"], 5),
                     "query_tokens_per_s": round(B / (g["proto_ms"] * 1e-3), 1)},
        "roofline": {"bound": "hbm", "achieved": round(stage_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(stage_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(args.workload),
                     "kernel": g["stage_name"],
                     "avg_launch_us": round(g["stage_ms"] * 1e3, 2),
                     "algorithmic_bytes_per_launch": g["stage_bytes"],
                     "mfma": {"achieved_tflops": round(stage_tflops, 1), "peak_tflops": MFMA_PEAK_TFLOPS,
                              "frac": round(stage_tflops / MFMA_PEAK_TFLOPS, 4),
                              "algorithmic_flops_per_launch": algorithmic_flops(w)},
                     "read_probe": (None if probe is None else
                                    {"gbps": round(probe, 1), "frac_of_peak": round(probe / HBM_PEAK_GBPS, 4),
                                     "frac_achieved_of_probe": round(stage_gbps / probe, 4),
                                     "kernel": READ_PROBE}),
                     **({"stage": {"kernels": g["whole_name"],
                                   "avg_launch_us": round(g["whole_ms"] * 1e3, 2),
                                   "algorithmic_bytes_per_launch": g["whole_bytes"],
                                   "achieved": round(whole_gbps, 1),
                                   "frac": round(whole_gbps / HBM_PEAK_GBPS, 4)}}
                        if g["whole_ms"] is not None else {})},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
