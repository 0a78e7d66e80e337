#!/usr/bin/env python3
"""Throughput of one CSA2 decode step on one MI355X; prints one JSON line.

A step is one pass of the whole hot path over one batch: quantize-and-append
of every sequence's newest row into the FP4 cache, then for every layer of the
workload the index scoring + Top-K (Full / Reindex / Reuse, with the candidate
pool) and the sparse attention over the selected rows.  Inputs are seeded
synthetic tensors (``synth``) resident in HBM before the timed region.

Headline workload: decode_64k_b32 (batch 32, 65536-token contexts, 64 query
heads on one FP4 KV head, indexer 8x64 E4M3 keys, Top-K 2048).  The 1M-token
decode (decode_1m), the 8-layer Full/Reindex/Reuse chain (chain8_256k_b8) and
the 4096-query prefill chunk on a 128K cache (prefill_4k_on_128k, index
product on matrix cores, reported against the fp8 MFMA peak) are measured in
the same run and reported under "extra".

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-extra]
                    [--no-cpu-baseline] [--graph] [--copy-probe MIB]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0      # dense E4M3 matrix-core peak of MI355X
BF16_PEAK_TFLOPS = 2500.0     # dense bf16 matrix-core peak of MI355X
FP16_PEAK_TFLOPS = 2500.0     # dense fp16 matrix-core peak of MI355X
METRIC = "CSA2 decode queries/s and achieved HBM GB/s (% of peak), 64K and 1M context"
MIN_WARMUP_S = 0.3            # the GPU clock needs ~0.3 s of work to ramp
# What the path computes in: every sum is fp32; the operands of the products are
# narrower (and the products exact).
DTYPE = "fp32 (accumulation; operands bf16/E4M3 index, fp16 attention)"
PRECISION = {
    "index_scores": "fp32 fused multiply-adds of the bf16 (or E4M3) index query and the E4M3 or "
                    "bf16 keys, exact products, left-to-right order",
    "prefill_index_product": "E4M3 x E4M3 on matrix cores (exact products), fp32 accumulation",
    "attention": "FP4 rows dequantized exactly to fp16; q rounded to fp16, probabilities fp16; "
                 "fp32 accumulation on matrix cores",
    "cache": "main KV FP4 E2M1 + E4M3 scale per 16 channels; index keys E4M3 or bf16",
}


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--workload", default="decode_64k_b32")
    p.add_argument("--no-extra", action="store_true", help="skip the 1M-context line item")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--proj-append", action="store_true",
                   help="also time csa2_proj_append (d_model 4096) on 4096 and 32 tokens")
    p.add_argument("--local-window", type=int, default=0,
                   help="also time the local window branch (csa2_local_attn) over this many rows")
    p.add_argument("--graph", action="store_true", help="replay the step as a captured graph")
    p.add_argument("--copy-probe", type=int, default=0,
                   help="only run a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


class Hip:
    """hipEvent helpers (the runtime torch already loaded)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def elapsed_ms(self, a, b) -> float:
        f = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return f.value

    def destroy(self, e):
        self.lib.hipEventDestroy(e)

    def record(self, e, stream: int):
        assert self.lib.hipEventRecord(e, ctypes.c_void_p(stream)) == 0


class WorkloadRun:
    """Cache filled with every row but the step's own, inputs resident on the GPU."""

    def __init__(self, wl, dev):
        import numpy as np
        import torch
        import synth
        import sparse_attention_fp4_e2m1_amd as m
        from sparse_attention_fp4_e2m1_amd.pipeline import LayerStack

        self.wl = wl
        t0 = time.time()
        data = synth.gen_batch(wl, threads=16)
        self.gen_s = time.time() - t0
        u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).to(dev)
        self.cache = m.Cache(wl.batch, wl.context, idx_heads=wl.idx_heads, idx_k_dtype=wl.idx_k_dtype)
        pre = wl.context - wl.appended
        for b in range(wl.batch):
            for lo in range(0, pre, 1 << 18):
                hi = min(pre, lo + (1 << 18))
                m.csa2_kv_append(self.cache, u16(data.k[b, lo:hi]), u16(data.v[b, lo:hi]),
                                 u16(data.ik[b, lo:hi]), i32(np.full(hi - lo, b)),
                                 i32(np.arange(lo, hi)))
        rb = np.repeat(np.arange(wl.batch), wl.appended)
        rp = np.tile(np.arange(pre, wl.context), wl.batch)
        self.append = (u16(data.k[rb, rp]), u16(data.v[rb, rp]), u16(data.ik[rb, rp]), i32(rb), i32(rp))
        del data
        qs = [synth.gen_queries(wl, li) for li in range(len(wl.layers))]
        self.q = [u16(x.q) for x in qs]
        self.q_idx = [u16(x.q_idx) for x in qs]
        self.q_seq = i32(wl.query_seq())
        self.q_pos = i32(wl.query_pos())
        self.stack = LayerStack(self.cache, wl.layers, wl.nq, wl.heads, wl.top_k,
                                q_idx_dtype=wl.q_idx_dtype)
        torch.cuda.synchronize()
        self.setup_s = time.time() - t0

    def step(self, scan_events=None, mark=None):
        self.stack.run(self.q, self.q_idx, self.q_seq, self.q_pos, append=self.append,
                       scan_events=scan_events, mark=mark)

    def attn_flops(self, layer: int = 0) -> int:
        """Multiply-adds x 2 of one layer's attention: per query and head,
        q.K over K rows of 128 channels and P.V over the same rows."""
        wl = self.wl
        return 4 * wl.nq * wl.heads * self.stack.k[layer] * 128

    def scan_flops(self) -> int:
        """Multiply-adds x 2 of the first Full layer's index product (every query
        against every visible position, idx_heads x 64 channels)."""
        wl = self.wl
        vis = int((wl.query_pos().astype("int64") + 1).sum())
        return 2 * vis * wl.idx_heads * wl.idx_dim

    # ---- algorithmic bytes (what the method must move; scratch and re-reads excluded)
    def scan_bytes(self) -> int:
        """Index keys streamed by the first Full layer's scoring kernel, plus its queries."""
        wl = self.wl
        vis = int((wl.query_pos().astype("int64") + 1).sum())
        return vis * wl.idx_bytes_per_token() + wl.nq * wl.idx_heads * wl.idx_dim * 2

    def step_bytes(self) -> int:
        wl = self.wl
        nq = wl.nq
        total = 0
        vis = int((wl.query_pos().astype("int64") + 1).sum())
        total += wl.batch * wl.appended * (wl.dk * 2 + wl.dv * 2 + wl.idx_heads * wl.idx_dim * 2)  # append in
        total += wl.batch * wl.appended * (144 + wl.idx_bytes_per_token())                       # append out
        # a dense (matrix-core) product reads each sequence's keys once, not once per query
        seq_vis = {}
        for b, p in zip(wl.query_seq(), wl.query_pos()):
            seq_vis[int(b)] = max(seq_vis.get(int(b), 0), int(p) + 1)
        dense_keys = sum(seq_vis.values()) * wl.idx_bytes_per_token()
        for li, L in enumerate(wl.layers):
            k = self.stack.k[li]
            if L.mode == "full" and matrix_core_scan(wl) and L is wl.layers[0]:
                total += dense_keys
                total += nq * wl.idx_heads * wl.idx_dim * 2
                total += nq * k * 4
            elif L.mode == "full":
                total += vis * wl.idx_bytes_per_token()
                total += nq * wl.idx_heads * wl.idx_dim * 2
                total += nq * k * 4 + (nq * 8 * L.pool_blocks * 4 if L.pool_blocks else 0)
            elif L.mode == "reindex":
                pool = 8 * wl.layers[L.pool_from].pool_blocks if L.pool_from >= 0 else 0
                if pool:
                    total += nq * pool * (wl.idx_bytes_per_token() + 4)
                else:
                    total += dense_keys if matrix_core_scan(wl) else vis * wl.idx_bytes_per_token()
                total += nq * wl.idx_heads * wl.idx_dim * 2 + nq * k * 4
            else:
                pass                                             # Reuse: the source list itself
            total += nq * k * (144 + 4)                          # selected rows + their indices
            total += nq * wl.heads * (wl.dk * 2 + wl.dv * 4 + 4)  # q in, out + lse out
        return total


def matrix_core_scan(wl) -> bool:
    """The first layer is scored on matrix cores (E4M3 index query and keys, no pool)."""
    L = wl.layers[0]
    return (wl.q_idx_dtype == "fp8" and wl.idx_k_dtype == "fp8" and L.mode == "full"
            and L.pool_blocks == 0)


def time_run(run, steps, warmup, hip, use_graph=False):
    """Returns (seconds for the K timed steps, scan ms per launch, step-time
    percentiles, ms per step of the instrumented pass).

    The timed pass holds nothing but the K steps: a HIP event recorded between
    two kernels keeps the GPU idle for a few microseconds, so the events that
    time the index scan (on the stream it runs on) and the step boundaries are
    recorded in a second pass of the same K steps right after it."""
    import torch
    t_warm = time.perf_counter()
    done = 0
    for _ in range(warmup):
        run.step()
        done += 1
    torch.cuda.synchronize()
    # at least MIN_WARMUP_S of steps whatever `warmup` says, so that a short
    # run is not timed on a cold clock
    while time.perf_counter() - t_warm < MIN_WARMUP_S:
        for _ in range(5):
            run.step()
        done += 5
        torch.cuda.synchronize()
    run.warmup_steps = done
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            run.step()
        torch.cuda.current_stream().wait_stream(s)
        with torch.cuda.graph(graph):
            run.step()
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()

    def one(i, scan_events=None, mark=None):
        if graph is not None:
            graph.replay()
        else:
            run.step(scan_events=scan_events, mark=mark)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    # instrumented pass: an event at every step boundary (per-step times for
    # the percentiles) and around every scan launch
    evs = [(hip.event(), hip.event()) for _ in range(steps)]
    aevs = [(hip.event(), hip.event()) for _ in range(steps)]
    bounds = [hip.event() for _ in range(steps + 1)]
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()

    def marker(i):
        def mark(kind, layer, when):   # the first layer's attention call
            if kind == "attn" and layer == 0:
                hip.record(aevs[i][0 if when == "before" else 1], stream)
        return mark

    hip.record(bounds[0], stream)
    for i in range(steps):
        one(i, evs[i], marker(i))
        hip.record(bounds[i + 1], stream)
    torch.cuda.synchronize()
    scan_ms = None
    run.attn_ms = None
    if graph is None:
        scan_ms = sum(hip.elapsed_ms(a, b) for a, b in evs) / steps
        run.attn_ms = sum(hip.elapsed_ms(a, b) for a, b in aevs) / steps
    per_step = sorted(hip.elapsed_ms(bounds[i], bounds[i + 1]) for i in range(steps))
    pct = {f"p{p}": per_step[min(steps - 1, (p * steps) // 100)] for p in (10, 50, 90)}
    inst_ms = hip.elapsed_ms(bounds[0], bounds[steps]) / steps
    for a, b in evs + aevs:
        hip.destroy(a)
        hip.destroy(b)
    for e in bounds:
        hip.destroy(e)
    return (t1 - t0), scan_ms, pct, inst_ms


def source_sha(name: str = "csa2_index.hip") -> str:
    src = os.path.join(ROOT, "sparse_attention_fp4_e2m1_amd", "csrc", name)
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def traffic_for(workload: str):
    """HBM bytes per launch of the workload's dominant kernel from committed
    rocprofv3 counter runs, if they were taken on the current source of that
    kernel (else None)."""
    path = os.path.join(ROOT, "profiles", "index_scan_traffic.json")
    if not os.path.exists(path):
        return None
    doc = json.load(open(path))
    rec = doc.get(workload)
    if not rec:
        return None
    want = rec.get("source_sha", doc.get("kernel_sha"))
    if want != source_sha(rec.get("source", "csa2_index.hip")):
        return None
    return rec.get("hbm_bytes_per_launch")


def measure(name, steps, warmup, hip, use_graph):
    import torch
    import synth
    wl = synth.workload(name)
    dev = torch.device("cuda:0")
    run = WorkloadRun(wl, dev)
    elapsed, scan_ms, pct, inst_ms = time_run(run, steps, warmup, hip, use_graph)
    ms = elapsed * 1e3 / steps
    qps = wl.nq * steps / elapsed
    step_gbps = run.step_bytes() / (elapsed / steps) / 1e9
    res = {
        "value": qps, "ms_per_step": ms, "step_ms_percentiles": pct,
        "instrumented_ms_per_step": inst_ms,
        "step_hbm_gbps": step_gbps, "step_hbm_frac": step_gbps / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": run.step_bytes(),
        "setup_s": round(run.setup_s, 1),
        "layer_top_k": list(run.stack.k),
    }
    res["warmup_steps_run"] = run.warmup_steps
    if scan_ms is not None and matrix_core_scan(wl):
        # the matrix-core scorer: the method's index product (every query
        # against every visible position) counted once, over the time of its
        # product passes and the threshold and checking launches between them
        flops = run.scan_flops()
        ach = flops / (scan_ms * 1e-3) / 1e12
        res["roofline"] = {"bound": "mfma",
                           "kernel": "gemm_score_kernel sampled pass + emitting pass, with the "
                                     "threshold and checking launches between them (fp8 index "
                                     "product, counted once)",
                           "achieved": ach, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": ach / FP8_PEAK_TFLOPS, "traffic": None,
                           "flops_per_launch": flops, "avg_launch_ms": scan_ms}
        if run.attn_ms:
            af = run.attn_flops(0)
            aach = af / (run.attn_ms * 1e-3) / 1e12
            res["attention_roofline"] = {
                "bound": "mfma", "kernel": "attn_partial_kernel + attn_combine_kernel (layer 0)",
                "achieved": aach, "peak": FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": aach / FP16_PEAK_TFLOPS, "flops_per_call": af, "avg_call_ms": run.attn_ms}
    elif scan_ms is not None:
        ach = run.scan_bytes() / (scan_ms * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "kernel": "score_kernel (index scan, first Full layer)",
                           "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": ach / HBM_PEAK_GBPS, "traffic": traffic_for(name),
                           "bytes_per_launch": run.scan_bytes(), "avg_launch_ms": scan_ms}
    del run
    torch.cuda.empty_cache()
    return wl, res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name, n_sample=32, runs=3):
    """The oracle (as it stands) on a bounded sample of the same step: the first
    n_sample queries (the whole batch of the headline workload) with their full
    contexts, one step (the new rows' append, then every layer), on the host's
    cores: a thread pool over the queries (numpy releases the interpreter lock
    inside its array operations; BLAS limited to one thread per worker).  The
    median of `runs` runs."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    import synth
    from oracle import csa2 as O
    wl = synth.workload(name)
    samp = list(range(min(n_sample, wl.nq)))
    oc = O.OracleCache(len(samp), wl.context, idx_heads=wl.idx_heads, idx_k_dtype=wl.idx_k_dtype)
    pre = wl.context - wl.appended
    rows = []
    for i, b in enumerate(samp):
        d = synth.gen_sequence(wl, b, threads=16)
        oc.append(d.k[:pre], d.v[:pre], d.ik[:pre], np.full(pre, i), np.arange(pre))
        rows.append((d.k[pre:], d.v[pre:], d.ik[pre:]))
    qs = []
    for li in range(len(wl.layers)):
        q = synth.gen_queries(wl, li)
        qs.append(synth.QueryData(q.q[samp], q.q_idx[samp]))
    qpos = wl.query_pos()[samp]
    # the machine's CPU share for one GPU is 16 cores, whatever the host reports
    workers = max(1, min(16, os.cpu_count() or 1, len(samp)))

    def one_query(i):
        k, v, ik = rows[i]
        oc.append(k, v, ik, np.full(wl.appended, i), np.arange(pre, wl.context))
        O.run_layers(oc, wl.layers, np.arange(len(samp)), qpos, qs, wl.top_k, wl.q_idx_dtype,
                     only=[i])

    times = []
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        for _ in range(runs):
            t0 = time.perf_counter()
            list(ex.map(one_query, range(len(samp))))
            times.append(time.perf_counter() - t0)
    t = sorted(times)[len(times) // 2]
    return {"value": len(samp) / t, "unit": "queries/s", "cores": workers, "kind": "oracle",
            "cpu": cpu_model(), "host_cpus": os.cpu_count(),
            "runs_s": [round(x, 3) for x in times],
            "sample": f"{len(samp)} of {wl.nq} queries of {name} (full {wl.context}-token "
                      f"contexts), one step incl. append, numpy oracle, {workers} threads over "
                      f"queries; median of {runs} runs {t:.2f} s"}


def local_item(name, window, steps, warmup, hip):
    """The local window branch alone on the workload's queries: every query's
    window full (positions q_pos - window + 1 .. q_pos), merged into a finite
    (out, lse).  Algorithmic bytes per launch: per query the window's K and V
    codes (2 x 128 B per row) and slot positions (4 B per row), the bf16
    queries, and out and lse read and written back in fp32."""
    import numpy as np
    import torch
    import synth
    import sparse_attention_fp4_e2m1_amd as m
    wl = synth.workload(name)
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(11)
    lc = m.LocalCache(wl.batch, window)
    qpos = wl.query_pos()
    for b in range(wl.batch):
        p = np.arange(max(0, int(qpos.max()) - window + 1), int(qpos.max()) + 1)
        rows = rng.standard_normal((2, len(p), 128)).astype(np.float32)
        kv = torch.from_numpy(synth.f32_to_bf16_bits(rows).view(np.int16)).to(dev)
        m.csa2_local_append(lc, kv[0], kv[1], torch.full((len(p),), b, dtype=torch.int32, device=dev),
                            torch.from_numpy(p.astype(np.int32)).to(dev))
    q = torch.from_numpy(synth.gen_queries(wl, 0).q.view(np.int16)).to(dev)
    q_seq = torch.from_numpy(wl.query_seq().astype(np.int32)).to(dev)
    q_pos = torch.from_numpy(qpos.astype(np.int32)).to(dev)
    out = torch.zeros((wl.nq, wl.heads, 128), dtype=torch.float32, device=dev)
    lse = torch.zeros((wl.nq, wl.heads), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        m.csa2_local_attn(lc, q, q_seq, q_pos, out, lse)
    stream = torch.cuda.current_stream().cuda_stream
    a, b = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(a, stream)
    for _ in range(steps):
        m.csa2_local_attn(lc, q, q_seq, q_pos, out, lse)
    hip.record(b, stream)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(a, b) / steps
    hip.destroy(a)
    hip.destroy(b)
    rows = int(np.minimum(qpos + 1, window).sum())
    nbytes = rows * (2 * 128 + 4) + wl.nq * wl.heads * (128 * 2 + 2 * 128 * 4 + 2 * 4)
    ach = nbytes / (ms * 1e-3) / 1e9

    # the sparse branch alone, both branches as two calls, and both in one
    # launch (csa2_sparse_local_attn), over the workload's K rows of a
    # zero-filled FP4 cache of the workload's size (the gather's traffic and
    # the arithmetic do not depend on the values)
    cache = m.Cache(wl.batch, wl.context, idx_heads=wl.idx_heads, idx_k_dtype=wl.idx_k_dtype)
    topk = torch.from_numpy(rng.integers(0, wl.context, (wl.nq, wl.top_k)).astype(np.int32)).to(dev)
    ws_s = torch.empty(max(m.csa2_sparse_attn_workspace(cache, wl.nq, wl.heads, wl.top_k), 256),
                       dtype=torch.uint8, device=dev)
    ws_f = torch.empty(max(int(m.LIB.csa2_sparse_local_attn_workspace(
        cache.ref, lc.ref, wl.nq, wl.heads, wl.top_k)), 256), dtype=torch.uint8, device=dev)

    def sparse():
        m.csa2_sparse_attn(cache, q, q_seq, topk, out=out, lse=lse, workspace=ws_s)

    def two_calls():
        sparse()
        m.csa2_local_attn(lc, q, q_seq, q_pos, out, lse)

    def fused():
        m.csa2_sparse_local_attn(cache, lc, q, q_seq, q_pos, topk, out=out, lse=lse, workspace=ws_f)

    times = {}
    for name, fn in (("sparse_only", sparse), ("sparse_then_local", two_calls), ("fused", fused)):
        for _ in range(warmup):
            fn()
        a, b = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(a, stream)
        for _ in range(steps):
            fn()
        hip.record(b, stream)
        torch.cuda.synchronize()
        times[name + "_ms"] = hip.elapsed_ms(a, b) / steps
        hip.destroy(a)
        hip.destroy(b)
    del cache
    return {"window": window, "queries": wl.nq, "heads": wl.heads, "avg_launch_ms": ms,
            "with_sparse_branch": times,
            "queries_per_s": wl.nq / (ms * 1e-3),
            "roofline": {"bound": "hbm", "kernel": "local_attn_kernel", "achieved": ach,
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                         "traffic": None, "bytes_per_launch": nbytes}}


def proj_item(steps, warmup, hip, d_model=4096):
    """csa2_proj_append alone: n tokens of hidden states (d_model bf16) through
    the 768 x d_model projection (K, V, 8 E4M3 index-key heads) into the cache.
    FLOPs per launch 2 n d_model 768; algorithmic bytes: x and w read once, the
    appended rows (144 B main KV + 512 B index keys) written."""
    import numpy as np
    import torch
    import sparse_attention_fp4_e2m1_amd as m
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(12)
    ch = 256 + 8 * 64
    res = {}
    for n in (4096, 32):
        cache = m.Cache(1, 4096, idx_heads=8, idx_k_dtype="fp8")
        x = torch.from_numpy(rng.standard_normal((n, d_model)).astype(np.float32)).to(dev)
        w = torch.from_numpy((rng.standard_normal((ch, d_model)) / np.sqrt(d_model)).astype(np.float32)).to(dev)
        x, w = x.to(torch.bfloat16), w.to(torch.bfloat16)
        seq = torch.zeros(n, dtype=torch.int32, device=dev)
        pos = torch.arange(n, dtype=torch.int32, device=dev)
        for _ in range(warmup):
            m.csa2_proj_append(cache, x, w, seq, pos)
        stream = torch.cuda.current_stream().cuda_stream
        a, b = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(a, stream)
        for _ in range(steps):
            m.csa2_proj_append(cache, x, w, seq, pos)
        hip.record(b, stream)
        torch.cuda.synchronize()
        ms = hip.elapsed_ms(a, b) / steps
        hip.destroy(a)
        hip.destroy(b)
        flops = 2 * n * d_model * ch
        nbytes = 2 * n * d_model + 2 * ch * d_model + n * (144 + 512) + 8 * n
        tf = flops / (ms * 1e-3) / 1e12
        gb = nbytes / (ms * 1e-3) / 1e9
        res[f"tokens_{n}"] = {"avg_launch_ms": ms, "tokens_per_s": n / (ms * 1e-3),
                              "roofline": {"bound": "mfma",
                                           "kernel": "proj_tile_kernel" if n >= 512
                                           else "proj_append_kernel",
                                           "achieved": tf, "peak": BF16_PEAK_TFLOPS,
                                           "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS,
                                           "traffic": None, "flops_per_launch": flops},
                              "hbm": {"achieved": gb, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                      "frac": gb / HBM_PEAK_GBPS, "bytes_per_launch": nbytes}}
        del cache, x, w
    res["d_model"] = d_model
    return res


def synth_prefill(name) -> bool:
    import synth
    return synth.workload(name).prefill > 0


def copy_probe(mib):
    import torch
    n = mib << 20
    a = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n}), flush=True)


def copy_reference(hip, gib=1, reps=20):
    """A plain 1 GiB device-to-device copy (torch's copy kernel) timed with HIP
    events in the same run: the practical read+write rate the roofline's 8 TB/s
    peak is measured against."""
    import torch
    n = gib << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < MIN_WARMUP_S:
        b.copy_(a)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for _ in range(reps):
        b.copy_(a)
    hip.record(e1, stream)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(e0, e1) / reps
    hip.destroy(e0)
    hip.destroy(e1)
    del a, b
    torch.cuda.empty_cache()
    gbps = 2 * n / (ms * 1e-3) / 1e9
    return {"bytes_copied": n, "avg_ms": ms, "read_plus_write_gbps": gbps,
            "frac_of_peak": gbps / HBM_PEAK_GBPS}


def main():
    args = _args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr, flush=True)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    hip = Hip()
    print(f"[bench] {args.workload}: setup + {args.warmup} warmup + {args.steps} timed steps",
          file=sys.stderr, flush=True)
    wl, res = measure(args.workload, args.steps, args.warmup, hip, args.graph)
    line = {
        "metric": METRIC, "value": res["value"], "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
        "step_ms_percentiles": res["step_ms_percentiles"],
        "instrumented_ms_per_step": res["instrumented_ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE,
        "precision": PRECISION, "warmup_steps_run": res["warmup_steps_run"],
        "data": "synthetic (seeded numpy draws, shapes of the workload)",
        "config": {"workload": wl.name, "batch": wl.batch, "context": wl.context,
                   "heads": wl.heads, "idx_heads": wl.idx_heads, "idx_k_dtype": wl.idx_k_dtype,
                   "top_k": wl.top_k, "layers": [L.mode for L in wl.layers],
                   "layer_top_k": res["layer_top_k"],
                   "graph": bool(args.graph)},
        "step_hbm_gbps": res["step_hbm_gbps"], "step_hbm_frac": res["step_hbm_frac"],
        "roofline": res.get("roofline"),
    }
    if "attention_roofline" in res:
        line["attention_roofline"] = res["attention_roofline"]
    line["copy_reference"] = copy_reference(hip)
    if not args.no_extra:
        line["extra"] = {}
        for name in ("decode_1m", "chain8_256k_b8", "prefill_4k_on_128k", "released_256k_b8",
                     "encoder_4k_on_128k"):
            if name == args.workload:
                continue
            print(f"[bench] {name} line item", file=sys.stderr, flush=True)
            # a prefill step is ~1-2 ms: fewer steps keep its share of the run small
            prefill = synth_prefill(name)
            steps = args.steps if not prefill else max(3, args.steps // 5)
            wl2, res2 = measure(name, steps, args.warmup, hip, args.graph)
            line["extra"][name] = {k: res2[k] for k in
                                   ("value", "ms_per_step", "step_ms_percentiles",
                                    "instrumented_ms_per_step", "step_hbm_gbps", "step_hbm_frac")}
            line["extra"][name]["unit"] = "queries/s"
            line["extra"][name]["steps"] = steps
            line["extra"][name]["roofline"] = res2.get("roofline")
            if "attention_roofline" in res2:
                line["extra"][name]["attention_roofline"] = res2["attention_roofline"]
    if args.proj_append:
        print("[bench] projection + append", file=sys.stderr, flush=True)
        line["proj_append"] = proj_item(args.steps, args.warmup, hip)
    if args.local_window:
        print(f"[bench] local window branch, {args.local_window} rows", file=sys.stderr, flush=True)
        line["local_window_branch"] = local_item(args.workload, args.local_window, args.steps,
                                                 args.warmup, hip)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
