"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (its WorkloadRun: the same cache fill, step and layer stack).  The GPU
runs the whole batch; the oracle recomputes queries one by one (their
sequences regenerated from the same seeds) and checks Top-K sets, pools and
attention, plus the appended rows and a random sample of cache rows byte for
byte.  The headline workload (batch 32 at 65536 positions) is checked on every
query; the others, whose oracle runs take minutes per query, on samples."""
import numpy as np
import pytest
import torch

import synth
from oracle import csa2 as O
from gpu_util import DEV, announce, check_stack, host, untile_idx

pytestmark = pytest.mark.gpu

SAMPLES = {
    "decode_64k_b32": list(range(32)),   # the whole batch
    "decode_1m": [0],
    "chain8_256k_b8": [5],
    "prefill_4k_on_128k": [0, 1365, 2730, 4095],
    "released_256k_b8": [3],
    "encoder_4k_on_128k": [0, 2047, 4095],
}


@pytest.mark.parametrize("name", list(SAMPLES))
def test_full_size_sampled_queries(name):
    import bench
    wl = synth.workload(name)
    announce(f"full size {name}: setup")
    run = bench.WorkloadRun(wl, DEV)
    run.step()
    torch.cuda.synchronize()
    announce(f"full size {name}: GPU step done, oracle on queries {SAMPLES[name]}")

    queries = SAMPLES[name]
    seqs = sorted({int(wl.query_seq()[i]) for i in queries})
    oc = O.OracleCache(len(seqs), wl.context, idx_heads=wl.idx_heads, idx_k_dtype=wl.idx_k_dtype,
                       lazy=True)
    rng = np.random.default_rng(0)
    for j, b in enumerate(seqs):
        d = synth.gen_sequence(wl, b, threads=16)
        oc.append(d.k, d.v, d.ik, np.full(wl.context, j), np.arange(wl.context))
        # cache bytes: the step's appended rows and a random sample of the rest
        rows = np.unique(np.concatenate([np.arange(wl.context - wl.appended, wl.context),
                                         rng.integers(0, wl.context, 512)]))
        kc, ks = O.quantize_rows(d.k[rows])
        vc, vs = O.quantize_rows(d.v[rows])
        assert np.array_equal(host(run.cache.kv_codes[b])[rows], np.concatenate([kc, vc], 1))
        assert np.array_equal(host(run.cache.kv_scales[b])[rows], np.concatenate([ks, vs], 1))
        gik = untile_idx(host(run.cache.idx_k[b:b + 1]), wl.idx_heads, oc.idx_k.dtype)[0]
        assert np.array_equal(gik[rows], oc.idx_k[j][rows])
    seq_of = {b: j for j, b in enumerate(seqs)}
    qs = []
    for li in range(len(wl.layers)):
        q = synth.gen_queries(wl, li)
        qs.append(synth.QueryData(q.q[queries], q.q_idx[queries]))
    ref = O.run_layers(oc, wl.layers, np.array([seq_of[int(wl.query_seq()[i])] for i in queries]),
                       wl.query_pos()[queries], qs, wl.top_k, wl.q_idx_dtype)
    stack = run.stack
    rows = [(i, r, seq_of[int(wl.query_seq()[i])]) for r, i in enumerate(queries)]
    check_stack(wl, oc, stack, ref, [synth.gen_queries(wl, li) for li in range(len(wl.layers))],
                rows, log=announce)
    del run, stack
    torch.cuda.empty_cache()
