"""A layer-stack step captured in a HIP graph and replayed: every replay gives
the eager step's results bit for bit (Top-K lists, pools, attention outputs,
lse and the appended cache rows).  Replays alternate with eager work of the
program's own (another step through the library on other buffers) and with
synchronizations, since graph replays after the first have gone wrong on
this platform when a captured node misbehaves.  The step holds no memset and
no torch operation: only the library's kernels."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import announce, dev_i32, dev_u16, host, lib

pytestmark = pytest.mark.gpu


def _setup(name, **kw):
    m = lib()
    from sparse_attention_fp4_e2m1_amd.pipeline import LayerStack
    wl = synth.workload(name, **kw)
    data = synth.gen_batch(wl)
    gc = m.Cache(wl.batch, wl.context, idx_heads=wl.idx_heads, idx_k_dtype=wl.idx_k_dtype)
    pre = wl.context - wl.appended
    for b in range(wl.batch):
        m.csa2_kv_append(gc, dev_u16(data.k[b, :pre]), dev_u16(data.v[b, :pre]),
                         dev_u16(data.ik[b, :pre]), dev_i32(np.full(pre, b)),
                         dev_i32(np.arange(pre)))
    rb = np.repeat(np.arange(wl.batch), wl.appended)
    rp = np.tile(np.arange(pre, wl.context), wl.batch)
    app = (dev_u16(data.k[rb, rp]), dev_u16(data.v[rb, rp]), dev_u16(data.ik[rb, rp]),
           dev_i32(rb), dev_i32(rp))
    qs = [synth.gen_queries(wl, li) for li in range(len(wl.layers))]
    q = [dev_u16(x.q) for x in qs]
    qi = [dev_u16(x.q_idx) for x in qs]
    stack = LayerStack(gc, wl.layers, wl.nq, wl.heads, wl.top_k, q_idx_dtype=wl.q_idx_dtype)
    args = (q, qi, dev_i32(wl.query_seq()), dev_i32(wl.query_pos()))
    torch.cuda.synchronize()
    return m, gc, stack, args, app


def _snapshot(gc, stack):
    out = [host(t) for t in stack.topk]
    out += [host(p) for p in stack.pool if p is not None]
    out += [host(o) for o in stack.out] + [host(x) for x in stack.lse]
    out += [host(gc.kv_codes), host(gc.kv_scales), host(gc.idx_k)]
    return out


@pytest.mark.parametrize("name,kw", [
    ("decode_64k_b32", dict(context=8192, batch=4)),   # ranked records, append in the scan launch
    ("chain8_256k_b8", dict(context=16384, batch=2)),  # pool, Reindex over it, Reuse
    ("decode_1m", dict(context=65536)),                # histogram streams, Reindex pool records
])
def test_graph_replays_match_the_eager_step(name, kw):
    announce(f"graph replay {name} {kw}")
    m, gc, stack, args, app = _setup(name, **kw)
    # eager work between replays: a second stack over its own buffers
    _, gc2, stack2, args2, app2 = _setup(name, **kw)
    stack.run(*args, append=app)
    torch.cuda.synchronize()
    want = _snapshot(gc, stack)
    for t in stack.topk:
        t.fill_(-7)   # the replays must rewrite every list
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        stack.run(*args, append=app)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        stack.run(*args, append=app)
    for r in range(4):
        for t in stack.topk:
            t.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        stack2.run(*args2, append=app2)   # the program's own eager work
        torch.cuda.synchronize()
        got = _snapshot(gc, stack)
        for i, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(a, b), (r, i)
