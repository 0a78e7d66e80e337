"""End-to-end GPU parity of a whole step (append + every layer's index Top-K and
attention) on each workload preset at reduced context, against the oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import csa2 as O
from gpu_util import announce, check_stack, dev_i32, dev_u16, host, lib

pytestmark = pytest.mark.gpu

REDUCED = {
    "tiny_4k": {},
    "decode_64k_b32": dict(context=8192, batch=4),
    "chain8_256k_b8": dict(context=16384, batch=2),
    "decode_1m": dict(context=65536),
    "prefill_4k_on_128k": dict(context=4096 + 256, prefill=256),
    "released_256k_b8": dict(context=32768, batch=2),
    "encoder_4k_on_128k": dict(context=4096 + 256, prefill=256),
}


def run_step_and_oracle(wl, only=None):
    m = lib()
    from sparse_attention_fp4_e2m1_amd.pipeline import LayerStack
    data = synth.gen_batch(wl)
    gc = m.Cache(wl.batch, wl.context, idx_heads=wl.idx_heads, idx_k_dtype=wl.idx_k_dtype)
    oc = O.OracleCache(wl.batch, wl.context, idx_heads=wl.idx_heads, idx_k_dtype=wl.idx_k_dtype)
    pre = wl.context - wl.appended
    for b in range(wl.batch):
        seq = np.full(pre, b, np.int32)
        pos = np.arange(pre, dtype=np.int32)
        m.csa2_kv_append(gc, dev_u16(data.k[b, :pre]), dev_u16(data.v[b, :pre]),
                         dev_u16(data.ik[b, :pre]), dev_i32(seq), dev_i32(pos))
        oc.append(data.k[b], data.v[b], data.ik[b], np.full(wl.context, b), np.arange(wl.context))
    # the step appends the newest row(s) of every sequence
    rows_b = np.repeat(np.arange(wl.batch), wl.appended)
    rows_p = np.tile(np.arange(pre, wl.context), wl.batch)
    app = (dev_u16(data.k[rows_b, rows_p]), dev_u16(data.v[rows_b, rows_p]),
           dev_u16(data.ik[rows_b, rows_p]), dev_i32(rows_b), dev_i32(rows_p))
    qs = [synth.gen_queries(wl, li) for li in range(len(wl.layers))]
    stack = LayerStack(gc, wl.layers, wl.nq, wl.heads, wl.top_k, q_idx_dtype=wl.q_idx_dtype)
    stack.run([dev_u16(x.q) for x in qs], [dev_u16(x.q_idx) for x in qs],
              dev_i32(wl.query_seq()), dev_i32(wl.query_pos()), append=app)
    torch.cuda.synchronize()
    ref = O.run_layers(oc, wl.layers, wl.query_seq(), wl.query_pos(), qs, wl.top_k,
                       wl.q_idx_dtype, only=only)
    return gc, oc, stack, ref


@pytest.mark.parametrize("name", list(REDUCED))
def test_step_matches_oracle(name):
    wl = synth.workload(name, **REDUCED[name])
    announce(f"e2e {name} {REDUCED[name]}")
    only = None
    if wl.prefill:
        only = list(range(0, wl.nq, 17)) + [wl.nq - 1]
    gc, oc, stack, ref = run_step_and_oracle(wl, only=only)
    # the append itself is bit-exact
    assert np.array_equal(host(gc.kv_codes), oc.kv_codes)
    assert np.array_equal(host(gc.kv_scales), oc.kv_scales)
    rows = [(i, i, int(wl.query_seq()[i])) for i in (range(wl.nq) if only is None else only)]
    qs = [synth.gen_queries(wl, li) for li in range(len(wl.layers))]
    check_stack(wl, oc, stack, ref, qs, rows, log=announce)
    if wl.prefill:   # causality: every selected row is visible to its query
        tk = host(stack.topk[0])
        qp = wl.query_pos()
        assert np.all((tk < 0) | (tk <= qp[:, None]))
