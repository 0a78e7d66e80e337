"""GPU parity of csa2_sparse_attn against the oracle's fp64 attention on the
same index lists: per (query, head) max_c |delta| / max_c |o_ref| <= 2e-3 and
|delta lse| <= 2e-3."""
import numpy as np
import pytest
import torch

import synth
from oracle import csa2 as O
from gpu_util import ATTN_TOL, DEFAULT_SCALE, DEV, announce, attn_errors, dev_i32, dev_u16, \
    filled_caches, host, lib

pytestmark = pytest.mark.gpu

_CACHES = {}


def _setup(heads):
    if heads not in _CACHES:
        wl = synth.workload("tiny_4k", context=3008, batch=3, heads=heads)
        gc, oc, _ = filled_caches(wl)
        _CACHES[heads] = (wl, gc, oc)
    return _CACHES[heads]


def _run(gc, q_bits, topk, scale=None):
    m = lib()
    nq = q_bits.shape[0]
    out, lse = m.csa2_sparse_attn(gc, dev_u16(q_bits), dev_i32(np.arange(nq) % gc.batch),
                                  dev_i32(topk), softmax_scale=scale)
    torch.cuda.synchronize()
    return host(out), host(lse)


def _oracle(oc, q_bits, topk, scale=DEFAULT_SCALE):
    outs, lses = [], []
    for i in range(q_bits.shape[0]):
        o, l = O.sparse_attention(q_bits[i], oc, i % oc.batch, topk[i], scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("heads", [16, 64, 48])
@pytest.mark.parametrize("top_k", [1, 64, 100, 2048])
def test_attention_random_lists(heads, top_k):
    announce(f"attn heads={heads} k={top_k}")
    wl, gc, oc = _setup(heads)
    qd = synth.gen_queries(wl, 0)
    rng = np.random.default_rng(top_k + heads)
    topk = rng.integers(0, 3000, (3, top_k)).astype(np.int32)
    topk[1, rng.random(top_k) < 0.3] = -1          # holes
    if top_k > 1:
        topk[2, : top_k // 2] = topk[2, 0]          # duplicates
    out, lse = _run(gc, qd.q, topk)
    ref_o, ref_l = _oracle(oc, qd.q, topk)
    rel, dl = attn_errors(out, lse, ref_o, ref_l)
    assert rel.max() <= ATTN_TOL, rel.max()
    assert dl.max() <= ATTN_TOL, dl.max()


def test_attention_empty_and_single():
    announce("attn empty/single")
    wl, gc, oc = _setup(64)
    qd = synth.gen_queries(wl, 1)
    topk = np.full((3, 130), -1, np.int32)
    topk[1, 77] = 1234
    out, lse = _run(gc, qd.q, topk)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    _, v = oc.kv_values(1, np.array([1234]))
    assert np.array_equal(out[1], np.broadcast_to(v[0], out[1].shape).astype(np.float32))
    ref_o, ref_l = _oracle(oc, qd.q, topk)
    rel, dl = attn_errors(out, lse, ref_o, ref_l)
    assert rel.max() <= ATTN_TOL and dl.max() <= ATTN_TOL


@pytest.mark.parametrize("heads", [16, 64])
@pytest.mark.parametrize("scale", [0.3, -0.2, 0.0])
def test_attention_custom_scale(heads, scale):
    # a negative scale (folded into the query's sign on the GPU) and a zero
    # scale (uniform weights over the valid rows, lse = ln n), with holes
    announce(f"attn scale={scale} heads={heads}")
    wl, gc, oc = _setup(heads)
    qd = synth.gen_queries(wl, 2)
    rng = np.random.default_rng(3)
    topk = rng.integers(0, 3000, (3, 300)).astype(np.int32)
    topk[2, rng.random(300) < 0.4] = -1
    out, lse = _run(gc, qd.q, topk, scale=scale)
    ref_o, ref_l = _oracle(oc, qd.q, topk, scale=float(np.float32(scale)))
    rel, dl = attn_errors(out, lse, ref_o, ref_l)
    assert rel.max() <= ATTN_TOL and dl.max() <= ATTN_TOL
    if scale == 0.0:
        n = (topk >= 0).sum(1)
        assert np.allclose(lse, np.log(n)[:, None], atol=1e-5)


def test_attention_deterministic():
    announce("attn determinism")
    wl, gc, oc = _setup(64)
    qd = synth.gen_queries(wl, 0)
    topk = np.random.default_rng(5).integers(0, 3000, (3, 2048)).astype(np.int32)
    a = _run(gc, qd.q, topk)
    b = _run(gc, qd.q, topk)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("nq,top_k,heads", [(32, 2048, 64), (32, 1500, 64), (16, 1000, 48),
                                            (256, 300, 16), (64, 2048, 32), (8, 2048, 64),
                                            (4, 65536, 16)])
def test_attention_batch_shapes(nq, top_k, heads):
    # Batch shapes whose splits hold several 64-row sub-chunks (an odd count:
    # 1500 rows give 3 per split), one split per query (256 queries: the final
    # output written directly, no combine), 16 splits of two sub-chunks (8
    # queries of 2048 rows) and the largest K (65536 rows: splits of the
    # most rows a split takes).  Holes, an empty list, duplicates; determinism.
    announce(f"attn batch shape nq={nq} k={top_k} heads={heads}")
    m = lib()
    wl, gc, oc = _setup(heads)
    rng = np.random.default_rng(nq + top_k + heads)
    q = synth.f32_to_bf16_bits(rng.standard_normal((nq, heads, 128)).astype(np.float32))
    topk = rng.integers(0, 3000, (nq, top_k)).astype(np.int32)
    topk[1, rng.random(top_k) < 0.3] = -1
    topk[2] = -1
    topk[3, : top_k // 2] = topk[3, 0]
    q_seq = np.arange(nq) % gc.batch
    out, lse = m.csa2_sparse_attn(gc, dev_u16(q), dev_i32(q_seq), dev_i32(topk))
    torch.cuda.synchronize()
    out, lse = host(out), host(lse)
    check = list(range(min(nq, 8))) + [nq - 1]
    for i in check:
        ro, rl = O.sparse_attention(q[i], oc, int(q_seq[i]), topk[i])
        rel, dl = attn_errors(out[i], lse[i], ro, rl)
        assert rel.max() <= ATTN_TOL and dl.max() <= ATTN_TOL, (i, rel.max(), dl.max())
    assert np.all(out[2] == 0.0) and np.all(np.isneginf(lse[2]))
    # deterministic
    out2, lse2 = m.csa2_sparse_attn(gc, dev_u16(q), dev_i32(q_seq), dev_i32(topk))
    torch.cuda.synchronize()
    assert np.array_equal(host(out2), out) and np.array_equal(host(lse2), lse)


@pytest.mark.parametrize("nq,top_k", [(800, 2048), (1600, 1000), (3200, 300), (800, 100), (800, 64),
                                      (800, 1)])
def test_attention_large_grids_match_small(nq, top_k):
    # Calls of at least 768 workgroups with 64 heads take the four-per-CU form
    # (the row list through an LDS ring, the gathers one sub-chunk ahead); the
    # same queries in calls of fewer workgroups take the three-per-CU form.
    # Both run the same sub-chunk updates in the same order: identical bytes.
    # Holes, an empty list, duplicates; and the oracle on a few queries.
    announce(f"attn large grid nq={nq} k={top_k}")
    m = lib()
    wl, gc, oc = _setup(64)
    rng = np.random.default_rng(nq * 7 + top_k)
    q = synth.f32_to_bf16_bits(rng.standard_normal((nq, 64, 128)).astype(np.float32))
    topk = rng.integers(0, 3000, (nq, top_k)).astype(np.int32)
    topk[1, rng.random(top_k) < 0.3] = -1
    topk[2] = -1
    topk[3, : max(top_k // 2, 1)] = topk[3, 0]
    q_seq = np.arange(nq) % gc.batch
    out, lse = m.csa2_sparse_attn(gc, dev_u16(q), dev_i32(q_seq), dev_i32(topk))
    torch.cuda.synchronize()
    out, lse = host(out), host(lse)
    # pieces of 400 queries: still one split per query (256 workgroups or
    # more), but grids of fewer than 768
    for s0 in range(0, nq, 400):
        sl = slice(s0, s0 + 400)
        o2, l2 = m.csa2_sparse_attn(gc, dev_u16(q[sl]), dev_i32(q_seq[sl]), dev_i32(topk[sl]))
        torch.cuda.synchronize()
        assert np.array_equal(host(o2), out[sl]) and np.array_equal(host(l2), lse[sl]), s0
    for i in [0, 1, 3, nq - 1]:
        ro, rl = O.sparse_attention(q[i], oc, int(q_seq[i]), topk[i])
        rel, dl = attn_errors(out[i], lse[i], ro, rl)
        assert rel.max() <= ATTN_TOL and dl.max() <= ATTN_TOL, (i, rel.max(), dl.max())
    assert np.all(out[2] == 0.0) and np.all(np.isneginf(lse[2]))
