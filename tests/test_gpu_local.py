"""GPU parity of the local sliding-window branch: csa2_local_append codes and
slot positions bit-exact against the oracle; csa2_sparse_attn followed by
csa2_local_attn (the merge through lse) against the oracle's single softmax
over both sets of rows, per (query, head) max_c |delta| / max_c |o_ref| <=
2e-3 and |delta lse| <= 2e-3."""
import numpy as np
import pytest
import torch

import synth
from oracle import csa2 as O
from gpu_util import ATTN_TOL, DEFAULT_SCALE, DEV, announce, attn_errors, dev_i32, dev_u16, \
    filled_caches, host, lib

pytestmark = pytest.mark.gpu

CONTEXT = 3008
_CACHES = {}


def _global(heads):
    if heads not in _CACHES:
        wl = synth.workload("tiny_4k", context=CONTEXT, batch=3, heads=heads)
        gc, oc, _ = filled_caches(wl)
        _CACHES[heads] = (wl, gc, oc)
    return _CACHES[heads]


def _local(window, seed=7):
    """GPU and oracle windows over the same rows.  Sequence 0: positions
    0..2999; sequence 1: positions 0..40 only; sequence 2: 0..2999 without
    2990..2993 (their slots keep older positions)."""
    m = lib()
    gl = m.LocalCache(3, window)
    ol = O.OracleLocalCache(3, window)
    rng = np.random.default_rng(seed)
    for b, pos in ((0, np.arange(3000)), (1, np.arange(41)),
                   (2, np.setdiff1d(np.arange(3000), np.arange(2990, 2994)))):
        k = synth.f32_to_bf16_bits(rng.standard_normal((len(pos), 128)).astype(np.float32))
        v = synth.f32_to_bf16_bits(rng.standard_normal((len(pos), 128)).astype(np.float32) * 2)
        # appended in chunks that never hold two positions of one slot
        for lo in range(0, len(pos), window):
            sl = slice(lo, lo + window)
            seq = np.full(len(pos[sl]), b, np.int32)
            m.csa2_local_append(gl, dev_u16(k[sl]), dev_u16(v[sl]), dev_i32(seq),
                                dev_i32(pos[sl].astype(np.int32)))
            ol.append(k[sl], v[sl], seq, pos[sl])
    torch.cuda.synchronize()
    return gl, ol


@pytest.mark.parametrize("window", [1, 64, 128, 300])
def test_local_append_bit_exact(window):
    announce(f"local append window={window}")
    gl, ol = _local(window)
    assert np.array_equal(host(gl.k), ol.k)
    assert np.array_equal(host(gl.v), ol.v)
    assert np.array_equal(host(gl.pos).astype(np.int64), ol.pos)


def _run(heads, window, topk, qpos, qseq, scale=None, qset=0):
    m = lib()
    wl, gc, oc = _global(heads)
    gl, ol = _local(window)
    q = synth.gen_queries(wl, qset).q
    q = np.concatenate([q] * ((len(qpos) + len(q) - 1) // len(q)))[: len(qpos)]
    out, lse = m.csa2_sparse_attn(gc, dev_u16(q), dev_i32(qseq), dev_i32(topk), softmax_scale=scale)
    m.csa2_local_attn(gl, dev_u16(q), dev_i32(qseq), dev_i32(qpos), out, lse, softmax_scale=scale)
    torch.cuda.synchronize()
    s = DEFAULT_SCALE if scale is None else float(np.float32(scale))
    ref = [O.attention_with_window(q[i], oc, int(qseq[i]), topk[i], ol, int(qpos[i]), s)
           for i in range(len(qpos))]
    return host(out), host(lse), np.stack([r[0] for r in ref]), np.stack([r[1] for r in ref]), ol


@pytest.mark.parametrize("heads", [16, 48, 64])
@pytest.mark.parametrize("window", [64, 128, 300])
def test_local_attention_merged(heads, window):
    # full window, a short history (41 rows), a window with missing slots, a
    # query whose window was overwritten (sparse rows only) and one with no
    # sparse rows (window only)
    announce(f"local attn heads={heads} window={window}")
    qseq = np.array([0, 1, 2, 0, 2], np.int32)
    qpos = np.array([2999, 40, 2999, 2400, 2995], np.int32)
    rng = np.random.default_rng(heads + window)
    topk = rng.integers(0, 2400, (5, 256)).astype(np.int32)
    topk[2, rng.random(256) < 0.3] = -1
    topk[4] = -1
    out, lse, ro, rl, ol = _run(heads, window, topk, qpos, qseq)
    assert len(ol.window_rows(0, 2400)[0]) == 0 and len(ol.window_rows(1, 40)[0]) == min(41, window)
    rel, dl = attn_errors(out, lse, ro, rl)
    assert rel.max() <= ATTN_TOL, rel.max()
    assert dl.max() <= ATTN_TOL, dl.max()


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_local_attention_scale(scale):
    announce(f"local attn scale={scale}")
    qseq = np.array([0, 1, 2], np.int32)
    qpos = np.array([2999, 40, 2999], np.int32)
    topk = np.random.default_rng(9).integers(0, 2900, (3, 100)).astype(np.int32)
    out, lse, ro, rl, ol = _run(64, 128, topk, qpos, qseq, scale=scale, qset=1)
    rel, dl = attn_errors(out, lse, ro, rl)
    assert rel.max() <= ATTN_TOL and dl.max() <= ATTN_TOL
    if scale == 0.0:   # uniform weights: lse = ln(rows of both sets)
        n = np.array([100 + len(ol.window_rows(int(s), int(p))[0]) for s, p in zip(qseq, qpos)])
        assert np.allclose(lse, np.log(n)[:, None], atol=1e-5)


def test_local_attention_nothing_visible():
    # no sparse rows and no window rows: out stays 0, lse -inf
    announce("local attn nothing visible")
    out, lse, ro, rl, _ = _run(64, 64, np.full((2, 8), -1, np.int32), np.array([2400, 2400], np.int32),
                               np.array([0, 2], np.int32))
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def _run_fused(heads, window, topk, qpos, qseq, scale=None, qset=0):
    m = lib()
    wl, gc, oc = _global(heads)
    gl, ol = _local(window)
    q = synth.gen_queries(wl, qset).q
    q = np.concatenate([q] * ((len(qpos) + len(q) - 1) // len(q)))[: len(qpos)]
    out, lse = m.csa2_sparse_local_attn(gc, gl, dev_u16(q), dev_i32(qseq), dev_i32(qpos),
                                        dev_i32(topk), softmax_scale=scale)
    torch.cuda.synchronize()
    s = DEFAULT_SCALE if scale is None else float(np.float32(scale))
    ref = [O.attention_with_window(q[i], oc, int(qseq[i]), topk[i], ol, int(qpos[i]), s)
           for i in range(len(qpos))]
    return host(out), host(lse), np.stack([r[0] for r in ref]), np.stack([r[1] for r in ref])


@pytest.mark.parametrize("heads", [16, 64])
@pytest.mark.parametrize("window", [64, 300, 1024])
def test_fused_both_branches(heads, window):
    # one launch for both sets of rows: the same cases as the two-call merge
    announce(f"fused sparse+local heads={heads} window={window}")
    qseq = np.array([0, 1, 2, 0, 2], np.int32)
    qpos = np.array([2999, 40, 2999, 2400, 2995], np.int32)
    rng = np.random.default_rng(heads + window + 1)
    topk = rng.integers(0, 2400, (5, 256)).astype(np.int32)
    topk[2, rng.random(256) < 0.3] = -1
    topk[4] = -1
    out, lse, ro, rl = _run_fused(heads, window, topk, qpos, qseq)
    rel, dl = attn_errors(out, lse, ro, rl)
    assert rel.max() <= ATTN_TOL and dl.max() <= ATTN_TOL, (rel.max(), dl.max())


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_fused_single_query_many_splits(scale):
    # one query and a long list: the selected rows take nearly every split the
    # combine holds, the window's splits come on top
    announce(f"fused one query k=3000 scale={scale}")
    topk = np.random.default_rng(4).integers(0, 3000, (1, 3000)).astype(np.int32)
    out, lse, ro, rl = _run_fused(48, 300, topk, np.array([2999], np.int32),
                                  np.array([0], np.int32), scale=scale)
    rel, dl = attn_errors(out, lse, ro, rl)
    assert rel.max() <= ATTN_TOL and dl.max() <= ATTN_TOL, (rel.max(), dl.max())


def test_fused_nothing_visible():
    announce("fused nothing visible")
    out, lse, _, _ = _run_fused(64, 64, np.full((2, 8), -1, np.int32),
                                np.array([2400, 2400], np.int32), np.array([0, 2], np.int32))
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_fused_is_deterministic():
    # the fused call twice on the same inputs: identical bytes of out and lse
    announce("fused determinism")
    m = lib()
    wl, gc, oc = _global(64)
    gl, ol = _local(300)
    qseq = np.array([0, 1, 2, 0, 2], np.int32)
    qpos = np.array([2999, 40, 2999, 2400, 2995], np.int32)
    q = synth.gen_queries(wl, 0).q
    q = np.concatenate([q] * 2)[:5]
    topk = np.random.default_rng(8).integers(0, 2400, (5, 2048)).astype(np.int32)
    runs = []
    for _ in range(2):
        out, lse = m.csa2_sparse_local_attn(gc, gl, dev_u16(q), dev_i32(qseq), dev_i32(qpos),
                                            dev_i32(topk))
        torch.cuda.synchronize()
        runs.append((host(out), host(lse)))
    assert np.array_equal(runs[0][0], runs[1][0]) and np.array_equal(runs[0][1], runs[1][1])
