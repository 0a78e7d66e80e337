"""csa2_sparse_attn_noalloc (the attention call whose split partials live in
the library's static device scratch) against csa2_sparse_attn with a caller
workspace: the same kernels in the same split layout, so the outputs must be
identical bit for bit.  Two calls in a row, the second smaller; the first
call's results are checked against the oracle too (the attention tolerance).
A call whose partials would not fit the scratch is rejected before anything is
enqueued."""
import numpy as np
import pytest
import torch

import synth
from oracle import csa2 as O
from gpu_util import ATTN_TOL, DEV, announce, attn_errors, dev_i32, dev_u16, filled_caches, host, lib

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 16 << 20


def _both(m, gc, q, q_seq, topk):
    nq, heads = q.shape[0], q.shape[1]
    out_a = torch.full((nq, heads, 128), 7.0, dtype=torch.float32, device=DEV)
    lse_a = torch.full((nq, heads), 7.0, dtype=torch.float32, device=DEV)
    m.csa2_sparse_attn_noalloc(gc, q, q_seq, topk, out=out_a, lse=lse_a)
    out_b, lse_b = m.csa2_sparse_attn(gc, q, q_seq, topk)
    torch.cuda.synchronize()
    return (host(out_a), host(lse_a)), (host(out_b), host(lse_b))


def test_noalloc_matches_workspace_call_twice():
    m = lib()
    wl = synth.workload("tiny_4k", context=3008, batch=4, heads=64)
    announce("noalloc attention: filling a 4 x 3008 cache")
    gc, oc, _ = filled_caches(wl)
    rng = np.random.default_rng(31)

    # call 1: 32 queries x 64 heads x 2048 rows (8 splits per query: partials used)
    nq, k = 32, 2048
    assert m.csa2_sparse_attn_workspace(gc, nq, 64, k) <= SCRATCH_BYTES
    q = rng.standard_normal((nq, 64, 128)).astype(np.float32)
    qb = synth.f32_to_bf16_bits(q)
    topk = rng.integers(0, 3008, (nq, k)).astype(np.int32)
    topk[3, rng.random(k) < 0.4] = -1
    q_seq = np.arange(nq) % 4
    announce("noalloc attention: call 1 (32 queries, K 2048)")
    a, b = _both(m, gc, dev_u16(qb), dev_i32(q_seq), dev_i32(topk))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    for i in (0, 3, 31):
        ro, rl = O.sparse_attention(qb[i], oc, int(q_seq[i]), topk[i])
        rel, dl = attn_errors(a[0][i], a[1][i], ro, rl)
        assert rel.max() <= ATTN_TOL and dl.max() <= ATTN_TOL

    # call 2, smaller: 5 queries x 16 heads x 300 rows, one list empty
    nq, k = 5, 300
    q2 = synth.f32_to_bf16_bits(rng.standard_normal((nq, 16, 128)).astype(np.float32))
    topk2 = rng.integers(0, 3008, (nq, k)).astype(np.int32)
    topk2[2] = -1
    q_seq2 = np.array([3, 1, 0, 2, 3])
    announce("noalloc attention: call 2 (5 queries, K 300)")
    a, b = _both(m, gc, dev_u16(q2), dev_i32(q_seq2), dev_i32(topk2))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.all(a[0][2] == 0.0) and np.all(np.isneginf(a[1][2]))


def test_noalloc_rejects_calls_beyond_the_scratch():
    m = lib()
    gc = m.Cache(1, 4096, idx_heads=8, idx_k_dtype="fp8")
    nq, heads, k = 64, 128, 4096
    assert m.csa2_sparse_attn_workspace(gc, nq, heads, k) > SCRATCH_BYTES
    q = torch.zeros((nq, heads, 128), dtype=torch.int16, device=DEV)
    out = torch.full((nq, heads, 128), 5.0, dtype=torch.float32, device=DEV)
    z = torch.zeros(nq, dtype=torch.int32, device=DEV)
    topk = torch.zeros((nq, k), dtype=torch.int32, device=DEV)
    with pytest.raises(m.Csa2Error) as e:
        m.csa2_sparse_attn_noalloc(gc, q, z, topk, out=out)
    assert e.value.status == m.CSA2_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())   # nothing was enqueued
