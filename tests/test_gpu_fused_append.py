"""GPU parity of csa2_index_topk_append: the append and the first index layer
in one call give the same Top-K lists, pools and cache bytes as csa2_kv_append
followed by csa2_index_topk, and the oracle's Top-K after its own append.

Cases cover every scorer shape that takes the rows in its launch (ranked
records of 2048 and 4096 keys, the global histogram, a pool-building Full
layer, a Reindex layer over every visible position) and the ones that append
first on their own (one-wave shapes, the matrix-core scorer, more than 256
rows, a Reindex pool): rows at the queries' own positions (a decode step),
rows of sequences no query reads, rows past a query's position, rows without
index keys."""
import numpy as np
import pytest
import torch

import synth
from oracle import csa2 as O
from gpu_util import announce, dev_i32, dev_u16, host, lib, untile_idx

pytestmark = pytest.mark.gpu


def _bf16(rng, shape, scale=1.0):
    return synth.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _twin_caches(m, nseq, cap, heads, dtype, rng):
    """Two GPU caches and the oracle cache with the same seeded contents."""
    caches = [m.Cache(nseq, cap, idx_heads=heads, idx_k_dtype=dtype) for _ in range(2)]
    oc = O.OracleCache(nseq, cap, idx_heads=heads, idx_k_dtype=dtype)
    for b in range(nseq):
        k, v, ik = _bf16(rng, (cap, 128)), _bf16(rng, (cap, 128)), _bf16(rng, (cap, heads, 64))
        seq, pos = np.full(cap, b, np.int32), np.arange(cap, dtype=np.int32)
        for gc in caches:
            m.csa2_kv_append(gc, dev_u16(k), dev_u16(v), dev_u16(ik), dev_i32(seq), dev_i32(pos))
        oc.append(k, v, ik, seq, pos)
    torch.cuda.synchronize()
    return caches, oc


def _run_case(nq, nseq, cap, heads=8, dtype="fp8", q_dtype="bf16", mode="full", pool_blocks=0,
              top_k=256, extra_rows=0, with_idx=True, seed=0, oracle_every=5):
    m = lib()
    rng = np.random.default_rng(seed)
    (g1, g2), oc = _twin_caches(m, nseq, cap, heads, dtype, rng)
    qseq = (np.arange(nq) % nseq).astype(np.int32)
    # distinct (sequence, position) per query, query 0 at the last position: a
    # decode step's own rows
    qpos = np.empty(nq, np.int32)
    for b in range(nseq):
        idx = np.where(qseq == b)[0]
        qpos[idx] = rng.choice(cap - 1, len(idx), replace=False)
    qpos[0] = cap - 1
    aseq, apos = list(qseq), list(qpos)
    # rows of sequence nseq - 1 at other positions: before some of its queries'
    # positions and past others
    used = set(zip(aseq, apos))
    while len(aseq) < nq + extra_rows:
        s_, p_ = int(nseq - 1), int(rng.integers(0, cap))
        if (s_, p_) not in used:
            used.add((s_, p_))
            aseq.append(s_)
            apos.append(p_)
    n = len(aseq)
    k, v = _bf16(rng, (n, 128)), _bf16(rng, (n, 128))
    ik = _bf16(rng, (n, heads, 64)) if with_idx else None
    qidx = _bf16(rng, (nq, heads, 64))
    aseq, apos = np.array(aseq, np.int32), np.array(apos, np.int32)
    app = (dev_u16(k), dev_u16(v), dev_u16(ik) if with_idx else None, dev_i32(aseq), dev_i32(apos))
    pool_in = None
    if mode == "reindex_pool":
        pool_in = dev_i32(np.stack([np.sort(rng.choice(cap, 2048, replace=False))
                                    for _ in range(nq)]))
    md = "reindex" if mode.startswith("reindex") else mode
    kw = dict(q_dtype=q_dtype, pool_blocks=pool_blocks, pool_in=pool_in)
    # fused
    t1, p1 = m.csa2_index_topk_append(g1, *app, md, dev_u16(qidx), dev_i32(qseq), dev_i32(qpos),
                                      top_k, **kw)
    # separate
    m.csa2_kv_append(g2, *app)
    t2, p2 = m.csa2_index_topk(g2, md, dev_u16(qidx), dev_i32(qseq), dev_i32(qpos), top_k, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(host(t1), host(t2))
    if pool_blocks:
        assert np.array_equal(host(p1), host(p2))
    for a, b in ((g1.kv_codes, g2.kv_codes), (g1.kv_scales, g2.kv_scales), (g1.idx_k, g2.idx_k)):
        assert np.array_equal(host(a), host(b))
    # the oracle after its own append (exact where the streaming scorer runs)
    oc.append(k, v, ik if with_idx else None, aseq, apos)
    if q_dtype == "fp8" and dtype == "fp8" and mode in ("full", "reindex") and not pool_blocks:
        return   # matrix-core scorer: checked against the separate calls only
    got = host(t1)
    for i in range(0, nq, oracle_every):
        qi = O.query_index_values(qidx[i], q_dtype)
        pin = host(pool_in)[i] if pool_in is not None else None
        want, pool, _, _ = O.index_topk(md, oc, int(qseq[i]), int(qpos[i]), qi, top_k,
                                        pool_in=pin, pool_blocks=pool_blocks)
        assert np.array_equal(got[i], want), (i, int(qpos[i]))
        if pool_blocks:
            assert np.array_equal(host(p1)[i], pool), i


@pytest.mark.parametrize("nq,nseq,cap,kw", [
    (64, 4, 16400, {}),                                   # ranked records of 2048 keys
    (128, 8, 16400, {"top_k": 2048}),                     # ranked records of 4096 keys
    (128, 8, 16400, {"heads": 4, "dtype": "bf16"}),       # bf16 keys, four heads
    (8, 2, 70000, {}),                                    # global histogram
    (8, 2, 70000, {"pool_blocks": 300, "top_k": 2048}),   # pool-building Full layer
    (64, 4, 16400, {"mode": "reindex"}),                  # Reindex over every visible position
    (64, 4, 16400, {"extra_rows": 40}),                   # rows no query reads / past positions
    (64, 4, 16400, {"extra_rows": 192}),                  # 256 rows: the most one launch takes
    (64, 4, 16400, {"with_idx": False}),                  # rows without index keys
])
def test_fused_append_matches_separate_calls(nq, nseq, cap, kw):
    announce(f"fused append nq={nq} nseq={nseq} cap={cap} {kw}")
    _run_case(nq, nseq, cap, seed=nq + cap, **kw)


@pytest.mark.parametrize("nq,nseq,cap,kw", [
    (2, 2, 5008, {}),                                      # one-wave shapes: appended first
    (64, 4, 16400, {"q_dtype": "fp8"}),                   # matrix-core scorer: appended first
    (64, 4, 16400, {"extra_rows": 300}),                  # more than 256 rows: appended first
    (8, 2, 16400, {"mode": "reindex_pool"}),              # a Reindex pool: appended first
])
def test_fused_append_falls_back_to_a_separate_append(nq, nseq, cap, kw):
    announce(f"fused append fallback nq={nq} nseq={nseq} cap={cap} {kw}")
    _run_case(nq, nseq, cap, seed=7 + nq, **kw)


def test_fused_append_decode_steps_in_a_row():
    # three decode steps: each step appends the queries' next positions and
    # selects; the caches and lists stay equal to the two-call sequence
    announce("fused append, three steps")
    m = lib()
    rng = np.random.default_rng(11)
    nq, nseq, cap = 64, 4, 16400
    (g1, g2), oc = _twin_caches(m, nseq, cap, 8, "fp8", rng)
    qseq = (np.arange(nq) % nseq).astype(np.int32)
    qpos = np.empty(nq, np.int32)
    for b in range(nseq):   # positions 4 apart within a sequence: three steps never collide
        idx = np.where(qseq == b)[0]
        qpos[idx] = 4 * rng.choice(np.arange(250, cap // 4 - 1), len(idx), replace=False)
    for step in range(3):
        k, v, ik = _bf16(rng, (nq, 128)), _bf16(rng, (nq, 128)), _bf16(rng, (nq, 8, 64))
        qidx = _bf16(rng, (nq, 8, 64))
        app = (dev_u16(k), dev_u16(v), dev_u16(ik), dev_i32(qseq), dev_i32(qpos))
        t1, _ = m.csa2_index_topk_append(g1, *app, "full", dev_u16(qidx), dev_i32(qseq),
                                         dev_i32(qpos), 2048)
        m.csa2_kv_append(g2, *app)
        t2, _ = m.csa2_index_topk(g2, "full", dev_u16(qidx), dev_i32(qseq), dev_i32(qpos), 2048)
        torch.cuda.synchronize()
        assert np.array_equal(host(t1), host(t2)), step
        oc.append(k, v, ik, qseq, qpos)
        for i in (step, 20 + step):
            want, _, _, _ = O.index_topk("full", oc, int(qseq[i]), int(qpos[i]),
                                         O.query_index_values(qidx[i], "bf16"), 2048)
            assert np.array_equal(host(t1)[i], want), (step, i)
        qpos = qpos + 1
    assert np.array_equal(host(g1.idx_k), host(g2.idx_k))
    assert np.array_equal(untile_idx(host(g1.idx_k), 8, np.uint8), oc.idx_k)


def test_fused_append_without_queries_or_rows():
    # no queries: the call is the append alone; no rows: the index call alone
    announce("fused append, nq = 0 and n_append = 0")
    m = lib()
    rng = np.random.default_rng(5)
    nseq, cap = 2, 16400
    (g1, g2), oc = _twin_caches(m, nseq, cap, 8, "fp8", rng)
    n = 20
    aseq = np.array([i % nseq for i in range(n)], np.int32)
    apos = rng.choice(cap, n, replace=False).astype(np.int32)
    k, v, ik = _bf16(rng, (n, 128)), _bf16(rng, (n, 128)), _bf16(rng, (n, 8, 64))
    app = (dev_u16(k), dev_u16(v), dev_u16(ik), dev_i32(aseq), dev_i32(apos))
    empty_q = (torch.empty((0, 8, 64), dtype=torch.int16, device="cuda"),
               torch.empty(0, dtype=torch.int32, device="cuda"),
               torch.empty(0, dtype=torch.int32, device="cuda"))
    m.csa2_index_topk_append(g1, *app, "full", *empty_q, 2048)
    m.csa2_kv_append(g2, *app)
    torch.cuda.synchronize()
    for a, b in ((g1.kv_codes, g2.kv_codes), (g1.kv_scales, g2.kv_scales), (g1.idx_k, g2.idx_k)):
        assert np.array_equal(host(a), host(b))
    nq = 16
    qseq = (np.arange(nq) % nseq).astype(np.int32)
    qpos = rng.choice(cap, nq, replace=False).astype(np.int32)
    qidx = _bf16(rng, (nq, 8, 64))
    none = (torch.empty((0, 128), dtype=torch.int16, device="cuda"),
            torch.empty((0, 128), dtype=torch.int16, device="cuda"), None,
            torch.empty(0, dtype=torch.int32, device="cuda"),
            torch.empty(0, dtype=torch.int32, device="cuda"))
    t1, _ = m.csa2_index_topk_append(g1, *none, "full", dev_u16(qidx), dev_i32(qseq),
                                     dev_i32(qpos), 2048)
    t2, _ = m.csa2_index_topk(g2, "full", dev_u16(qidx), dev_i32(qseq), dev_i32(qpos), 2048)
    torch.cuda.synchronize()
    assert np.array_equal(host(t1), host(t2))
