"""GPU parity of csa2_index_topk in Full / Reindex / Reuse mode, with and
without the candidate pool: Top-K index sets and pools bit-exact against the
oracle (the streaming scorer follows the canonical fp32 order, so the scores
themselves are compared bit for bit too).  E4M3 index queries against E4M3
keys over every visible position are scored on matrix cores, whose fp32 sums
follow the hardware's order: those sets are checked with the relaxed rule of
gpu_util.relaxed_topk_check, and exactly where no rounding can matter."""
import numpy as np
import pytest
import torch

import synth
from oracle import csa2 as O
from gpu_util import (DEV, announce, dev_i32, dev_u16, filled_caches, host, lib,
                      relaxed_topk_check)

pytestmark = pytest.mark.gpu

CAP = 5008                       # several 2048-candidate tiles and a ragged tail
QPOS = [0, 5, 63, 2047, 2148, 4999]


def _score_keys(scores):
    u = (np.asarray(scores, np.float32) + np.float32(0.0)).view(np.uint32)
    return np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)


_SETUPS = {}


def _setup(heads, idx_dtype, seed=1):
    key = (heads, idx_dtype, seed)
    if key not in _SETUPS:
        wl = synth.workload("decode_64k_b32", context=CAP, batch=len(QPOS), idx_heads=heads,
                            idx_k_dtype=idx_dtype, seed=seed)
        gc, oc, _ = filled_caches(wl)
        _SETUPS[key] = (wl, gc, oc)
    return _SETUPS[key]


def _oracle_full(wl, oc, qd, q_dtype, top_k, pool_blocks=0, layer_q=None):
    tk, pools, scores = [], [], []
    for i, p in enumerate(QPOS):
        qi = O.query_index_values(qd.q_idx[i], q_dtype)
        t, pool, s, _ = O.index_topk("full", oc, i, p, qi, top_k, pool_blocks=pool_blocks)
        tk.append(t)
        pools.append(pool)
        scores.append(s)
    return np.stack(tk), pools, scores


@pytest.mark.parametrize("heads,idx_dtype,q_dtype", [
    (8, "fp8", "bf16"), (4, "bf16", "bf16"), (4, "fp8", "bf16"), (8, "bf16", "bf16"),
    (4, "bf16", "fp8"), (8, "bf16", "fp8")])
@pytest.mark.parametrize("top_k", [1, 37, 256, 3000])
def test_full_topk_bit_exact(heads, idx_dtype, q_dtype, top_k):
    announce(f"full topk heads={heads} idx={idx_dtype} q={q_dtype} k={top_k}")
    m = lib()
    wl, gc, oc = _setup(heads, idx_dtype)
    qd = synth.gen_queries(wl, 0)
    ws_bytes = m.csa2_index_topk_workspace(gc, "full", len(QPOS), top_k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    topk, _ = m.csa2_index_topk(gc, "full", dev_u16(qd.q_idx), dev_i32(np.arange(len(QPOS))),
                                dev_i32(QPOS), top_k, q_dtype=q_dtype, workspace=ws)
    torch.cuda.synchronize()
    want, _, scores = _oracle_full(wl, oc, qd, q_dtype, top_k)
    # scores: the workspace starts with the per-query score keys [nq][roundup64(capacity)]
    n_tok = (CAP + 63) // 64 * 64
    keys = host(ws[: len(QPOS) * n_tok * 4].view(torch.int32)).view(np.uint32).reshape(len(QPOS), n_tok)
    for i, p in enumerate(QPOS):
        assert np.array_equal(keys[i, :p + 1], _score_keys(scores[i])), f"scores of query {i}"
    assert np.array_equal(host(topk), want)


@pytest.mark.parametrize("pool_blocks", [1, 13, 300, 700])
@pytest.mark.parametrize("heads,idx_dtype", [(8, "fp8"), (4, "bf16")])
def test_full_pool_and_reindex_bit_exact(pool_blocks, heads, idx_dtype):
    announce(f"pool={pool_blocks} heads={heads} idx={idx_dtype}")
    m = lib()
    wl, gc, oc = _setup(heads, idx_dtype)
    top_k = 64
    qd0 = synth.gen_queries(wl, 0)
    qd1 = synth.gen_queries(wl, 1)
    q_seq = dev_i32(np.arange(len(QPOS)))
    q_pos = dev_i32(QPOS)
    topk, pool = m.csa2_index_topk(gc, "full", dev_u16(qd0.q_idx), q_seq, q_pos, top_k,
                                   pool_blocks=pool_blocks)
    torch.cuda.synchronize()
    want_tk, want_pool, _ = _oracle_full(wl, oc, qd0, "bf16", top_k, pool_blocks)
    assert np.array_equal(host(topk), want_tk)
    assert np.array_equal(host(pool), np.stack(want_pool))
    # Reindex over that pool with the next layer's index query
    rtk, _ = m.csa2_index_topk(gc, "reindex", dev_u16(qd1.q_idx), q_seq, q_pos, top_k, pool_in=pool)
    torch.cuda.synchronize()
    for i, p in enumerate(QPOS):
        qi = O.query_index_values(qd1.q_idx[i], "bf16")
        t, _, _, _ = O.index_topk("reindex", oc, i, p, qi, top_k, pool_in=want_pool[i])
        assert np.array_equal(host(rtk)[i], t), f"reindex query {i}"


def test_reindex_over_everything_equals_full():
    announce("reindex over full pool == full")
    m = lib()
    wl, gc, oc = _setup(8, "fp8")
    qd = synth.gen_queries(wl, 0)
    q_seq = dev_i32(np.arange(len(QPOS)))
    q_pos = dev_i32(QPOS)
    pb = (CAP + 7) // 8
    full, pool = m.csa2_index_topk(gc, "full", dev_u16(qd.q_idx), q_seq, q_pos, 100, pool_blocks=pb)
    re, _ = m.csa2_index_topk(gc, "reindex", dev_u16(qd.q_idx), q_seq, q_pos, 100, pool_in=pool)
    re2, _ = m.csa2_index_topk(gc, "reindex", dev_u16(qd.q_idx), q_seq, q_pos, 100)
    torch.cuda.synchronize()
    assert np.array_equal(host(full), host(re))
    assert np.array_equal(host(full), host(re2))


def test_reindex_crafted_pool_with_holes_and_invisible_entries():
    announce("reindex crafted pool")
    m = lib()
    wl, gc, oc = _setup(8, "fp8")
    qd = synth.gen_queries(wl, 2)
    rng = np.random.default_rng(7)
    pool_len = 777
    pools = np.full((len(QPOS), pool_len), -1, np.int32)
    for i in range(len(QPOS)):
        cnt = int(rng.integers(0, pool_len))
        pools[i, :cnt] = np.sort(rng.choice(CAP, cnt, replace=False))   # some beyond q_pos
    tk, _ = m.csa2_index_topk(gc, "reindex", dev_u16(qd.q_idx), dev_i32(np.arange(len(QPOS))),
                              dev_i32(QPOS), 50, pool_in=dev_i32(pools))
    torch.cuda.synchronize()
    for i, p in enumerate(QPOS):
        qi = O.query_index_values(qd.q_idx[i], "bf16")
        t, _, _, _ = O.index_topk("reindex", oc, i, p, qi, 50, pool_in=pools[i])
        assert np.array_equal(host(tk)[i], t), f"query {i}"


def test_reuse_copies_source():
    announce("reuse")
    m = lib()
    wl, gc, oc = _setup(8, "fp8")
    src = np.random.default_rng(0).integers(-1, CAP, (len(QPOS), 2048)).astype(np.int32)
    out, pool = m.csa2_index_topk(gc, "reuse", None, None, None, 2048, reuse_src=dev_i32(src))
    torch.cuda.synchronize()
    assert pool is None and np.array_equal(host(out), src)


@pytest.mark.parametrize("distinct,cap", [(1, 3008), (3, 3008), (1, 20000), (2, 40000)])
def test_tie_heavy_keys(distinct, cap):
    # cap 20000/40000 with few distinct scores: more candidates than the LDS
    # resolve holds, so the selection streams the full key array instead
    announce(f"ties distinct={distinct} cap={cap}")
    m = lib()
    gc = m.Cache(2, cap, idx_heads=8, idx_k_dtype="fp8")
    oc = O.OracleCache(2, cap, idx_heads=8, idx_k_dtype="fp8")
    rng = np.random.default_rng(distinct)
    base = synth.f32_to_bf16_bits(rng.standard_normal((distinct, 8, 64)).astype(np.float32))
    ik = base[rng.integers(0, distinct, cap)]
    kv = synth.f32_to_bf16_bits(rng.standard_normal((cap, 128)).astype(np.float32))
    for b in range(2):
        seq, pos = np.full(cap, b, np.int32), np.arange(cap, dtype=np.int32)
        m.csa2_kv_append(gc, dev_u16(kv), dev_u16(kv), dev_u16(ik), dev_i32(seq), dev_i32(pos))
        oc.append(kv, kv, ik, seq, pos)
    qi = synth.f32_to_bf16_bits(rng.standard_normal((2, 8, 64)).astype(np.float32))
    qpos = [cap - 1, 1234]
    tk, pool = m.csa2_index_topk(gc, "full", dev_u16(qi), dev_i32([0, 1]), dev_i32(qpos), 500,
                                 pool_blocks=40)
    torch.cuda.synchronize()
    for i in range(2):
        t, p, _, _ = O.index_topk("full", oc, i, qpos[i], O.query_index_values(qi[i], "bf16"), 500,
                                  pool_blocks=40)
        assert np.array_equal(host(tk)[i], t)
        assert np.array_equal(host(pool)[i], p)
    if distinct == 1:
        assert list(host(tk)[0]) == list(range(500))


@pytest.mark.parametrize("context,batch,qpos", [
    (70000, 2, [69999, 40000, 33000, 5000, 100]),
    (532480, 1, [532479, 300000, 7])])
def test_filter_path_bit_exact(context, batch, qpos):
    # key arrays past the short-array limit (32768 keys) go through the filter
    # kernel (second-level histogram of the threshold bin, early slot reads in
    # the resolve); past 512K keys the filter regions hold 1024 keys and the
    # scorer's histogram comes in several copies.  Tokens and pool blocks.
    announce(f"filter path context={context} batch={batch}")
    m = lib()
    wl = synth.workload("decode_1m", context=context, batch=batch)
    gc = m.Cache(batch, context, idx_heads=8, idx_k_dtype="fp8")
    oc = O.OracleCache(batch, context, idx_heads=8, idx_k_dtype="fp8", lazy=True)
    data = synth.gen_batch(wl)
    for b in range(batch):
        seq, pos = np.full(context, b, np.int32), np.arange(context, dtype=np.int32)
        m.csa2_kv_append(gc, dev_u16(data.k[b]), dev_u16(data.v[b]), dev_u16(data.ik[b]),
                         dev_i32(seq), dev_i32(pos))
        oc.append(data.k[b], data.v[b], data.ik[b], seq, pos)
    del data
    rng = np.random.default_rng(context)
    nq = len(qpos)
    qi = synth.f32_to_bf16_bits(rng.standard_normal((nq, 8, 64)).astype(np.float32))
    qseq = [i % batch for i in range(nq)]
    for top_k, pool_blocks in ((2048, 2048), (37, 0)):
        tk, pool = m.csa2_index_topk(gc, "full", dev_u16(qi), dev_i32(qseq), dev_i32(qpos), top_k,
                                     pool_blocks=pool_blocks)
        torch.cuda.synchronize()
        for i in range(nq):
            t, p, _, _ = O.index_topk("full", oc, qseq[i], qpos[i],
                                      O.query_index_values(qi[i], "bf16"), top_k,
                                      pool_blocks=pool_blocks)
            assert np.array_equal(host(tk)[i], t), (top_k, i)
            if pool_blocks:
                assert np.array_equal(host(pool)[i], p), (top_k, i)


@pytest.mark.parametrize("context,q_dtype", [(60000, "bf16"), (70000, "bf16"), (70000, "fp8")])
def test_largest_top_k(context, q_dtype):
    # K = 65536, the largest the calls take: over 60000 rows (the ranked
    # records: every candidate selected, then padding) and over 70000 rows
    # (the histogram stream with a real cut of 4464 candidates; and the
    # matrix-core scorer)
    announce(f"top_k 65536 context={context} q={q_dtype}")
    m = lib()
    batch = 2
    wl = synth.workload("decode_1m", context=context, batch=batch)
    gc = m.Cache(batch, context, idx_heads=8, idx_k_dtype="fp8")
    oc = O.OracleCache(batch, context, idx_heads=8, idx_k_dtype="fp8", lazy=True)
    data = synth.gen_batch(wl)
    for b in range(batch):
        seq, pos = np.full(context, b, np.int32), np.arange(context, dtype=np.int32)
        m.csa2_kv_append(gc, dev_u16(data.k[b]), dev_u16(data.v[b]), dev_u16(data.ik[b]),
                         dev_i32(seq), dev_i32(pos))
        oc.append(data.k[b], data.v[b], data.ik[b], seq, pos)
    del data
    top_k = 65536
    qpos = [context - 1, context - 1, 40000]
    qseq = [0, 1, 1]
    rng = np.random.default_rng(context + 3)
    qi = synth.f32_to_bf16_bits(rng.standard_normal((len(qpos), 8, 64)).astype(np.float32))
    tk, _ = m.csa2_index_topk(gc, "full", dev_u16(qi), dev_i32(qseq), dev_i32(qpos), top_k,
                              q_dtype=q_dtype)
    torch.cuda.synchronize()
    got = host(tk)
    for i, p in enumerate(qpos):
        n = min(p + 1, top_k)
        assert np.all(got[i, n:] == -1)
        if q_dtype == "fp8":
            _relaxed_query(oc, qseq[i], p, O.query_index_values(qi[i], "fp8"), got[i], top_k)
        else:
            want, _, _, _ = O.index_topk("full", oc, qseq[i], p, O.query_index_values(qi[i], "bf16"),
                                         top_k)
            assert np.array_equal(got[i], want), i


def test_large_pool_and_reindex():
    # a pool of 8192 blocks (65536 positions) over 70000 rows, then a Reindex
    # layer over it: pools past the ranked records' size (the pool scorer and
    # the histogram stream)
    announce("pool of 8192 blocks, Reindex over it")
    m = lib()
    context, batch = 70000, 1
    wl = synth.workload("decode_1m", context=context, batch=batch)
    gc = m.Cache(batch, context, idx_heads=8, idx_k_dtype="fp8")
    oc = O.OracleCache(batch, context, idx_heads=8, idx_k_dtype="fp8", lazy=True)
    data = synth.gen_batch(wl)
    seq, pos = np.zeros(context, np.int32), np.arange(context, dtype=np.int32)
    m.csa2_kv_append(gc, dev_u16(data.k[0]), dev_u16(data.v[0]), dev_u16(data.ik[0]),
                     dev_i32(seq), dev_i32(pos))
    oc.append(data.k[0], data.v[0], data.ik[0], seq, pos)
    del data
    qpos = [context - 1, 60000]
    rng = np.random.default_rng(8192)
    qi = synth.f32_to_bf16_bits(rng.standard_normal((2, 2, 8, 64)).astype(np.float32))
    tk, pool = m.csa2_index_topk(gc, "full", dev_u16(qi[0]), dev_i32([0, 0]), dev_i32(qpos), 2048,
                                 pool_blocks=8192)
    tk2, _ = m.csa2_index_topk(gc, "reindex", dev_u16(qi[1]), dev_i32([0, 0]), dev_i32(qpos), 2048,
                               pool_in=pool)
    torch.cuda.synchronize()
    for i, p in enumerate(qpos):
        t, pl, _, _ = O.index_topk("full", oc, 0, p, O.query_index_values(qi[0, i], "bf16"), 2048,
                                   pool_blocks=8192)
        assert np.array_equal(host(tk)[i], t) and np.array_equal(host(pool)[i], pl), i
        t2, _, _, _ = O.index_topk("reindex", oc, 0, p, O.query_index_values(qi[1, i], "bf16"),
                                   2048, pool_in=pl)
        assert np.array_equal(host(tk2)[i], t2), i


# ---------------------------------------------------------------------------
# matrix-core scorer (E4M3 index query, E4M3 keys, every visible position)
# ---------------------------------------------------------------------------

def _relaxed_query(oc, seq, qp, qi, got_row, top_k):
    cand = np.arange(qp + 1)
    keys = oc.index_key_values(seq, cand)
    canon = O.index_scores(qi, keys)
    exact, mag = O.index_scores_exact(qi, keys)
    want = O.topk_select(canon, cand, top_k)
    return relaxed_topk_check(got_row, want, cand, canon, exact, mag)


@pytest.mark.parametrize("mode", ["full", "reindex"])
@pytest.mark.parametrize("heads", [8, 4])
@pytest.mark.parametrize("top_k", [1, 37, 256, 3000])
def test_matrix_core_topk(mode, heads, top_k):
    # six queries, each of its own sequence: one query group spanning six sequences
    announce(f"matrix-core {mode} heads={heads} k={top_k}")
    m = lib()
    wl, gc, oc = _setup(heads, "fp8")
    qd = synth.gen_queries(wl, 0)
    ws_bytes = m.csa2_index_topk_workspace(gc, mode, len(QPOS), top_k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    topk, _ = m.csa2_index_topk(gc, mode, dev_u16(qd.q_idx), dev_i32(np.arange(len(QPOS))),
                                dev_i32(QPOS), top_k, q_dtype="fp8", workspace=ws)
    torch.cuda.synchronize()
    got = host(topk)
    swaps = 0
    for i, p in enumerate(QPOS):
        qi = O.query_index_values(qd.q_idx[i], "fp8")
        swaps += _relaxed_query(oc, i, p, qi, got[i], top_k)
        if p + 1 <= top_k:   # everything visible is selected: exact
            assert list(got[i, :p + 1]) == list(range(p + 1))
    announce(f"  swaps at the K-th score: {swaps}")


def test_matrix_core_prefill_chunk():
    # 700 consecutive queries of one sequence (two query groups, the second
    # ragged), causal: query i sees positions [0, 4308 + i]
    announce("matrix-core prefill chunk")
    m = lib()
    wl, gc, oc = _setup(8, "fp8")
    nq, top_k, seq = 700, 256, 3
    qpos = np.arange(CAP - nq, CAP)
    rng = np.random.default_rng(21)
    qidx = synth.f32_to_bf16_bits(rng.standard_normal((nq, 8, 64)).astype(np.float32) * 2)
    topk, _ = m.csa2_index_topk(gc, "full", dev_u16(qidx), dev_i32(np.full(nq, seq)),
                                dev_i32(qpos), top_k, q_dtype="fp8")
    torch.cuda.synchronize()
    got = host(topk)
    assert np.all((got >= 0) & (got <= qpos[:, None]))          # causal, no padding needed
    assert np.all(np.diff(got, axis=1) > 0)
    swaps = 0
    for i in list(range(0, nq, 23)) + [511, 512, nq - 1]:
        qi = O.query_index_values(qidx[i], "fp8")
        swaps += _relaxed_query(oc, seq, int(qpos[i]), qi, got[i], top_k)
    announce(f"  swaps at the K-th score: {swaps}")


@pytest.mark.parametrize("distinct,cap", [(1, 20000), (2, 40000), (3, 3008)])
def test_matrix_core_tie_heavy(distinct, cap):
    # few distinct scores: every position of a tied block reaches the
    # threshold, so the candidates overflow the LDS resolve (cap >= 20000)
    announce(f"matrix-core ties distinct={distinct} cap={cap}")
    m = lib()
    gc = m.Cache(2, cap, idx_heads=8, idx_k_dtype="fp8")
    oc = O.OracleCache(2, cap, idx_heads=8, idx_k_dtype="fp8")
    rng = np.random.default_rng(distinct)
    base = synth.f32_to_bf16_bits(rng.standard_normal((distinct, 8, 64)).astype(np.float32))
    ik = base[rng.integers(0, distinct, cap)]
    kv = synth.f32_to_bf16_bits(rng.standard_normal((cap, 128)).astype(np.float32))
    for b in range(2):
        seq, pos = np.full(cap, b, np.int32), np.arange(cap, dtype=np.int32)
        m.csa2_kv_append(gc, dev_u16(kv), dev_u16(kv), dev_u16(ik), dev_i32(seq), dev_i32(pos))
        oc.append(kv, kv, ik, seq, pos)
    qi = synth.f32_to_bf16_bits(rng.standard_normal((2, 8, 64)).astype(np.float32))
    qpos = [cap - 1, 1234]
    tk, _ = m.csa2_index_topk(gc, "full", dev_u16(qi), dev_i32([0, 1]), dev_i32(qpos), 500,
                              q_dtype="fp8")
    torch.cuda.synchronize()
    got = host(tk)
    for i in range(2):
        _relaxed_query(oc, i, qpos[i], O.query_index_values(qi[i], "fp8"), got[i], 500)
    if distinct == 1:   # identical keys give identical sums: ties to the lower position
        assert list(got[0]) == list(range(500)) and list(got[1]) == list(range(500))


def test_matrix_core_long_rows():
    # positions past 524288: a query's block maxima (one per 16 positions) no
    # longer fit the threshold kernel's registers and are counted from global
    # memory; a query below the limit in the same call keeps the register path
    context = 540000
    qpos = [539999, 530000, 100000]
    announce(f"matrix-core long rows context={context}")
    m = lib()
    wl = synth.workload("decode_1m", context=context, batch=1)
    gc = m.Cache(1, context, idx_heads=8, idx_k_dtype="fp8")
    oc = O.OracleCache(1, context, idx_heads=8, idx_k_dtype="fp8", lazy=True)
    data = synth.gen_batch(wl)
    seq, pos = np.zeros(context, np.int32), np.arange(context, dtype=np.int32)
    m.csa2_kv_append(gc, dev_u16(data.k[0]), dev_u16(data.v[0]), dev_u16(data.ik[0]),
                     dev_i32(seq), dev_i32(pos))
    oc.append(data.k[0], data.v[0], data.ik[0], seq, pos)
    del data
    rng = np.random.default_rng(context)
    qi = synth.f32_to_bf16_bits(rng.standard_normal((len(qpos), 8, 64)).astype(np.float32))
    top_k = 2048
    tk, _ = m.csa2_index_topk(gc, "full", dev_u16(qi), dev_i32([0] * len(qpos)), dev_i32(qpos),
                              top_k, q_dtype="fp8")
    torch.cuda.synchronize()
    got = host(tk)
    swaps = 0
    for i, p in enumerate(qpos):
        swaps += _relaxed_query(oc, 0, p, O.query_index_values(qi[i], "fp8"), got[i], top_k)
    announce(f"  swaps at the K-th score: {swaps}")


@pytest.mark.parametrize("context", [163840, 163856])
def test_matrix_core_threshold_register_edge(context):
    # 163840 positions: 10240 block maxima per row, every register group of the
    # one-wave threshold search full; 16 positions more and the calls take the
    # workgroup threshold kernel.  Queries at the last position, inside the
    # last block, with exactly K blocks, and with fewer than K blocks (no
    # threshold: every visible position is a candidate)
    qpos = [context - 1, context - 9, 16 * 2048 - 1, 16 * 2048 - 17, 100]
    announce(f"matrix-core threshold edge context={context}")
    m = lib()
    wl = synth.workload("decode_1m", context=context, batch=1)
    gc = m.Cache(1, context, idx_heads=8, idx_k_dtype="fp8")
    oc = O.OracleCache(1, context, idx_heads=8, idx_k_dtype="fp8", lazy=True)
    data = synth.gen_batch(wl)
    seq, pos = np.zeros(context, np.int32), np.arange(context, dtype=np.int32)
    m.csa2_kv_append(gc, dev_u16(data.k[0]), dev_u16(data.v[0]), dev_u16(data.ik[0]),
                     dev_i32(seq), dev_i32(pos))
    oc.append(data.k[0], data.v[0], data.ik[0], seq, pos)
    del data
    rng = np.random.default_rng(context + 1)
    qi = synth.f32_to_bf16_bits(rng.standard_normal((len(qpos), 8, 64)).astype(np.float32))
    top_k = 2048
    tk, _ = m.csa2_index_topk(gc, "full", dev_u16(qi), dev_i32([0] * len(qpos)), dev_i32(qpos),
                              top_k, q_dtype="fp8")
    torch.cuda.synchronize()
    got = host(tk)
    swaps = 0
    for i, p in enumerate(qpos):
        swaps += _relaxed_query(oc, 0, p, O.query_index_values(qi[i], "fp8"), got[i], top_k)
    assert list(got[4, :101]) == list(range(101)) and np.all(got[4, 101:] == -1)
    announce(f"  swaps at the K-th score: {swaps}")


def test_matrix_core_topk_is_deterministic():
    # run twice on the same inputs: identical bytes (the block maxima, the
    # threshold, the candidate totals and the candidate compaction use atomics
    # and cross-workgroup ordering, which must not leak into the result); a
    # 700-query chunk of one sequence (K 2048 and 128) plus six queries of six
    # sequences (the sampled threshold's run-twice check is in
    # test_matrix_core_sampled_threshold_matches_exact)
    announce("matrix-core determinism")
    m = lib()
    wl, gc, oc = _setup(8, "fp8")
    rng = np.random.default_rng(5)
    nq = 700
    qpos = np.arange(CAP - nq, CAP)
    qidx = synth.f32_to_bf16_bits(rng.standard_normal((nq, 8, 64)).astype(np.float32) * 2)
    cases = [(dev_u16(qidx), dev_i32(np.full(nq, 3)), dev_i32(qpos), 2048),
             (dev_u16(qidx), dev_i32(np.full(nq, 3)), dev_i32(qpos), 128),
             (dev_u16(synth.gen_queries(wl, 0).q_idx), dev_i32(np.arange(len(QPOS))),
              dev_i32(QPOS), 256)]
    for q_idx, q_seq, q_pos, top_k in cases:
        runs = []
        for _ in range(2):
            tk, _ = m.csa2_index_topk(gc, "full", q_idx, q_seq, q_pos, top_k, q_dtype="fp8")
            torch.cuda.synchronize()
            runs.append(host(tk))
        assert np.array_equal(runs[0], runs[1])


@pytest.mark.parametrize("nq,heads,idx_dtype,cap", [(64, 8, "fp8", 16400), (128, 8, "fp8", 16400),
                                                     (128, 4, "bf16", 16400), (64, 8, "fp8", 40000)])
def test_full_topk_chunk_histograms(nq, heads, idx_dtype, cap):
    # enough queries x candidates for the scorer's 2048- (64 queries x 16400)
    # and 4096-candidate workgroups, at most 16 chunks per query: each
    # workgroup stores its chunk's keys in bin order with the counts at or
    # above every bin (ranked chunk records), and one selection workgroup per
    # query reads the threshold bin off the counts and then only the keys at
    # or above it.  Queries at chunk boundaries and in the ragged last chunk.
    announce(f"chunk histograms nq={nq} heads={heads} idx={idx_dtype}")
    m = lib()
    nseq = 4
    wl = synth.workload("decode_64k_b32", context=cap, batch=nseq, idx_heads=heads,
                        idx_k_dtype=idx_dtype, seed=9)
    gc, oc, _ = filled_caches(wl)
    rng = np.random.default_rng(nq + heads)
    special = [p for p in (0, 5, 2047, 2048, 4095, 4096, 8191, 12288, 16383, 16384, 36863, 36864)
               if p < cap] + [cap - 1]
    qpos = np.concatenate([special, rng.integers(0, cap, nq - len(special))]).astype(np.int32)
    qseq = (np.arange(nq) % nseq).astype(np.int32)
    qidx = synth.f32_to_bf16_bits(rng.standard_normal((nq, heads, 64)).astype(np.float32))
    got = {}
    for top_k in (2048, 100):
        tk, _ = m.csa2_index_topk(gc, "full", dev_u16(qidx), dev_i32(qseq), dev_i32(qpos), top_k)
        torch.cuda.synchronize()
        got[top_k] = host(tk)
    for i in range(nq):
        qi = O.query_index_values(qidx[i], "bf16")
        want, _, scores, cand = O.index_topk("full", oc, int(qseq[i]), int(qpos[i]), qi, 2048)
        assert np.array_equal(got[2048][i], want), (2048, i, int(qpos[i]))
        assert np.array_equal(got[100][i], O.topk_select(scores, cand, 100)), (100, i, int(qpos[i]))


def _ranked_ws_keys(ws, nq, cap):
    """(keys, positions) of a ranked-chunk call from its workspace: the
    library's internal layout -- keys [nq][n] uint32 (each chunk's keys in bin
    order), then at the next 256-B boundary their chunk-local positions
    [nq][n] uint16, n = roundup64(capacity)."""
    n = (cap + 63) // 64 * 64
    kb = nq * n * 4
    raw = host(ws).view(np.uint8)
    keys = raw[:kb].view(np.uint32).reshape(nq, n)
    po = (kb + 255) // 256 * 256
    pos = raw[po:po + nq * n * 2].view(np.uint16).reshape(nq, n)
    return keys, pos


@pytest.mark.parametrize("nq,cap,chunk", [(64, 16400, 2048), (128, 16400, 4096)])
def test_ranked_chunk_records(nq, cap, chunk):
    # the scorer's ranked records: per chunk the keys are the oracle's score
    # keys of the chunk's positions (bit for bit), each position once, in
    # non-increasing order of their top 12 bits
    announce(f"ranked chunk records nq={nq} cap={cap}")
    m = lib()
    wl = synth.workload("decode_64k_b32", context=cap, batch=4, seed=21)
    gc, oc, _ = filled_caches(wl)
    rng = np.random.default_rng(nq)
    qpos = np.concatenate([[0, chunk - 1, chunk, cap - 1],
                           rng.integers(0, cap, nq - 4)]).astype(np.int32)
    qseq = (np.arange(nq) % 4).astype(np.int32)
    qidx = synth.f32_to_bf16_bits(rng.standard_normal((nq, 8, 64)).astype(np.float32))
    ws = torch.empty(m.csa2_index_topk_workspace(gc, "full", nq, 2048), dtype=torch.uint8, device=DEV)
    m.csa2_index_topk(gc, "full", dev_u16(qidx), dev_i32(qseq), dev_i32(qpos), 2048, workspace=ws)
    torch.cuda.synchronize()
    keys, pos = _ranked_ws_keys(ws, nq, cap)
    for i in range(0, nq, 7):
        p = int(qpos[i])
        cand = np.arange(p + 1)
        want = _score_keys(O.index_scores(O.query_index_values(qidx[i], "bf16"),
                                          oc.index_key_values(int(qseq[i]), cand)))
        for c0 in range(0, p + 1, chunk):
            cnt = min(chunk, p + 1 - c0)
            k = keys[i, c0:c0 + cnt]
            lp = pos[i, c0:c0 + cnt].astype(np.int64)
            assert np.array_equal(np.sort(lp), np.arange(cnt)), (i, c0)
            assert np.array_equal(k, want[c0 + lp]), (i, c0)
            assert np.all(np.diff((k >> 20).astype(np.int64)) <= 0), (i, c0)


@pytest.mark.parametrize("distinct", [1, 2, 3])
def test_ranked_tie_heavy_keys(distinct):
    # few distinct index keys over 16400 positions, 64 queries (ranked chunk
    # records of 2048 keys): the threshold bin holds thousands of equal keys
    # -- past 8192 of them the selection reads them from the records in every
    # pass -- and the keys equal to the K-th go to the lowest positions
    announce(f"ranked ties distinct={distinct}")
    m = lib()
    cap, nq = 16400, 64
    gc = m.Cache(2, cap, idx_heads=8, idx_k_dtype="fp8")
    oc = O.OracleCache(2, cap, idx_heads=8, idx_k_dtype="fp8")
    rng = np.random.default_rng(100 + distinct)
    base = synth.f32_to_bf16_bits(rng.standard_normal((distinct, 8, 64)).astype(np.float32))
    kv = synth.f32_to_bf16_bits(rng.standard_normal((cap, 128)).astype(np.float32))
    for b in range(2):
        ik = base[rng.integers(0, distinct, cap)]
        seq, pos = np.full(cap, b, np.int32), np.arange(cap, dtype=np.int32)
        m.csa2_kv_append(gc, dev_u16(kv), dev_u16(kv), dev_u16(ik), dev_i32(seq), dev_i32(pos))
        oc.append(kv, kv, ik, seq, pos)
    qpos = np.concatenate([[cap - 1, 0, 99, 2047, 2048, 9000],
                           rng.integers(0, cap, nq - 6)]).astype(np.int32)
    qseq = (np.arange(nq) % 2).astype(np.int32)
    qidx = synth.f32_to_bf16_bits(rng.standard_normal((nq, 8, 64)).astype(np.float32))
    got = {}
    for top_k in (2048, 100, 9000):
        tk, _ = m.csa2_index_topk(gc, "full", dev_u16(qidx), dev_i32(qseq), dev_i32(qpos), top_k)
        torch.cuda.synchronize()
        got[top_k] = host(tk)
    for i in range(nq):
        _, _, scores, cand = O.index_topk("full", oc, int(qseq[i]), int(qpos[i]),
                                          O.query_index_values(qidx[i], "bf16"), 1)
        for top_k, g in got.items():
            assert np.array_equal(g[i], O.topk_select(scores, cand, top_k)), (top_k, i, int(qpos[i]))


def test_ranked_poisoned_workspace_reused():
    # a workspace full of stale bytes, then the same workspace again (ranked
    # records of 2048 keys): the same exact Top-K both times
    announce("ranked selection, poisoned then reused workspace")
    m = lib()
    cap, nq = 16400, 64
    wl = synth.workload("decode_64k_b32", context=cap, batch=2, seed=5)
    gc, oc, _ = filled_caches(wl)
    rng = np.random.default_rng(3)
    qpos = rng.integers(0, cap, nq).astype(np.int32)
    qpos[0] = cap - 1
    qseq = (np.arange(nq) % 2).astype(np.int32)
    qidx = synth.f32_to_bf16_bits(rng.standard_normal((nq, 8, 64)).astype(np.float32))
    ws = torch.full((m.csa2_index_topk_workspace(gc, "full", nq, 300),), 0xAB, dtype=torch.uint8,
                    device=DEV)
    runs = []
    for _ in range(2):
        tk, _ = m.csa2_index_topk(gc, "full", dev_u16(qidx), dev_i32(qseq), dev_i32(qpos), 300,
                                  workspace=ws)
        torch.cuda.synchronize()
        runs.append(host(tk))
    for i in range(nq):
        want, _, _, _ = O.index_topk("full", oc, int(qseq[i]), int(qpos[i]),
                                     O.query_index_values(qidx[i], "bf16"), 300)
        assert np.array_equal(runs[0][i], want), i
        assert np.array_equal(runs[1][i], want), i


def test_matrix_core_sampled_threshold_matches_exact():
    # Rows of at least 2K blocks, with position ranges of at least 8 groups of
    # 256 positions, take the sampled first pass: the block maxima of each
    # range's first eighth of groups.  600 queries make 128 ranges, so the
    # 262144-position cache has ranges of 2048 positions, sampled in their
    # first 256; a 1572864-position cache has more sampled block maxima than
    # one wave's threshold registers hold and takes the exact two-pass path.
    # The same keys in both give the same scores (same instructions per
    # position), so every Top-K must be the same bytes.  Query 5 is built so
    # that the sample misleads it: the keys of the sampled positions point
    # along its own direction, so its sampled threshold admits fewer than K
    # positions and the checking launch gives it every visible position.  The
    # sampled path runs twice (identical bytes: determinism).
    cap_a, cap_b, top_k, nq = 262144, 1572864, 512, 600
    announce(f"matrix-core sampled threshold vs exact cap={cap_a} k={top_k} nq={nq}")
    m = lib()
    rng = np.random.default_rng(77)
    u = rng.standard_normal((8, 64)).astype(np.float32)
    ik = rng.standard_normal((cap_a, 8, 64)).astype(np.float32)
    sampled = (np.arange(cap_a) % 2048) < 256
    ik[sampled] = 2 * u + 0.3 * ik[sampled]
    ik = synth.f32_to_bf16_bits(ik)
    kv = synth.f32_to_bf16_bits(rng.standard_normal((cap_a, 128)).astype(np.float32))
    qidx = rng.standard_normal((nq, 8, 64)).astype(np.float32)
    qidx[5] = u
    qidx = synth.f32_to_bf16_bits(qidx)
    qpos = rng.integers(cap_a // 2, cap_a, nq).astype(np.int32)
    qpos[5] = cap_a - 1
    seq, pos = np.zeros(cap_a, np.int32), np.arange(cap_a, dtype=np.int32)
    got = []
    for cap in (cap_a, cap_a, cap_b):
        gc = m.Cache(1, cap, idx_heads=8, idx_k_dtype="fp8")
        m.csa2_kv_append(gc, dev_u16(kv), dev_u16(kv), dev_u16(ik), dev_i32(seq), dev_i32(pos))
        tk, _ = m.csa2_index_topk(gc, "full", dev_u16(qidx), dev_i32(np.zeros(nq)), dev_i32(qpos),
                                  top_k, q_dtype="fp8")
        torch.cuda.synchronize()
        got.append(host(tk))
        del gc, tk
        torch.cuda.empty_cache()
    assert np.array_equal(got[0], got[1])
    assert np.array_equal(got[0], got[2])
    oc = O.OracleCache(1, cap_a, idx_heads=8, idx_k_dtype="fp8", lazy=True)
    oc.append(kv, kv, ik, seq, pos)
    swaps = 0
    for i in [5, 0, 511, nq - 1]:
        qi = O.query_index_values(qidx[i], "fp8")
        swaps += _relaxed_query(oc, 0, int(qpos[i]), qi, got[0][i], top_k)
    announce(f"  swaps at the K-th score: {swaps}")


@pytest.mark.parametrize("distinct", [1, 3])
def test_matrix_core_sampled_threshold_tie_heavy(distinct):
    # 4096 queries of one sequence on 65536 positions: 32 position ranges of
    # 2048, so the sampled first pass runs.  Few distinct index keys give few
    # distinct scores: the sampled threshold equals a tied value, every
    # position of that value is a candidate (the resolve streams them) and the
    # ties go to the lower positions.
    cap, nq, top_k = 65536, 4096, 256
    announce(f"matrix-core sampled threshold, ties distinct={distinct}")
    m = lib()
    rng = np.random.default_rng(100 + distinct)
    base = synth.f32_to_bf16_bits(rng.standard_normal((distinct, 8, 64)).astype(np.float32))
    ik = base[rng.integers(0, distinct, cap)]
    kv = synth.f32_to_bf16_bits(rng.standard_normal((cap, 128)).astype(np.float32))
    gc = m.Cache(1, cap, idx_heads=8, idx_k_dtype="fp8")
    oc = O.OracleCache(1, cap, idx_heads=8, idx_k_dtype="fp8", lazy=True)
    seq, pos = np.zeros(cap, np.int32), np.arange(cap, dtype=np.int32)
    m.csa2_kv_append(gc, dev_u16(kv), dev_u16(kv), dev_u16(ik), dev_i32(seq), dev_i32(pos))
    oc.append(kv, kv, ik, seq, pos)
    qi = synth.f32_to_bf16_bits(rng.standard_normal((nq, 8, 64)).astype(np.float32))
    qpos = np.arange(cap - nq, cap, dtype=np.int32)
    tk, _ = m.csa2_index_topk(gc, "full", dev_u16(qi), dev_i32(np.zeros(nq)), dev_i32(qpos), top_k,
                              q_dtype="fp8")
    torch.cuda.synchronize()
    got = host(tk)
    assert np.all(np.diff(got, axis=1) > 0)
    for i in [0, 1, 2047, nq - 1]:
        _relaxed_query(oc, 0, int(qpos[i]), O.query_index_values(qi[i], "fp8"), got[i], top_k)
    if distinct == 1:   # identical keys give identical sums: ties to the lower position
        assert np.array_equal(got, np.broadcast_to(np.arange(top_k), got.shape))


def test_matrix_core_sampled_threshold_two_sequences():
    # The sampled path with two sequences in one 512-query group (one pass per
    # sequence) and a ragged second group: 700 queries (300 of sequence 0, 400
    # of sequence 1, at scattered positions), against the exact two-pass path
    # on a cache too long for the sample (same keys, same score bits).
    cap_a, cap_b, top_k, nq = 262144, 1572864, 384, 700
    announce(f"matrix-core sampled threshold, two sequences, nq={nq}")
    m = lib()
    rng = np.random.default_rng(91)
    ik = [synth.f32_to_bf16_bits(rng.standard_normal((cap_a, 8, 64)).astype(np.float32))
          for _ in range(2)]
    kv = synth.f32_to_bf16_bits(rng.standard_normal((cap_a, 128)).astype(np.float32))
    qidx = synth.f32_to_bf16_bits(rng.standard_normal((nq, 8, 64)).astype(np.float32))
    qseq = np.array([0] * 300 + [1] * 400, np.int32)
    qpos = rng.integers(cap_a // 2, cap_a, nq).astype(np.int32)
    qpos[0] = qpos[300] = cap_a - 1
    pos = np.arange(cap_a, dtype=np.int32)
    got = []
    for cap in (cap_a, cap_b):
        gc = m.Cache(2, cap, idx_heads=8, idx_k_dtype="fp8")
        for b in range(2):
            m.csa2_kv_append(gc, dev_u16(kv), dev_u16(kv), dev_u16(ik[b]),
                             dev_i32(np.full(cap_a, b)), dev_i32(pos))
        tk, _ = m.csa2_index_topk(gc, "full", dev_u16(qidx), dev_i32(qseq), dev_i32(qpos), top_k,
                                  q_dtype="fp8")
        torch.cuda.synchronize()
        got.append(host(tk))
        del gc, tk
        torch.cuda.empty_cache()
    assert np.array_equal(got[0], got[1])
    oc = O.OracleCache(2, cap_a, idx_heads=8, idx_k_dtype="fp8", lazy=True)
    for b in range(2):
        oc.append(kv, kv, ik[b], np.full(cap_a, b), pos)
    for i in [0, 299, 300, 511, 512, nq - 1]:
        _relaxed_query(oc, int(qseq[i]), int(qpos[i]), O.query_index_values(qidx[i], "fp8"),
                       got[0][i], top_k)
