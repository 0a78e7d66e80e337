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
