"""Pins of the oracle's Top-K, candidate pool and Full/Reindex/Reuse modes.

Top-K and the pool are checked against brute force (Python's sorted on tuples,
explicit loops over blocks) and special cases; the modes against the invariants
the pages fix (a Reindex over everything equals Full; Reuse returns the source
indices unchanged).
"""
import numpy as np
import pytest

import synth
from oracle import csa2 as O


def _brute_topk(scores, positions, k):
    items = sorted(zip((-float(np.float32(s)) + 0.0 for s in scores), positions))
    chosen = sorted(p for _, p in items[:k])
    return chosen + [-1] * (k - len(chosen))


@pytest.mark.parametrize("seed", range(40))
def test_topk_vs_sorted_tuples(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 60))
    k = int(rng.integers(1, 40))
    # few distinct values -> many ties
    s = rng.integers(-3, 4, n).astype(np.float32) * np.float32(0.5)
    pos = np.sort(rng.choice(1000, n, replace=False))
    assert list(O.topk_select(s, pos, k)) == _brute_topk(s, pos, k)


def test_topk_all_equal_takes_lowest_positions():
    s = np.full(100, 3.25, np.float32)
    assert list(O.topk_select(s, np.arange(100), 10)) == list(range(10))


def test_topk_signed_zeros_are_equal():
    s = np.array([-0.0, 0.0, -0.0, 0.0, -1.0], np.float32)
    assert list(O.topk_select(s, np.arange(5), 3)) == [0, 1, 2]
    s = np.array([0.0, -0.0, 0.0], np.float32)
    assert list(O.topk_select(s, np.array([7, 3, 9]), 2)) == [3, 7]


def test_topk_fewer_candidates_pads():
    s = np.array([1.0, 2.0], np.float32)
    assert list(O.topk_select(s, np.array([4, 2]), 5)) == [2, 4, -1, -1, -1]
    assert list(O.topk_select(np.zeros(0, np.float32), np.zeros(0, int), 3)) == [-1, -1, -1]


def _brute_pool(scores, pool_blocks):
    n = len(scores)
    blocks = []
    for b in range((n + 7) // 8):
        members = list(range(8 * b, min(n, 8 * b + 8)))
        blocks.append((-max(float(scores[p]) for p in members) + 0.0, b, members))
    blocks.sort()
    kept = sorted(blocks[:pool_blocks], key=lambda t: t[1])
    pos = [p for _, _, m in kept for p in m]
    return pos + [-1] * (8 * pool_blocks - len(pos))


@pytest.mark.parametrize("seed", range(30))
def test_pool_vs_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 120))
    pb = int(rng.integers(1, 12))
    s = rng.integers(-4, 5, n).astype(np.float32)
    assert list(O.build_pool(s, pb)) == _brute_pool(s, pb)


def _small_cache(seed=0, context=200, idx_k_dtype="fp8", heads=8):
    wl = synth.workload("decode_64k_b32", context=context, batch=2, idx_k_dtype=idx_k_dtype,
                        idx_heads=heads, seed=seed)
    c = O.OracleCache(2, context, idx_heads=heads, idx_k_dtype=idx_k_dtype)
    for b in range(2):
        d = synth.gen_sequence(wl, b)
        c.append(d.k, d.v, d.ik, np.full(context, b), np.arange(context))
    return wl, c


@pytest.mark.parametrize("q_pos", [0, 5, 8, 101, 199])
def test_reindex_over_full_pool_equals_full(q_pos):
    wl, c = _small_cache()
    qd = synth.gen_queries(wl, 0)
    qi = O.query_index_values(qd.q_idx[1], "bf16")
    pb = (q_pos + 1 + 7) // 8     # pool as large as the visible context
    full, pool, _, _ = O.index_topk("full", c, 1, q_pos, qi, 16, pool_blocks=pb)
    assert list(pool[pool >= 0]) == list(range(q_pos + 1))
    re, _, _, _ = O.index_topk("reindex", c, 1, q_pos, qi, 16, pool_in=pool)
    assert np.array_equal(full, re)
    # no pool = all visible
    re2, _, _, _ = O.index_topk("reindex", c, 1, q_pos, qi, 16, pool_in=None)
    assert np.array_equal(full, re2)


def test_reindex_searches_only_the_pool():
    wl, c = _small_cache(seed=3)
    qd = synth.gen_queries(wl, 0)
    qi = O.query_index_values(qd.q_idx[0], "bf16")
    pool = np.array([3, 4, 5, 40, 41, 190, -1, -1], np.int32)
    topk, _, scores, cand = O.index_topk("reindex", c, 0, 150, qi, 4, pool_in=pool)
    assert set(topk[topk >= 0]) <= {3, 4, 5, 40, 41}           # 190 is beyond q_pos
    assert list(cand) == [3, 4, 5, 40, 41]


def test_reuse_is_identity():
    wl, c = _small_cache()
    src = np.array([0, 5, 9, -1], np.int32)
    out, pool, _, _ = O.index_topk("reuse", c, 0, 10, None, 4, reuse_src=src)
    assert np.array_equal(out, src) and pool is None


def test_full_topk_is_causal_and_matches_brute_force():
    wl, c = _small_cache(seed=5, context=96)
    qd = synth.gen_queries(wl, 0)
    qi = O.query_index_values(qd.q_idx[0], "bf16")
    topk, _, scores, cand = O.index_topk("full", c, 0, 60, qi, 10)
    assert list(cand) == list(range(61))
    assert np.all(topk <= 60)
    assert list(topk) == _brute_topk(scores, list(range(61)), 10)


def test_layer_stack_with_a_smaller_reindex_k():
    # the released pool setting in miniature: Full (K 16) builds a 4-block pool,
    # Reindex selects 5 from it, Reuse recycles those 5
    wl, c = _small_cache(seed=7)
    layers = (synth.Layer("full", pool_blocks=4), synth.Layer("reindex", pool_from=0, top_k=5),
              synth.Layer("reuse", reuse_from=1))
    qs = [synth.gen_queries(wl, li) for li in range(3)]
    q_seq, q_pos = np.array([0, 1]), np.array([199, 120])
    res = O.run_layers(c, layers, q_seq, q_pos, qs, 16, "bf16")
    assert [r["topk"].shape[1] for r in res] == [16, 5, 5]
    for i in range(2):
        qi = O.query_index_values(qs[1].q_idx[i], "bf16")
        pool = res[0]["pool"][i]
        k16, _, scores, cand = O.index_topk("reindex", c, int(q_seq[i]), int(q_pos[i]), qi, 16,
                                            pool_in=pool)
        k5 = res[1]["topk"][i]
        # the 5 best pool members by brute force, and a prefix-closed selection
        assert sorted(k5) == sorted(_brute_topk(scores, list(cand), 5))
        assert set(k5) <= set(k16)
        assert set(k5) <= set(pool[pool >= 0])
        assert np.array_equal(res[2]["topk"][i], k5)
    # the released preset: Reindex layers select 512 from the 2048-block pool
    rel = synth.workload("released_256k_b8")
    assert rel.layers[0].pool_blocks == 2048 and rel.layers[0].top_k == 0 and rel.top_k == 2048
    assert all(L.top_k == 512 for L in rel.layers[1:4])
