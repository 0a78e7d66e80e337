"""Pins of the oracle's local sliding-window branch: the ring of slots, E4M3
codes the OCP format fixes, and the joint softmax against textbook dense
attention and closed forms."""
import math

import numpy as np
import torch

import synth
from oracle import csa2 as O


def _bits(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_ring_holds_the_latest_position_per_slot():
    lc = O.OracleLocalCache(1, 4, dk=128, dv=128)
    rows = np.zeros((10, 128), np.uint16)
    lc.append(rows, rows, np.zeros(10, int), np.arange(10))
    # slot s holds the last position p <= 9 with p % 4 == s
    assert list(lc.pos[0]) == [8, 9, 6, 7]
    assert list(lc.window_rows(0, 9)[0]) == [6, 7, 8, 9]
    assert list(lc.window_rows(0, 7)[0]) == [6, 7]          # 4 and 5 were overwritten
    assert list(lc.window_rows(0, 5)[0]) == []
    # a window wider than the history: positions 0 .. q_pos
    wide = O.OracleLocalCache(1, 128)
    wide.append(rows[:3], rows[:3], np.zeros(3, int), np.arange(3))
    assert list(wide.window_rows(0, 2)[0]) == [0, 1, 2]


def test_e4m3_codes_of_the_window():
    # OCP E4M3FN: 1.0 = 0x38, -2.0 = 0xC0, 448 = 0x7E (largest finite), larger
    # values saturate to it, -0 keeps its sign, 1.0625 lies halfway between
    # 1.0 and 1.125 and rounds to the even code 0x38, 2^-9 = 0x01 (smallest
    # subnormal), 0.375 = 0x2C
    vals = [1.0, -2.0, 448.0, 1000.0, -0.0, 1.0625, 2.0 ** -9, 0.375]
    want = [0x38, 0xC0, 0x7E, 0x7E, 0x80, 0x38, 0x01, 0x2C]
    lc = O.OracleLocalCache(1, 8, dk=8, dv=8)
    k = np.tile(_bits(vals), (8, 1))
    lc.append(k, k, np.zeros(8, int), np.arange(8))
    assert list(lc.k[0, 0]) == want
    _, kv, _ = lc.window_rows(0, 0)
    assert list(kv[0]) == [1.0, -2.0, 448.0, 448.0, 0.0, 1.0, 2.0 ** -9, 0.375]


def _caches(context=64, window=32, seed=0):
    wl = synth.workload("tiny_4k", context=context, seed=seed)
    c = O.OracleCache(1, context, idx_heads=4, idx_k_dtype="bf16")
    d = synth.gen_sequence(wl, 0)
    c.append(d.k, d.v, d.ik, np.zeros(context, int), np.arange(context))
    lc = O.OracleLocalCache(1, window)
    rng = np.random.default_rng(seed)
    lk = _bits(rng.standard_normal((context, 128)))
    lv = _bits(rng.standard_normal((context, 128)))
    lc.append(lk, lv, np.zeros(context, int), np.arange(context))
    return wl, c, lc


def test_union_equals_dense_attention_over_both_sets_textbook():
    wl, c, lc = _caches()
    q = synth.gen_queries(wl, 0).q[0]
    topk = np.array([3, 17, -1, 40, 5])
    out, lse = O.attention_with_window(q, c, 0, topk, lc, q_pos=63)
    ks, vs = c.kv_values(0, np.array([3, 17, 40, 5]))
    _, kl, vl = lc.window_rows(0, 63)
    assert len(kl) == 32
    k = torch.from_numpy(np.concatenate([ks, kl]))
    v = torch.from_numpy(np.concatenate([vs, vl]))
    qv = torch.from_numpy(synth.bf16_bits_to_f32(q).astype(np.float64))
    scale = float(np.float32(1 / math.sqrt(128)))
    H = qv.shape[0]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qv[None, :, None], k[None, None].expand(1, H, -1, 128), v[None, None].expand(1, H, -1, 128),
        scale=scale)
    assert np.allclose(out, ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)
    ref_lse = torch.logsumexp((qv @ k.T) * scale, dim=1).numpy()
    assert np.allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_empty_window_reduces_to_sparse_attention():
    wl, c, _ = _caches()
    q = synth.gen_queries(wl, 0).q[0]
    empty = O.OracleLocalCache(1, 32)
    topk = np.array([1, 2, 9, 30])
    a = O.attention_with_window(q, c, 0, topk, empty, q_pos=40)
    b = O.sparse_attention(q, c, 0, topk)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_zero_keys_give_uniform_weights():
    # q . K = 0 for every row: each row weighs 1/n, lse = ln n
    wl, c, _ = _caches()
    q = synth.gen_queries(wl, 0).q[0]
    lc = O.OracleLocalCache(1, 16)
    rng = np.random.default_rng(3)
    zero = np.zeros((5, 128), np.uint16)
    lv = _bits(rng.standard_normal((5, 128)))
    lc.append(zero, lv, np.zeros(5, int), np.arange(5))
    out, lse = O.attention_with_window(q, c, 0, np.full(4, -1), lc, q_pos=4)
    _, _, vl = lc.window_rows(0, 4)
    assert np.allclose(out, vl.mean(axis=0)[None], rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, math.log(5), rtol=0, atol=1e-12)
    # the same position in both sets counts twice: one FP4 row and one FP8
    # row, both with zero keys, weigh one half each
    c0 = O.OracleCache(1, 16, idx_heads=4, idx_k_dtype="bf16")
    c0.append(zero[:1], lv[:1], np.zeros((1, 4, 64), np.uint16), [0], [0])
    lc1 = O.OracleLocalCache(1, 16)
    lc1.append(zero[:1], lv[:1], [0], [0])
    out, lse = O.attention_with_window(q, c0, 0, np.array([0]), lc1, q_pos=0)
    _, v4 = c0.kv_values(0, np.array([0]))
    _, _, v8 = lc1.window_rows(0, 0)
    assert np.allclose(out, 0.5 * (v4 + v8), rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, math.log(2), rtol=0, atol=1e-12)


def test_nothing_visible():
    wl, c, _ = _caches()
    q = synth.gen_queries(wl, 0).q[0]
    out, lse = O.attention_with_window(q, c, 0, np.full(3, -1), O.OracleLocalCache(1, 8), q_pos=5)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_bounded_replay_rebuilds_the_window_exactly():
    # after positions 0 .. n-1 the ring holds exactly the last min(n, window)
    # of them, so replaying only those rows into an empty ring gives the same
    # codes and slot positions; replaying fewer leaves the older slots empty
    rng = np.random.default_rng(5)
    for n, window in ((300, 64), (40, 64), (64, 64), (65, 64), (1, 1), (7, 1)):
        k = _bits(rng.standard_normal((n, 128)))
        v = _bits(rng.standard_normal((n, 128)))
        live = O.OracleLocalCache(1, window)
        live.append(k, v, np.zeros(n, int), np.arange(n))
        replay = O.OracleLocalCache(1, window)
        lo = max(0, n - window)
        replay.append(k[lo:], v[lo:], np.zeros(n - lo, int), np.arange(lo, n))
        assert np.array_equal(live.k, replay.k) and np.array_equal(live.v, replay.v)
        assert np.array_equal(live.pos, replay.pos)
        for q_pos in (n - 1, max(0, n - 3)):
            a, b = live.window_rows(0, q_pos), replay.window_rows(0, q_pos)
            assert all(np.array_equal(x, y) for x, y in zip(a, b))
    rows = _bits(rng.standard_normal((10, 128)))
    short = O.OracleLocalCache(1, 64)
    short.append(rows, rows, np.zeros(10, int), np.arange(290, 300))
    assert list(short.window_rows(0, 299)[0]) == list(range(290, 300))
