"""Pins of the oracle's sparse attention: textbook dense attention and closed forms."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import csa2 as O


def _cache(context=64, seed=0):
    wl = synth.workload("tiny_4k", context=context, seed=seed)
    c = O.OracleCache(1, context, idx_heads=4, idx_k_dtype="bf16")
    d = synth.gen_sequence(wl, 0)
    c.append(d.k, d.v, d.ik, np.zeros(context, int), np.arange(context))
    return wl, c


def test_all_rows_equals_dense_attention_textbook():
    wl, c = _cache()
    q = synth.gen_queries(wl, 0).q[0]
    out, lse = O.sparse_attention(q, c, 0, np.arange(64))
    k, v = c.kv_values(0, np.arange(64))
    qv = torch.from_numpy(synth.bf16_bits_to_f32(q).astype(np.float64))[None]      # [1, H, d]
    kt = torch.from_numpy(k)[None, None].expand(1, qv.shape[1], 64, 128)
    vt = torch.from_numpy(v)[None, None].expand(1, qv.shape[1], 64, 128)
    scale = float(np.float32(1 / math.sqrt(128)))
    ref = torch.nn.functional.scaled_dot_product_attention(qv[:, :, None], kt, vt, scale=scale)
    assert np.allclose(out, ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)
    z = (qv[0] @ torch.from_numpy(k).T) * scale
    assert np.allclose(lse, torch.logsumexp(z, dim=1).numpy(), rtol=1e-12, atol=1e-12)


def test_single_row_returns_that_row():
    wl, c = _cache()
    q = synth.gen_queries(wl, 0).q[0]
    out, lse = O.sparse_attention(q, c, 0, np.array([17, -1, -1]))
    k, v = c.kv_values(0, np.array([17]))
    assert np.array_equal(out, np.broadcast_to(v, out.shape))
    qv = synth.bf16_bits_to_f32(q).astype(np.float64)
    assert np.allclose(lse, (qv @ k[0]) * float(np.float32(1 / math.sqrt(128))), rtol=1e-14)


def test_equal_keys_give_mean_of_values():
    wl, c = _cache()
    c.kv_codes[0, :, :64] = c.kv_codes[0, 0, :64]
    c.kv_scales[0, :, :8] = c.kv_scales[0, 0, :8]
    q = synth.gen_queries(wl, 0).q[0]
    rows = np.array([3, 9, 20, 33])
    out, lse = O.sparse_attention(q, c, 0, rows)
    _, v = c.kv_values(0, rows)
    assert np.allclose(out, v.mean(axis=0)[None], rtol=1e-12, atol=1e-12)
    out1, lse1 = O.sparse_attention(q, c, 0, rows[:1])
    assert np.allclose(lse, lse1 + math.log(4), rtol=1e-12)


def test_convex_hull_and_permutation_invariance():
    wl, c = _cache(seed=4)
    q = synth.gen_queries(wl, 0).q[0]
    rng = np.random.default_rng(0)
    rows = rng.choice(64, 20, replace=False)
    out, lse = O.sparse_attention(q, c, 0, rows)
    _, v = c.kv_values(0, rows)
    assert np.all(out <= v.max(axis=0) + 1e-12) and np.all(out >= v.min(axis=0) - 1e-12)
    out2, lse2 = O.sparse_attention(q, c, 0, rng.permutation(rows))
    assert np.allclose(out, out2, rtol=1e-13, atol=1e-13) and np.allclose(lse, lse2, rtol=1e-13)


def test_empty_selection():
    wl, c = _cache()
    q = synth.gen_queries(wl, 0).q[0]
    out, lse = O.sparse_attention(q, c, 0, np.full(8, -1))
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_duplicate_entries_count_twice():
    wl, c = _cache()
    q = synth.gen_queries(wl, 0).q[0]
    a, la = O.sparse_attention(q, c, 0, np.array([5, 5, 6]))
    k, v = c.kv_values(0, np.array([5, 6]))
    qv = synth.bf16_bits_to_f32(q).astype(np.float64)
    z = (qv @ k.T) * float(np.float32(1 / math.sqrt(128)))
    w = np.exp(z) * np.array([2.0, 1.0])
    want = (w @ v) / w.sum(axis=1, keepdims=True)
    assert np.allclose(a, want, rtol=1e-12, atol=1e-12)
