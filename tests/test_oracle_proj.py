"""Pins of the oracle's encoder-side projection: closed forms (a selection
matrix reproduces the hidden state's channels; a sum that lies exactly
between two bf16 values takes the even one) and the bf16 rounding against
float32 conversion where that is exact."""
import numpy as np

import synth
from oracle import csa2 as O


def _bits(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_selection_weights_copy_the_hidden_channels():
    rng = np.random.default_rng(0)
    d = 96
    x = _bits(rng.standard_normal((5, d)))
    sel = rng.permutation(d)[:40]
    w = np.zeros((40, d), np.float32)
    w[np.arange(40), sel] = 1.0
    assert np.array_equal(O.project_rows(x, _bits(w)), x[:, sel])
    # -1 weights flip the sign bit only
    assert np.array_equal(O.project_rows(x, _bits(-w)), x[:, sel] ^ np.uint16(0x8000))


def test_ties_round_to_even():
    # 1 + 2^-8 lies halfway between 1 (even) and 1 + 2^-7: it becomes 1.0;
    # (1 + 2^-7) + 2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6: it
    # becomes 1 + 2^-6; a hair above the first tie rounds up
    x = _bits([[1.0, 2.0 ** -8, 0.0], [1.0 + 2.0 ** -7, 2.0 ** -8, 0.0],
               [1.0, 2.0 ** -8, 2.0 ** -20]])
    w = _bits([[1.0, 1.0, 1.0]])
    got = O.project_rows(x, w)[:, 0]
    assert list(got) == [0x3F80, 0x3F82, 0x3F81]


def test_rounding_matches_float32_conversion_where_exact():
    # values already representable in float32: bf16 RNE of the float64 value
    # equals the float32 -> bf16 RNE of the same value
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(4000) * np.exp2(rng.integers(-30, 30, 4000))).astype(np.float32)
    v = np.concatenate([v, np.float32([0.0, -0.0, 1.0, -3.5, 2.0 ** -126, 2.0 ** -133])])
    assert np.array_equal(O.bf16_round_bits(v.astype(np.float64)), synth.f32_to_bf16_bits(v))


def test_project_and_append_is_append_of_the_projection():
    rng = np.random.default_rng(2)
    d = 64
    x = _bits(rng.integers(-4, 5, (6, d)) / 4)
    w = _bits(rng.integers(-4, 5, (256 + 8 * 64, d)) / 8)
    a = O.OracleCache(1, 16, idx_heads=8, idx_k_dtype="fp8")
    y = O.project_and_append(a, x, w, np.zeros(6, int), np.arange(6))
    b = O.OracleCache(1, 16, idx_heads=8, idx_k_dtype="fp8")
    b.append(y[:, :128], y[:, 128:256], y[:, 256:].reshape(6, 8, 64), np.zeros(6, int), np.arange(6))
    assert np.array_equal(a.kv_codes, b.kv_codes) and np.array_equal(a.idx_k, b.idx_k)
    # on this grid every sum is exact: y is the exact product, rounded once
    exact = (synth.bf16_bits_to_f32(x).astype(np.float64) @ synth.bf16_bits_to_f32(w).astype(np.float64).T)
    assert np.array_equal(synth.bf16_bits_to_f32(y).astype(np.float64),
                          synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(exact.astype(np.float32))))
