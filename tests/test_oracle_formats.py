"""Pins of the oracle's number formats (E2M1, E4M3, bf16, fp32 FMA).

Each check compares the oracle with something other than itself: the value set
the pages state, the OCP E4M3FN closed form, nearest-value brute force over the
whole grid, or exact rational arithmetic.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    return bits[exp != 0xFF]


def test_e2m1_table_matches_pages():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_values.txt")) if not l.startswith("#")]
    assert len(rows) == 16
    for code, val in rows:
        got = F.e2m1_value(int(code))
        assert float(got) == float(val)
        assert np.signbit(got) == val.startswith("-")


def test_e4m3_closed_form():
    # OCP E4M3FN: bias 7, subnormal step 2^-9, max 448, 0x7F NaN, no infinities.
    v = F.e4m3_value(np.arange(256))
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9
    assert v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6
    assert v[0x38] == 1.0
    assert v[0x39] == 1.125
    assert v[0x30] == 0.5
    assert v[0x7E] == 448.0
    assert v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    finite = v[:127]
    assert np.all(np.diff(finite) > 0)                 # strictly increasing
    assert np.all(v[128:255] == -finite)


def test_e4m3_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(F.e4m3_encode(F.e4m3_value(codes)), codes.astype(np.uint8))


def _brute_nearest(x_abs, grid, window_ok):
    """Index of the grid value nearest x_abs; ties to the even index (lower bit 0)."""
    d = np.abs(x_abs[:, None] - grid[None, :])
    dmin = d.min(axis=1, keepdims=True)
    is_min = d == dmin
    idx = np.arange(len(grid))[None, :]
    even_min = is_min & ((idx & 1) == 0)
    # ties between two neighbours: exactly one of them is even
    best = np.where(even_min.any(axis=1), np.argmax(even_min, axis=1), np.argmax(is_min, axis=1))
    assert np.all(is_min.sum(axis=1)[window_ok] <= 2)
    return best


def test_e4m3_encode_vs_brute_force_all_bf16():
    bits = _all_finite_bf16()
    x = F.bf16_value(bits)
    ax = np.abs(x)
    grid = F.E4M3_NONNEG
    # Exact window: |x| in [2^-14, 2^12] makes every |x - v| exact in float64.
    win = (ax >= 2.0 ** -14) & (ax <= 2.0 ** 12)
    got = F.e4m3_encode(x)
    brute = _brute_nearest(ax[win], grid, np.ones(win.sum(), bool))
    assert np.array_equal(got[win] & 0x7F, brute.astype(np.uint8))
    # Outside the window the answer is forced: tiny -> 0, huge -> 448 (saturation).
    assert np.all((got[~win & (ax < 1)] & 0x7F) == 0)
    assert np.all((got[~win & (ax > 1)] & 0x7F) == 0x7E)
    assert np.array_equal((got & 0x80) != 0, np.signbit(x))


def test_e4m3_scale_rule_vs_brute_force_all_bf16_amax():
    # Scale = E4M3 value nearest amax/6.  Brute force on |amax - 6 v| (exact in the window).
    bits = _all_finite_bf16()
    amax = np.unique(np.abs(F.bf16_value(bits)))
    got = F.e4m3_encode_ratio(amax, 6.0)
    win = (amax >= 2.0 ** -14) & (amax <= 2.0 ** 13)
    brute = _brute_nearest(amax[win], 6.0 * F.E4M3_NONNEG, np.ones(win.sum(), bool))
    assert np.array_equal(got[win], brute.astype(np.uint8))
    assert np.all(got[~win & (amax < 1)] == 0)
    assert np.all(got[~win & (amax > 1)] == 0x7E)
    # Exact-rational spot check against Fraction arithmetic around every tie of the grid.
    for c in range(126):
        mid = (Fraction(F.E4M3_NONNEG[c]) + Fraction(F.E4M3_NONNEG[c + 1])) / 2
        tie = float(mid * 6)
        want = c if c % 2 == 0 else c + 1
        assert int(F.e4m3_encode_ratio(np.array([tie]), 6.0)[0]) == want


def test_e2m1_encode_vs_brute_force_all_bf16_all_scales():
    x = F.bf16_value(_all_finite_bf16())
    ax = np.abs(x)
    for sc in range(127):
        s = float(F.E4M3_NONNEG[sc])
        got = F.e2m1_encode(x, s)
        assert np.array_equal((got & 8) != 0, np.signbit(x))
        mag = got & 7
        if s == 0.0:
            assert np.all(mag == 0)
            continue
        # Exact window |x|/s in [1/16, 16]: all |x| - v*s exact in float64.
        win = (ax >= s / 16) & (ax <= s * 16)
        brute = _brute_nearest(ax[win], F.E2M1_MAGNITUDES * s, np.ones(win.sum(), bool))
        assert np.array_equal(mag[win], brute.astype(np.uint8)), sc
        assert np.all(mag[~win & (ax < s)] == 0)
        assert np.all(mag[~win & (ax > s)] == 7)


def test_bf16_value_exact():
    assert F.bf16_value(np.array([0x3F80]))[0] == 1.0
    assert F.bf16_value(np.array([0xC040]))[0] == -3.0
    assert F.bf16_value(np.array([0x0001]))[0] == 2.0 ** -133
    assert F.bf16_value(np.array([0x7F7F]))[0] == float(Fraction(255, 128) * 2 ** 127)


@pytest.mark.parametrize("seed", range(4))
def test_fma_f32_single_rounding_vs_fractions(seed):
    rng = np.random.default_rng(seed)
    # bf16-valued a, b (16-bit products) and arbitrary fp32 c, including cancellations.
    def rand_bf16(n):
        sign = rng.integers(0, 2, n) << 15
        exp = rng.integers(100, 155, n) << 7
        man = rng.integers(0, 128, n)
        return F.bf16_value((sign | exp | man).astype(np.uint16))
    a = rand_bf16(4000)
    b = rand_bf16(4000)
    c = rng.standard_normal(4000).astype(np.float32) * np.float32(2.0) ** rng.integers(-30, 30, 4000)
    c[::7] = -(a[::7] * b[::7]).astype(np.float32)   # near-cancellation
    got = F.fma_f32(a, b, c)
    for i in range(0, 4000, 13):
        exact = Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i]))
        # round exact to fp32 by exhaustive neighbour check
        g = np.float32(got[i])
        lo = np.nextafter(g, np.float32(-np.inf))
        hi = np.nextafter(g, np.float32(np.inf))
        dg = abs(Fraction(float(g)) - exact)
        assert dg <= abs(Fraction(float(lo)) - exact)
        assert dg <= abs(Fraction(float(hi)) - exact)
