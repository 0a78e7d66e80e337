"""Pins of the oracle's index score (sum over indexer heads of q_h . k_h in fp32).

The pages give no score values; the fp32 rounding sequence is a reading.  These
tests pin the oracle against the exact dot product: bit-exact where every
partial sum is exactly representable, and within the fp32 error bound of the
fixed evaluation order otherwise.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import csa2 as O
from oracle import formats as F


def _exact_scores(q, k):
    return np.einsum("hd,nhd->n", q.astype(np.float64), k.astype(np.float64))


@pytest.mark.parametrize("heads", [4, 8])
def test_integer_inputs_exact(heads):
    # Small integers: products and every partial sum are exact in fp32, so the
    # result must equal the exact dot product whatever the summation order.
    rng = np.random.default_rng(heads)
    q = rng.integers(-8, 9, (heads, 64)).astype(np.float32)
    k = rng.integers(-16, 17, (300, heads, 64)).astype(np.float32)
    got = O.index_scores(q, k)
    want = np.einsum("hd,nhd->n", q.astype(np.int64), k.astype(np.int64))
    assert np.array_equal(got.astype(np.int64), want)


def test_fp8_grid_values_exact_when_small():
    # E4M3 values times E4M3 values are multiples of 2^-18; with few nonzeros the sums are exact.
    rng = np.random.default_rng(5)
    codes_q = rng.integers(0, 0x50, (8, 64))
    codes_k = rng.integers(0, 0x50, (64, 8, 64))
    q = F.e4m3_value(codes_q).astype(np.float32)
    k = F.e4m3_value(codes_k).astype(np.float32)
    q[:, 2:] = 0
    got = O.index_scores(q, k).astype(np.float64)
    want = _exact_scores(q, k)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("heads,dtype", [(4, "bf16"), (8, "fp8"), (8, "bf16")])
def test_error_bound_vs_exact(heads, dtype):
    rng = np.random.default_rng(heads)
    qv = rng.standard_normal((heads, 64)) * np.exp(rng.standard_normal((heads, 64)))
    kv = rng.standard_normal((2000, heads, 64)) * 3
    q = F.bf16_value(np.frombuffer(qv.astype(np.float32).tobytes(), np.uint32).reshape(qv.shape) >> 16)
    if dtype == "fp8":
        k = F.e4m3_value(F.e4m3_encode(kv))
    else:
        k = F.bf16_value(np.frombuffer(kv.astype(np.float32).tobytes(), np.uint32).reshape(kv.shape) >> 16)
    q = q.astype(np.float32)
    k = k.astype(np.float32)
    got = O.index_scores(q, k).astype(np.float64)
    exact = _exact_scores(q, k)          # fp64; its own error is ~2^-53 relative
    mag = np.einsum("hd,nhd->n", np.abs(q).astype(np.float64), np.abs(k).astype(np.float64))
    depth = 16 + 2 + 3                   # longest chain of roundings in the fixed order
    bound = depth * 2.0 ** -24 * mag * (1 + 1e-6)
    assert np.all(np.abs(got - exact) <= bound)
    # and the fixed order actually rounds (not computed in higher precision)
    assert np.all(got == got.astype(np.float32))


def test_one_hot_query_selects_channel_sum():
    rng = np.random.default_rng(9)
    k = F.e4m3_value(F.e4m3_encode(rng.standard_normal((100, 8, 64)))).astype(np.float32)
    q = np.zeros((8, 64), np.float32)
    q[:, 17] = 1.0
    got = O.index_scores(q, k)
    # eight terms in a balanced fp32 tree; fp8 values sum exactly in fp32 here (|v| <= 448, 2^-9 grid)
    want = k[:, :, 17].astype(np.float64).sum(axis=1)
    assert np.array_equal(got.astype(np.float64), want)


def test_sign_and_linearity_exact_cases():
    rng = np.random.default_rng(3)
    q = rng.integers(-4, 5, (8, 64)).astype(np.float32)
    k = rng.integers(-4, 5, (50, 8, 64)).astype(np.float32)
    assert np.array_equal(O.index_scores(-q, k), -O.index_scores(q, k))
    assert np.array_equal(O.index_scores(2 * q, k), 2 * O.index_scores(q, k))


def test_head_order_is_balanced_tree_on_cancellation():
    # The sum over heads is a balanced fp32 tree: with head sums (2^24, 1, -2^24, 1, 0...)
    # the tree gives round(2^24 + 1) + (-2^24 + 1) = 2^24 - 2^24 + 1 = 1, not 2.
    # Check only against exact rational evaluation of that tree, not against the code.
    heads = [2.0 ** 24, 1.0, -(2.0 ** 24), 1.0, 0.0, 0.0, 0.0, 0.0]
    q = np.zeros((8, 64), np.float32)
    q[:, 0] = 1.0
    k = np.zeros((1, 8, 64), np.float32)
    k[0, :, 0] = heads

    def rnd(x):   # exact rational -> nearest fp32, ties to even
        return Fraction(float(np.float32(float(x))))
    a01 = rnd(Fraction(heads[0]) + Fraction(heads[1]))     # 2^24 + 1 -> 2^24 (tie to even)
    a23 = rnd(Fraction(heads[2]) + Fraction(heads[3]))     # -2^24 + 1 -> -2^24 + 1 (exact)
    want = rnd(a01 + a23)
    assert Fraction(float(O.index_scores(q, k)[0])) == want
    assert want == 1   # the unrounded sum would be 2


def test_exact_scores_equal_rational_sums_for_e4m3():
    # The claim of index_scores_exact: for E4M3 x E4M3 the float64 sum is the
    # exact rational sum, whatever order BLAS takes.  Checked against Fractions
    # over the full E4M3 range (subnormals up to 448, both signs).
    rng = np.random.default_rng(11)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    for heads in (4, 8):
        q = F.e4m3_value(rng.choice(finite, (heads, 64))).astype(np.float32)
        k = F.e4m3_value(rng.choice(finite, (40, heads, 64))).astype(np.float32)
        got, mag = O.index_scores_exact(q, k)
        for n in range(len(k)):
            want = sum(Fraction(float(a)) * Fraction(float(b))
                       for a, b in zip(q.reshape(-1), k[n].reshape(-1)))
            assert Fraction(float(got[n])) == want
            assert Fraction(float(mag[n])) == sum(abs(Fraction(float(a)) * Fraction(float(b)))
                                                  for a, b in zip(q.reshape(-1), k[n].reshape(-1)))


def test_canonical_scores_within_rounding_bound_of_exact():
    # The fp32 canonical score sits within 512 * 2^-24 * sum|q||k| of the exact
    # one: the bound the relaxed index-set rule leans on.
    rng = np.random.default_rng(12)
    q = F.e4m3_value(F.e4m3_encode(rng.standard_normal((8, 64)) * 4)).astype(np.float32)
    k = F.e4m3_value(F.e4m3_encode(rng.standard_normal((3000, 8, 64)) * 2)).astype(np.float32)
    exact, mag = O.index_scores_exact(q, k)
    got = O.index_scores(q, k).astype(np.float64)
    assert np.all(np.abs(got - exact) <= 512 * 2.0 ** -24 * mag)
    assert np.any(got != exact)   # the rounding is really there
