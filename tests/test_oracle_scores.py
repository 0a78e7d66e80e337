"""Pins of the oracle's index score (sum over indexer heads of q_h . k_h in fp32).

The pages give no score values; the fp32 rounding sequence is a reading: per
head one chain of fused multiply-adds over the channels in increasing order,
then the head sums added left to right.  These tests pin the oracle against the
exact dot product (bit-exact where every partial sum is representable, within
the fp32 error bound otherwise) and pin the order itself with cancelling inputs
whose left-to-right fp32 result is derived by hand and by exact rational
evaluation, and differs from the exact sum and from the other plausible orders.
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
    depth = 64 + 7                       # roundings: a 64-step chain per head, 7 head additions
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
    # eight terms summed in fp32; fp8 values sum exactly in fp32 here (|v| <= 448, 2^-9 grid)
    want = k[:, :, 17].astype(np.float64).sum(axis=1)
    assert np.array_equal(got.astype(np.float64), want)


def test_sign_and_linearity_exact_cases():
    rng = np.random.default_rng(3)
    q = rng.integers(-4, 5, (8, 64)).astype(np.float32)
    k = rng.integers(-4, 5, (50, 8, 64)).astype(np.float32)
    assert np.array_equal(O.index_scores(-q, k), -O.index_scores(q, k))
    assert np.array_equal(O.index_scores(2 * q, k), 2 * O.index_scores(q, k))


def _rnd(x):
    """Exact rational -> the nearest fp32 value (ties to even), as a Fraction.

    Rounded once, straight from the rational (no float64 step in between):
    24 significant bits, spacing 2^(e-23) for 2^e <= |x| < 2^(e+1), subnormal
    spacing 2^-149."""
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (max(e, -126) - 23)
    r = round(a / ulp) * ulp          # Fraction.__round__: nearest integer, ties to even
    return r if x > 0 else -r


def _left_to_right(q, k):
    """The reading's order evaluated in exact rationals with one fp32 rounding
    per step: per head fma(q, k, acc) over channels 0..D-1, then the head sums
    from head 0 up.  q [H, D], k [H, D] float32."""
    heads = []
    for h in range(q.shape[0]):
        acc = Fraction(0)
        for c in range(q.shape[1]):
            acc = _rnd(Fraction(float(q[h, c])) * Fraction(float(k[h, c])) + acc)
        heads.append(acc)
    s = heads[0]
    for a in heads[1:]:
        s = _rnd(s + a)
    return s


@pytest.mark.parametrize("heads", [4, 8])
def test_channel_order_is_one_chain_from_channel_0(heads):
    # Terms 1, 2^24, 1, -2^24 at channels 0, 16, 32, 48 of head 0 (q = 1 there).
    # Left to right in fp32: 1 -> 1 + 2^24 is a tie between 2^24 and 2^24 + 2,
    # kept at the even 2^24 -> + 1 ties again, 2^24 -> - 2^24 = 0.  The exact sum
    # is 2; 16-channel block sums added (b0+b1)+(b2+b3) give 1; the reversed
    # chain gives -2^24 + 1 (exact) + 1 + 2^24 = 2.
    q = np.zeros((heads, 64), np.float32)
    k = np.zeros((1, heads, 64), np.float32)
    for c, v in zip((0, 16, 32, 48), (1.0, 2.0 ** 24, 1.0, -(2.0 ** 24))):
        q[0, c] = 1.0
        k[0, 0, c] = v
    got = Fraction(float(O.index_scores(q, k)[0]))
    assert got == 0
    assert got == _left_to_right(q, k[0])
    # neighbouring channels: the same terms at channels 5, 6, 7, 8
    q2 = np.zeros_like(q)
    k2 = np.zeros_like(k)
    for c, v in zip((5, 6, 7, 8), (1.0, 2.0 ** 24, 1.0, -(2.0 ** 24))):
        q2[0, c] = 1.0
        k2[0, 0, c] = v
    assert O.index_scores(q2, k2)[0] == 0.0


@pytest.mark.parametrize("heads", [4, 8])
def test_head_order_is_left_to_right(heads):
    # Head sums 2^24, 1, 1, -2^24 (heads 0..3; the rest 0).  Left to right:
    # 2^24 + 1 -> 2^24 (tie to even), + 1 -> 2^24, - 2^24 -> 0.  The exact sum
    # is 2; a balanced tree gives (2^24 + 1 -> 2^24) + (1 - 2^24, exact) = 1.
    q = np.zeros((heads, 64), np.float32)
    q[:, 0] = 1.0
    k = np.zeros((1, heads, 64), np.float32)
    k[0, :4, 0] = [2.0 ** 24, 1.0, 1.0, -(2.0 ** 24)]
    got = Fraction(float(O.index_scores(q, k)[0]))
    assert got == 0
    assert got == _left_to_right(q, k[0])


def test_heads_summed_after_their_chains():
    # Summing per channel over heads first would mix the heads' terms: head 0
    # holds 2^24 at channel 0 and -2^24 at channel 1, head 1 holds 1 at channel 0
    # and 1 at channel 1.  Per head: acc_0 = 0 exactly, acc_1 = 2, total 2.
    # Channel-outer order: 2^24 + 1 -> 2^24, then + (-2^24) -> 0, + 1 -> 1.
    q = np.ones((4, 64), np.float32)
    k = np.zeros((1, 4, 64), np.float32)
    k[0, 0, 0], k[0, 0, 1] = 2.0 ** 24, -(2.0 ** 24)
    k[0, 1, 0], k[0, 1, 1] = 1.0, 1.0
    got = Fraction(float(O.index_scores(q, k)[0]))
    assert got == 2
    assert got == _left_to_right(q, k[0])


def test_random_cancellation_matches_rational_left_to_right():
    # Mixed magnitudes (2^-20 .. 2^20, both signs) on the bf16 and E4M3 grids,
    # so nearly every step rounds; the oracle must equal the exact rational
    # evaluation of the stated order with one rounding per step, bit for bit.
    rng = np.random.default_rng(21)
    for heads in (4, 8):
        mant = rng.integers(1, 256, (6, heads, 64)) * rng.choice([-1, 1], (6, heads, 64))
        k = (mant * np.exp2(rng.integers(-20, 20, (6, heads, 64)))).astype(np.float32)
        q = F.e4m3_value(rng.integers(0, 0x7E, (heads, 64))).astype(np.float32)
        got = O.index_scores(q, k)
        for n in range(len(k)):
            assert Fraction(float(got[n])) == _left_to_right(q, k[n])


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
