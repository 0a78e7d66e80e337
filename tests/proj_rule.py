"""Per-element acceptance rule for the projection's cache bytes on inputs whose
fp32 sums are not exact (test infrastructure).

The library sums the bf16 products of y = W x in fp32 in the matrix cores'
order and rounds y once to bf16; the oracle takes the exact sum.  The products
are exact (8-bit by 8-bit significands).  If no product passes through more
than `depth` fp32 roundings on its way to y, the library's fp32 value lies
within delta = depth * 2^-24 * sum|x||w| of the exact one (first order; the
factor 1 + 1e-4 covers the rest), and its bf16 value lies between
rne(y - delta) and rne(y + delta).  The library's kernel splits the
contraction over four waves, each adding one 32-product matrix-core step at a
time to its accumulator (d_model / 128 steps; at most 32 roundings inside a
step, whatever its internal order), and adds the four partial sums in three
steps: proj_depth(d_model) = 32 + d_model / 128 + 3.  Every stored byte must
be the encoding of some value in that range:

* an index key (bf16 bits, or the E4M3 code of the bf16 value) lies between
  the encodings of the range's ends, with a sign that some value of the range
  has;
* the E4M3 scale of a 16-channel K or V block lies between the scales of the
  smallest and the largest block maximum the ranges allow;
* every E2M1 code of the block, under the stored scale, lies between the
  codes of its range's ends, with a possible sign.

Where the range holds one bf16 value (most elements) the byte is fixed: a
wrong channel, a wrong scale or a swapped code fails.  The encodings are
monotone in the value, so checking the ends covers the whole range.
"""
from __future__ import annotations

import numpy as np

from oracle import csa2 as O
from oracle import formats as F


def _signs_allowed(lo, hi):
    """(negative sign possible, positive sign possible) for values in [lo, hi]."""
    neg = (lo < 0) | ((lo == 0) & np.signbit(lo))
    pos = (hi > 0) | ((hi == 0) & ~np.signbit(hi))
    return neg, pos


def _sign_ok(code_sign, lo, hi):
    neg, pos = _signs_allowed(lo, hi)
    return np.where(code_sign, neg, pos)


def proj_depth(d_model: int) -> int:
    """fp32 roundings a product passes through in the library's projection."""
    return 32 + (d_model + 127) // 128 + 3


def value_ranges(x_bits, w_bits, depth=None):
    """bf16 values lo, hi [n, channels] (float64) bracketing the library's y."""
    x = F.bf16_value(x_bits)
    w = F.bf16_value(w_bits)
    d = x.shape[1]
    depth = proj_depth(d) if depth is None else depth
    y = x @ w.T
    mag = np.abs(x) @ np.abs(w).T
    delta = depth * 2.0 ** -24 * mag * (1 + 1e-4) + 2.0 ** -140
    lo = F.bf16_value(O.bf16_round_bits(y - delta))
    hi = F.bf16_value(O.bf16_round_bits(y + delta))
    return lo, hi


def check_projection_bytes(x_bits, w_bits, heads, idx_dtype, codes, scales, idx, depth=None):
    """codes [n, 128], scales [n, 16], idx [n, heads, 64] (uint8 E4M3 or uint16
    bf16): the cache bytes of the n projected rows.  Raises AssertionError
    naming the first offending element; returns the number of elements whose
    range holds more than one bf16 value."""
    lo, hi = value_ranges(x_bits, w_bits, depth)
    n = lo.shape[0]
    ambiguous = int(np.sum(lo != hi))
    # index keys
    ilo = lo[:, 256:].reshape(n, heads, 64)
    ihi = hi[:, 256:].reshape(n, heads, 64)
    if idx_dtype == "fp8":
        g = F.e4m3_value(idx)
        vlo = F.e4m3_value(F.e4m3_encode(ilo))
        vhi = F.e4m3_value(F.e4m3_encode(ihi))
        sign = (np.asarray(idx) & 0x80) != 0
    else:
        g = F.bf16_value(idx)
        vlo, vhi = ilo, ihi
        sign = (np.asarray(idx, np.uint16) & 0x8000) != 0
    ok = (vlo <= g) & (g <= vhi) & _sign_ok(sign, ilo, ihi)
    if not ok.all():
        t, h, c = np.argwhere(~ok)[0]
        raise AssertionError(f"index key of row {t} head {h} channel {c}: stored {g[t, h, c]}, "
                             f"range [{ilo[t, h, c]}, {ihi[t, h, c]}]")
    # K and V: scale and codes per 16-channel block
    cd = O.unpack_nibbles(np.asarray(codes, np.uint8))          # [n, 256] codes, K then V
    sc = np.asarray(scales, np.uint8)                            # [n, 16]
    blo = lo[:, :256].reshape(n, 16, 16)
    bhi = hi[:, :256].reshape(n, 16, 16)
    amag_lo = np.where((blo <= 0) & (bhi >= 0), 0.0, np.minimum(np.abs(blo), np.abs(bhi)))
    amag_hi = np.maximum(np.abs(blo), np.abs(bhi))
    amax_lo = amag_lo.max(axis=2)
    amax_hi = amag_hi.max(axis=2)
    s_lo = F.e4m3_value(F.e4m3_encode_ratio(amax_lo, 6.0))
    s_hi = F.e4m3_value(F.e4m3_encode_ratio(amax_hi, 6.0))
    s = F.e4m3_value(sc)
    ok = (s_lo <= s) & (s <= s_hi)
    if not ok.all():
        t, b = np.argwhere(~ok)[0]
        raise AssertionError(f"scale of row {t} block {b}: stored {s[t, b]}, "
                             f"range [{s_lo[t, b]}, {s_hi[t, b]}]")
    g = F.e2m1_value(cd).reshape(n, 16, 16)
    sb = s[:, :, None]
    clo = F.e2m1_value(F.e2m1_encode(blo, sb))
    chi = F.e2m1_value(F.e2m1_encode(bhi, sb))
    sign = ((cd & 8) != 0).reshape(n, 16, 16)
    ok = (clo <= g) & (g <= chi) & _sign_ok(sign, blo, bhi)
    if not ok.all():
        t, b, c = np.argwhere(~ok)[0]
        raise AssertionError(f"code of row {t} channel {16 * b + c}: stored {g[t, b, c]}, "
                             f"range [{clo[t, b, c]}, {chi[t, b, c]}] at scale {s[t, b]}")
    return ambiguous
