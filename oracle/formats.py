"""Number formats of the FP4 KV cache: E2M1 values, E4M3 scales, bf16 inputs.

Source: the model card "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
Compression", Introduction, CSA2 paragraph (main KV stored in FP4, E2M1 values
with one E4M3 scale per 16 channels); the thinkplainai post's "Key specs" table
(global KV cache in FP4 E2M1).  The pages name the formats only.  Readings:

* E2M1 is the OCP microscaling element format: code bits ``s e e m``,
  magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, bit 3 the sign.
* E4M3 is OCP E4M3FN: bias 7, no infinities, 0x7F/0xFF are NaN, largest
  finite 448, subnormals m * 2^-9.
* Rounding to either format is to nearest, ties to the even code (code LSB 0),
  saturating at the largest finite magnitude.

All arithmetic here is exact: every comparison is between values that are
exactly representable in float64.
"""
from __future__ import annotations

import numpy as np

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
# Midpoints between consecutive E2M1 magnitudes.
_E2M1_MID = (E2M1_MAGNITUDES[:-1] + E2M1_MAGNITUDES[1:]) / 2.0


def e2m1_value(code) -> np.ndarray:
    """Value of 4-bit E2M1 codes (bit 3 sign; code 8 is -0.0)."""
    code = np.asarray(code, dtype=np.int64)
    mag = E2M1_MAGNITUDES[code & 7]
    return np.where((code & 8) != 0, -mag, mag)


def e4m3_value(code) -> np.ndarray:
    """Value of 8-bit OCP E4M3FN codes; 0x7F and 0xFF decode to NaN."""
    code = np.asarray(code, dtype=np.int64)
    e = (code >> 3) & 15
    m = (code & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((code & 0x7F) == 0x7F, np.nan, mag)
    return np.where((code & 0x80) != 0, -mag, mag)


# The 127 non-negative finite E4M3 values (codes 0..126) and their 126 midpoints.
E4M3_NONNEG = e4m3_value(np.arange(127))
_E4M3_MID = (E4M3_NONNEG[:-1] + E4M3_NONNEG[1:]) / 2.0


def _rne_index(x, bounds):
    """Index of the grid value nearest to x, for sorted midpoints `bounds`.

    Counts the midpoints strictly below x; a value exactly on a midpoint goes to
    the even neighbour (index i+1 when i+1 is even).  Values above the last
    midpoint land on the last grid value (saturation).
    """
    idx = np.searchsorted(bounds, x, side="left")
    on_mid = np.zeros(np.shape(x), dtype=bool)
    inside = idx < len(bounds)
    on_mid[inside] = bounds[idx[inside]] == x[inside]
    up = on_mid & (((idx + 1) & 1) == 0)
    return idx + up


def e4m3_encode_ratio(num, den: float) -> np.ndarray:
    """E4M3 code (0..126) of the non-negative real num/den, RNE, saturating at 448.

    Decided by comparing num against den * midpoint, which is exact in float64
    for den in {1, 6} (a midpoint has at most 5 significant bits), so no
    division is rounded.
    """
    num = np.asarray(num, dtype=np.float64)
    flat = num.reshape(-1)
    if np.any(flat < 0) or np.any(~np.isfinite(flat)):
        raise ValueError("e4m3_encode_ratio expects finite non-negative values")
    return _rne_index(flat, _E4M3_MID * float(den)).reshape(num.shape).astype(np.uint8)


def e4m3_encode(x) -> np.ndarray:
    """OCP E4M3FN code of finite real values x (RNE, saturating), sign kept (-0 -> 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    code = e4m3_encode_ratio(np.abs(x), 1.0)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def e2m1_encode(x, s) -> np.ndarray:
    """E2M1 code of element x under decoded scale s (broadcast), sign kept.

    The magnitude code is the E2M1 value nearest |x|/s (RNE, saturating at 6),
    decided by comparing |x| with midpoint * s, both exact in float64.  A zero
    scale gives magnitude code 0 (reading: the block dequantizes to zero).
    """
    x = np.asarray(x, dtype=np.float64)
    s = np.broadcast_to(np.asarray(s, dtype=np.float64), x.shape)
    ax = np.abs(x)
    mag = np.zeros(x.shape, dtype=np.int64)
    for i, m in enumerate(_E2M1_MID):
        t = m * s                     # exact: <= 3 significant bits times <= 4
        up = (ax > t) | ((ax == t) & (((i + 1) & 1) == 0))
        mag += up
    mag = np.where(s == 0.0, 0, mag)
    return (mag | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def bf16_value(bits) -> np.ndarray:
    """Value of bfloat16 bit patterns as float64 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32).astype(np.float64)


def fma_f32(a, b, c) -> np.ndarray:
    """fp32 fused multiply-add: round_to_f32(a*b + c) with a single rounding.

    a, b, c are float32 values.  a*b is exact in float64 (48 bits).  When a*b
    has at most 29 significant bits (true for every product in this path:
    bf16*bf16 has 16, bf16*e4m3 12, e4m3*e4m3 8), a*b + c is either exact in
    float64 or the smaller addend lies below half an fp32 ulp of the larger, so
    rounding the float64 sum to float32 gives the singly-rounded result.
    """
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    b = np.asarray(b, dtype=np.float32).astype(np.float64)
    c = np.asarray(c, dtype=np.float32).astype(np.float64)
    return (a * b + c).astype(np.float32)
