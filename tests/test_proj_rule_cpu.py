"""The per-element rule that judges the projection's cache bytes on inputs
whose fp32 sums are not exact (tests/proj_rule.py), checked on the CPU: the
oracle's own bytes pass, bytes of a projection perturbed within the fp32
error bound pass, and planted mistakes fail -- one corrupted index-key channel,
one FP4 code off by one step, one scale off by one code, a sign flipped."""
import numpy as np
import pytest

import synth
from oracle import csa2 as O
from oracle import formats as F
from proj_rule import check_projection_bytes, value_ranges


def _case(heads=8, dtype="fp8", n=40, d=2048, seed=3):
    rng = np.random.default_rng(seed)
    ch = 256 + heads * 64
    x = synth.f32_to_bf16_bits(rng.standard_normal((n, d)).astype(np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((ch, d)) / np.sqrt(d)).astype(np.float32))
    return x, w


def _bytes_of(y_bits, heads, dtype):
    n = y_bits.shape[0]
    oc = O.OracleCache(1, ((n + 15) // 16) * 16, idx_heads=heads, idx_k_dtype=dtype)
    oc.append(y_bits[:, :128], y_bits[:, 128:256], y_bits[:, 256:].reshape(n, heads, 64),
              np.zeros(n, int), np.arange(n))
    return oc.kv_codes[0, :n].copy(), oc.kv_scales[0, :n].copy(), oc.idx_k[0, :n].copy()


@pytest.mark.parametrize("heads,dtype", [(8, "fp8"), (4, "bf16")])
def test_oracle_bytes_pass(heads, dtype):
    x, w = _case(heads, dtype)
    y = O.project_rows(x, w)
    amb = check_projection_bytes(x, w, heads, dtype, *_bytes_of(y, heads, dtype))
    assert amb > 0      # the random case really has elements next to a rounding boundary


@pytest.mark.parametrize("heads,dtype", [(8, "fp8"), (4, "bf16")])
def test_perturbed_within_the_bound_passes(heads, dtype):
    # any value in [y - delta, y + delta] rounds to an admissible byte: take
    # both ends of every element's range (a per-element choice of the library)
    x, w = _case(heads, dtype, seed=4)
    lo, hi = value_ranges(x, w)
    rng = np.random.default_rng(0)
    pick = np.where(rng.random(lo.shape) < 0.5, lo, hi)
    y = O.bf16_round_bits(pick)
    check_projection_bytes(x, w, heads, dtype, *_bytes_of(y, heads, dtype))


def test_planted_mistakes_fail():
    heads, dtype = 8, "fp8"
    x, w = _case(heads, dtype, seed=5)
    y = O.project_rows(x, w)
    codes, scales, idx = _bytes_of(y, heads, dtype)
    lo, hi = value_ranges(x, w)
    fixed = lo == hi
    # one index-key channel of one row replaced by its neighbour channel's code
    bad = idx.copy()
    t, h, c = [int(v) for v in np.argwhere((idx[:, :, :-1] != idx[:, :, 1:])
                                           & fixed[:, 256:].reshape(-1, heads, 64)[:, :, :-1])[0]]
    bad[t, h, c] = idx[t, h, c + 1]
    with pytest.raises(AssertionError, match="index key"):
        check_projection_bytes(x, w, heads, dtype, codes, scales, bad)
    # a sign flipped on a nonzero key
    bad = idx.copy()
    t, h, c = [int(v) for v in np.argwhere((idx & 0x7F) != 0)[0]]
    bad[t, h, c] ^= 0x80
    with pytest.raises(AssertionError, match="index key"):
        check_projection_bytes(x, w, heads, dtype, codes, scales, bad)
    # one scale one code up
    bad = scales.copy()
    bad[3, 5] += 1
    with pytest.raises(AssertionError):
        check_projection_bytes(x, w, heads, dtype, codes, bad, idx)
    # one FP4 magnitude one step up (1 -> 1.5) where the value is fixed
    un = O.unpack_nibbles(codes)
    cand = np.argwhere(((un & 7) == 2) & fixed[:, :256])
    t, c = [int(v) for v in cand[0]]
    un2 = un.copy()
    un2[t, c] += 1
    with pytest.raises(AssertionError, match="code of row"):
        check_projection_bytes(x, w, heads, dtype, O.pack_nibbles(un2), scales, idx)
    # a whole V channel taken from another token
    un3 = un.copy()
    un3[:, 200] = np.roll(un[:, 200], 1)
    with pytest.raises(AssertionError):
        check_projection_bytes(x, w, heads, dtype, O.pack_nibbles(un3), scales, idx)
