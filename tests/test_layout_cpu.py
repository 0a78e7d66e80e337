"""The tiled index-key layout stated in include/csa2.h, written out element by
element, agrees with the vectorized un-tiling the GPU tests use."""
import numpy as np
import pytest

from gpu_util import untile_idx


@pytest.mark.parametrize("heads,esz", [(8, 1), (4, 1), (8, 2), (4, 2)])
def test_untile_matches_header_formula(heads, esz):
    cap, batch = 32, 2
    rng = np.random.default_rng(heads * esz)
    dt = np.uint8 if esz == 1 else np.uint16
    logical = rng.integers(0, 1 << (8 * esz), (batch, cap, heads, 64)).astype(dt)
    raw = np.zeros(batch * cap * heads * 64 * esz, np.uint8)
    t = 64 // heads
    for s in range(batch):
        for p in range(cap):
            for h in range(heads):
                for c in range(64):
                    elem = logical[s, p, h, c].tobytes()
                    base = (s * cap * heads * 64 * esz + (p // t) * (64 * 64 * esz)
                            + ((c * esz) // 16) * 1024 + ((p % t) * heads + h) * 16 + (c * esz) % 16)
                    raw[base:base + esz] = np.frombuffer(elem, np.uint8)
    got = untile_idx(raw.reshape(batch, -1), heads, dt)
    assert np.array_equal(got, logical)
