"""GPU parity of csa2_kv_append: packed FP4 bytes, E4M3 scales and index keys
bit-exact against the oracle, including an exhaustive sweep of every finite
bf16 element under every reachable scale."""
import numpy as np
import pytest
import torch

import synth
from oracle import csa2 as O
from oracle import formats as F
from gpu_util import DEV, announce, dev_i32, dev_u16, filled_caches, host, lib, untile_idx

pytestmark = pytest.mark.gpu


def _finite_bf16_bits():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return bits[((bits >> 7) & 0xFF) != 0xFF]


@pytest.mark.parametrize("idx_dtype,heads", [("fp8", 8), ("bf16", 4), ("fp8", 4), ("bf16", 8)])
def test_append_seeded_rows_bit_exact(idx_dtype, heads):
    announce(f"append seeded rows idx={idx_dtype} heads={heads}")
    wl = synth.workload("tiny_4k", context=1008, batch=2, idx_heads=heads, idx_k_dtype=idx_dtype)
    gc, oc, _ = filled_caches(wl)
    assert np.array_equal(host(gc.kv_codes), oc.kv_codes)
    assert np.array_equal(host(gc.kv_scales), oc.kv_scales)
    assert np.array_equal(untile_idx(host(gc.idx_k), heads, oc.idx_k.dtype), oc.idx_k)


def _sweep_rows():
    """Blocks [amax, x1..x15] for every scale code: amax is the largest bf16
    value mapping to that scale and x runs over every finite bf16 value with
    |x| <= amax (both signs), so every reachable (element, scale) pair occurs."""
    bits = _finite_bf16_bits()
    vals = F.bf16_value(bits)
    pos_bits = bits[(vals > 0)]
    pos_vals = F.bf16_value(pos_bits)
    sc_of = F.e4m3_encode_ratio(pos_vals, 6.0)
    order = np.argsort(np.abs(vals), kind="stable")
    sorted_abs = np.abs(vals)[order]
    blocks = []
    for sc in range(127):
        cand = pos_bits[sc_of == sc]
        if len(cand) == 0:
            continue
        a_bits = cand[np.argmax(F.bf16_value(cand))]
        a = F.bf16_value(np.array([a_bits]))[0]
        xs = bits[order[:np.searchsorted(sorted_abs, a, side="right")]]
        nblk = (len(xs) + 14) // 15
        xs = np.concatenate([xs, np.zeros(nblk * 15 - len(xs), np.uint16)])
        blk = np.empty((nblk, 16), np.uint16)
        blk[:, 0] = a_bits
        blk[:, 1:] = xs.reshape(nblk, 15)
        blocks.append(blk)
    blocks = np.concatenate(blocks)
    nrow = (len(blocks) + 15) // 16
    nrow = (nrow + 15) // 16 * 16          # capacity must be a multiple of 16
    pad = np.zeros((nrow * 16 - len(blocks), 16), np.uint16)
    blocks = np.concatenate([blocks, pad]).reshape(nrow, 16, 16)
    k = blocks[:, :8].reshape(nrow, 128)
    v = blocks[:, 8:].reshape(nrow, 128)
    return k, v


def test_append_exhaustive_element_and_scale_sweep():
    k, v = _sweep_rows()
    n = k.shape[0]
    announce(f"append exhaustive sweep rows={n}")
    m = lib()
    # index keys: every finite bf16 value, 512 per row, cast to E4M3
    ib = _finite_bf16_bits()
    ik = np.zeros((n, 8, 64), np.uint16).reshape(n, -1)
    flat = ik.reshape(-1)
    flat[:len(ib)] = ib
    ik = flat.reshape(n, 8, 64)
    gc = m.Cache(1, n, idx_heads=8, idx_k_dtype="fp8")
    oc = O.OracleCache(1, n, idx_heads=8, idx_k_dtype="fp8")
    seq = np.zeros(n, np.int32)
    pos = np.arange(n, dtype=np.int32)[::-1].copy()      # scattered destination order
    m.csa2_kv_append(gc, dev_u16(k), dev_u16(v), dev_u16(ik), dev_i32(seq), dev_i32(pos))
    oc.append(k, v, ik, seq, pos)
    torch.cuda.synchronize()
    assert np.array_equal(host(gc.kv_scales), oc.kv_scales)
    assert np.array_equal(host(gc.kv_codes), oc.kv_codes)
    assert np.array_equal(untile_idx(host(gc.idx_k), 8, np.uint8), oc.idx_k)
    # every scale code 0..126 occurred
    assert len(np.unique(oc.kv_scales)) == 127


def test_append_without_index_keys_leaves_them_untouched():
    announce("append without index keys")
    m = lib()
    wl = synth.workload("tiny_4k", context=64)
    d = synth.gen_sequence(wl, 0)
    gc = m.Cache(1, 64, idx_heads=4, idx_k_dtype="bf16")
    gc.idx_k.fill_(7)
    m.csa2_kv_append(gc, dev_u16(d.k), dev_u16(d.v), None, dev_i32(np.zeros(64)), dev_i32(np.arange(64)))
    torch.cuda.synchronize()
    assert torch.all(gc.idx_k == 7)
    kc, ks = O.quantize_rows(d.k)
    assert np.array_equal(host(gc.kv_codes)[0, :, :64], kc)


def test_append_is_deterministic_and_idempotent():
    announce("append determinism")
    wl = synth.workload("tiny_4k", context=256, batch=1)
    gc, oc, data = filled_caches(wl)
    before = [host(t).copy() for t in (gc.kv_codes, gc.kv_scales, gc.idx_k)]
    m = lib()
    m.csa2_kv_append(gc, dev_u16(data.k[0]), dev_u16(data.v[0]), dev_u16(data.ik[0]),
                     dev_i32(np.zeros(256)), dev_i32(np.arange(256)))
    torch.cuda.synchronize()
    after = [host(t) for t in (gc.kv_codes, gc.kv_scales, gc.idx_k)]
    for a, b in zip(before, after):
        assert np.array_equal(a, b)
