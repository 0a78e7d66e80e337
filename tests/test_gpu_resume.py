"""GPU tests of the persistent-KV image and of the bounded replay of the local
window: the exported image is the oracle's rows byte for byte, importing it
into another cache (other batch, capacity and sequence slot) reproduces those
rows, the replayed window is byte-identical to the live one, and a step after
the resume (more appends, Full + pool, Reindex, sparse attention, local
window merge) gives bit-identical results on the live and the resumed cache."""
import numpy as np
import pytest
import torch

import synth
from oracle import csa2 as O
from gpu_util import announce, dev_i32, dev_u16, host, lib, untile_idx

pytestmark = pytest.mark.gpu

WINDOW = 96


def _sections(img, n, heads, esz):
    per_tile = 64 // heads
    tiles = (n + per_tile - 1) // per_tile
    codes = img[: n * 128].reshape(n, 128)
    scales = img[n * 128: n * 144].reshape(n, 16)
    idx = img[n * 144: n * 144 + tiles * 4096 * esz]
    assert len(img) >= n * 144 + tiles * 4096 * esz
    return codes, scales, idx


@pytest.mark.parametrize("name,heads,dtype", [("decode_64k_b32", 8, "fp8"), ("tiny_4k", 4, "bf16")])
@pytest.mark.parametrize("n_resume", [1000, 1003])
def test_export_import_replay_resume(name, heads, dtype, n_resume):
    m = lib()
    announce(f"resume {name} heads={heads} idx={dtype} n={n_resume}")
    total = n_resume + 37
    wl = synth.workload(name, context=total, batch=2, idx_heads=heads, idx_k_dtype=dtype)
    data = synth.gen_batch(wl)
    rng = np.random.default_rng(n_resume)
    lk = synth.f32_to_bf16_bits(rng.standard_normal((total, 128)).astype(np.float32))
    lv = synth.f32_to_bf16_bits(rng.standard_normal((total, 128)).astype(np.float32))
    esz = 1 if dtype == "fp8" else 2

    def append(cache, local, seq, lo, hi):
        pos = np.arange(lo, hi, dtype=np.int32)
        s = dev_i32(np.full(hi - lo, seq))
        m.csa2_kv_append(cache, dev_u16(data.k[1, lo:hi]), dev_u16(data.v[1, lo:hi]),
                         dev_u16(data.ik[1, lo:hi]), s, dev_i32(pos))
        for a in range(lo, hi, WINDOW):   # no two rows of one call share a slot
            b = min(hi, a + WINDOW)
            m.csa2_local_append(local, dev_u16(lk[a:b]), dev_u16(lv[a:b]), s[a - lo:b - lo],
                                dev_i32(pos[a - lo:b - lo]))

    # live: sequence 1 of a (2, total) cache up to the resume point
    live = m.Cache(2, 1024 * ((total + 1023) // 1024), idx_heads=heads, idx_k_dtype=dtype)
    llocal = m.LocalCache(2, WINDOW)
    append(live, llocal, 1, 0, n_resume)
    n_bytes = m.csa2_kv_export_bytes(live, n_resume)
    host_img = torch.empty(n_bytes, dtype=torch.uint8, pin_memory=True)
    m.csa2_kv_export(live, 1, n_resume, host_img)
    dev_img = m.csa2_kv_export(live, 1, n_resume)
    torch.cuda.synchronize()
    img = host_img.numpy().copy()
    assert np.array_equal(img, host(dev_img)[:n_bytes])

    # the image is the oracle's rows of the same inputs
    oc = O.OracleCache(1, total, idx_heads=heads, idx_k_dtype=dtype)
    oc.append(data.k[1], data.v[1], data.ik[1], np.zeros(total, int), np.arange(total))
    codes, scales, idx = _sections(img, n_resume, heads, esz)
    assert np.array_equal(codes, oc.kv_codes[0, :n_resume])
    assert np.array_equal(scales, oc.kv_scales[0, :n_resume])
    gidx = untile_idx(idx[None], heads, oc.idx_k.dtype)[0]
    assert np.array_equal(gidx[:n_resume], oc.idx_k[0, :n_resume])

    # resume into sequence 2 of a (3, other capacity) cache from the host image
    res = m.Cache(3, live.capacity + 512, idx_heads=heads, idx_k_dtype=dtype)
    rlocal = m.LocalCache(3, WINDOW)
    junk = synth.f32_to_bf16_bits(rng.standard_normal((WINDOW, 128)).astype(np.float32))
    m.csa2_local_append(rlocal, dev_u16(junk), dev_u16(junk), dev_i32(np.full(WINDOW, 2)),
                        dev_i32(np.arange(WINDOW) + 7))
    m.csa2_kv_import(res, 2, n_resume, host_img)
    m.csa2_local_clear(rlocal, 2)
    lo = max(0, n_resume - WINDOW)                       # bounded replay of the window
    m.csa2_local_append(rlocal, dev_u16(lk[lo:n_resume]), dev_u16(lv[lo:n_resume]),
                        dev_i32(np.full(n_resume - lo, 2)), dev_i32(np.arange(lo, n_resume)))
    torch.cuda.synchronize()
    assert np.array_equal(host(res.kv_codes[2, :n_resume]), host(live.kv_codes[1, :n_resume]))
    assert np.array_equal(host(res.kv_scales[2, :n_resume]), host(live.kv_scales[1, :n_resume]))
    ri = untile_idx(host(res.idx_k[2:3]), heads, oc.idx_k.dtype)[0]
    assert np.array_equal(ri[:n_resume], oc.idx_k[0, :n_resume])
    assert np.array_equal(host(rlocal.k[2]), host(llocal.k[1]))
    assert np.array_equal(host(rlocal.v[2]), host(llocal.v[1]))
    assert np.array_equal(host(rlocal.pos[2]), host(llocal.pos[1]))

    # continue both: the same appends, then one decode step on each
    append(live, llocal, 1, n_resume, total)
    append(res, rlocal, 2, n_resume, total)
    qd = synth.gen_queries(wl, 0)
    qd1 = synth.gen_queries(wl, 1)
    q_pos = dev_i32([total - 1])
    outs = []
    for cache, local, seq in ((live, llocal, 1), (res, rlocal, 2)):
        s = dev_i32([seq])
        tk, pool = m.csa2_index_topk(cache, "full", dev_u16(qd.q_idx[:1]), s, q_pos, 64,
                                     pool_blocks=16)
        rtk, _ = m.csa2_index_topk(cache, "reindex", dev_u16(qd1.q_idx[:1]), s, q_pos, 24,
                                   pool_in=pool)
        out, lse = m.csa2_sparse_attn(cache, dev_u16(qd.q[:1]), s, rtk)
        m.csa2_local_attn(local, dev_u16(qd.q[:1]), s, q_pos, out, lse)
        torch.cuda.synchronize()
        outs.append([host(x) for x in (tk, pool, rtk, out, lse)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    assert np.all(np.isfinite(outs[0][4]))
