"""The C-ABI library loads, exports every declared entry point, and validates
its arguments on the host (no GPU needed: every call here is rejected before
anything is enqueued, or only queries sizes)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from sparse_attention_fp4_e2m1_amd import csa2 as b
    return b


def test_header_declares_the_boundary():
    names = _declared()
    for want in ("csa2_kv_append", "csa2_index_topk", "csa2_sparse_attn",
                 "csa2_index_topk_workspace", "csa2_sparse_attn_workspace",
                 "csa2_local_append", "csa2_local_attn", "csa2_local_clear",
                 "csa2_kv_export", "csa2_kv_export_bytes", "csa2_kv_import", "csa2_proj_append",
                 "csa2_sparse_local_attn", "csa2_sparse_local_attn_workspace",
                 "csa2_index_topk_append", "csa2_strerror", "csa2_abi_version"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(lib.LIB_PATH)
    for name in _declared():
        assert hasattr(raw, name), name
    assert lib.LIB.csa2_abi_version() == 1


def _cache(lib, **kw):
    c = dict(kv_codes=1 << 20, kv_scales=1 << 21, idx_k=1 << 22, batch=2, capacity=4096, dk=128,
             dv=128, idx_heads=8, idx_dim=64, idx_k_dtype=1)
    c.update(kw)
    return lib.csa2_cache(**c)


def test_strerror_covers_all_codes(lib):
    for s in range(7):
        assert lib.LIB.csa2_strerror(s)
    assert b"unknown" in lib.LIB.csa2_strerror(99)


def test_append_validation(lib):
    L = lib.LIB
    P = ctypes.c_void_p
    assert L.csa2_kv_append(None, P(1), P(1), None, P(1), P(1), 4, None) == lib.CSA2_ERR_NULL
    c = _cache(lib, dk=64)
    assert L.csa2_kv_append(ctypes.byref(c), P(1), P(1), None, P(1), P(1), 4, None) == lib.CSA2_ERR_UNSUPPORTED
    c = _cache(lib, idx_heads=6)
    assert L.csa2_kv_append(ctypes.byref(c), P(1), P(1), None, P(1), P(1), 4, None) == lib.CSA2_ERR_UNSUPPORTED
    c = _cache(lib)
    assert L.csa2_kv_append(ctypes.byref(c), P(1), P(1), None, P(1), P(1), -1, None) == lib.CSA2_ERR_SHAPE
    assert L.csa2_kv_append(ctypes.byref(c), None, P(1), None, P(1), P(1), 4, None) == lib.CSA2_ERR_NULL
    assert L.csa2_kv_append(ctypes.byref(c), P(1), P(1), None, P(1), P(1), 0, None) == lib.CSA2_OK
    c = _cache(lib, idx_k=None)
    assert L.csa2_kv_append(ctypes.byref(c), P(1), P(1), P(1), P(1), P(1), 4, None) == lib.CSA2_ERR_NULL
    c = _cache(lib, batch=0)
    assert L.csa2_kv_append(ctypes.byref(c), P(1), P(1), None, P(1), P(1), 4, None) == lib.CSA2_ERR_SHAPE
    c = _cache(lib, capacity=1000)          # the tiled index keys need capacity % 16 == 0
    assert L.csa2_kv_append(ctypes.byref(c), P(1), P(1), None, P(1), P(1), 4, None) == lib.CSA2_ERR_SHAPE
    # 32-bit offsets within a sequence: at most 2^23 positions
    c = _cache(lib, capacity=1 << 23)
    assert L.csa2_kv_append(ctypes.byref(c), P(1), P(1), None, P(1), P(1), 0, None) == lib.CSA2_OK
    c = _cache(lib, capacity=(1 << 23) + 16)
    assert L.csa2_kv_append(ctypes.byref(c), P(1), P(1), None, P(1), P(1), 4, None) == lib.CSA2_ERR_SHAPE
    assert L.csa2_index_topk_workspace(ctypes.byref(c), lib.CSA2_FULL, 1, 16, 0, 0) == 0
    assert L.csa2_sparse_attn_workspace(ctypes.byref(c), 1, 64, 16) == 0
    assert L.csa2_kv_export_bytes(ctypes.byref(c), 16) == 0


def test_index_topk_validation(lib):
    L = lib.LIB
    P = ctypes.c_void_p
    c = ctypes.byref(_cache(lib))

    def call(mode=0, nq=2, top_k=16, pool_in=None, pool_len=0, pool_blocks=0, pool_out=None,
             reuse=None, out=P(1), q=P(1), ws=P(1), ws_bytes=1 << 40):
        return L.csa2_index_topk(c, mode, q, 0, P(1), P(1), nq, top_k, pool_in, pool_len,
                                 pool_blocks, pool_out, reuse, out, ws, ws_bytes, None)

    assert call(top_k=0) == lib.CSA2_ERR_SHAPE
    assert call(top_k=(1 << 16) + 1) == lib.CSA2_ERR_SHAPE
    assert call(nq=-1) == lib.CSA2_ERR_SHAPE
    assert call(mode=7) == lib.CSA2_ERR_ARG
    assert call(out=None) == lib.CSA2_ERR_NULL
    assert call(q=None) == lib.CSA2_ERR_NULL
    assert call(pool_blocks=4) == lib.CSA2_ERR_ARG                 # pool_out missing
    assert call(mode=0, pool_in=P(1), pool_len=8) == lib.CSA2_ERR_ARG
    assert call(mode=1, pool_blocks=4, pool_out=P(1)) == lib.CSA2_ERR_ARG
    assert call(mode=1, pool_in=None, pool_len=8) == lib.CSA2_ERR_ARG
    assert call(mode=2) == lib.CSA2_ERR_ARG                         # reuse_src missing
    assert call(mode=0, reuse=P(1)) == lib.CSA2_ERR_ARG
    assert call(ws=None) == lib.CSA2_ERR_WORKSPACE
    assert call(ws_bytes=16) == lib.CSA2_ERR_WORKSPACE
    assert call(nq=0) == lib.CSA2_OK
    assert call(mode=2, reuse=P(1), nq=0) == lib.CSA2_OK
    assert call(nq=0, q=None, out=None, ws=None) == lib.CSA2_OK   # nothing to point at
    assert call(nq=0, top_k=0) == lib.CSA2_ERR_SHAPE


def test_index_topk_append_validation(lib):
    # the rows are checked first (csa2_kv_append's rules), then the index call
    L = lib.LIB
    P = ctypes.c_void_p
    c = ctypes.byref(_cache(lib))

    def call(n=4, k=P(1), seq=P(1), ik=None, cache=c, mode=0, nq=2, top_k=16, out=P(1), ws=P(1),
             ws_bytes=1 << 40):
        return L.csa2_index_topk_append(cache, k, P(1), ik, seq, P(1), n, mode, P(1), 0, P(1),
                                        P(1), nq, top_k, None, 0, 0, None, None, out, ws,
                                        ws_bytes, None)

    assert call(cache=None) == lib.CSA2_ERR_NULL
    assert call(n=-1) == lib.CSA2_ERR_SHAPE
    assert call(k=None) == lib.CSA2_ERR_NULL
    assert call(seq=None) == lib.CSA2_ERR_NULL
    assert call(ik=P(1), cache=ctypes.byref(_cache(lib, idx_k=None))) == lib.CSA2_ERR_NULL
    assert call(top_k=0) == lib.CSA2_ERR_SHAPE
    assert call(mode=7) == lib.CSA2_ERR_ARG
    assert call(out=None) == lib.CSA2_ERR_NULL
    assert call(ws=None) == lib.CSA2_ERR_WORKSPACE
    assert call(n=0, k=None, seq=None, nq=0) == lib.CSA2_OK        # nothing to do
    assert call(n=0, k=None, seq=None, nq=0, out=None, ws=None) == lib.CSA2_OK


def test_workspace_queries(lib):
    L = lib.LIB
    c = ctypes.byref(_cache(lib))
    full = L.csa2_index_topk_workspace(c, 0, 4, 256, 0, 0)
    pool = L.csa2_index_topk_workspace(c, 0, 4, 256, 0, 64)
    reidx = L.csa2_index_topk_workspace(c, 1, 4, 256, 512, 0)
    assert full >= 4 * 4096 * 4 and pool > full and 0 < reidx < full
    assert L.csa2_index_topk_workspace(c, 2, 4, 256, 0, 0) == 0
    assert L.csa2_index_topk_workspace(c, 0, 4, 0, 0, 0) == 0      # invalid -> 0
    attn = L.csa2_sparse_attn_workspace(c, 4, 64, 2048)
    assert attn >= 4 * 32 * 64 * 128 * 4
    assert L.csa2_sparse_attn_workspace(c, 4, 24, 2048) == 0


def test_workspace_queries_for_no_queries(lib):
    # nq = 0 is a valid call (a no-op), so its size queries must answer too,
    # for both index-key dtypes (the E4M3 one also sizes the matrix-core
    # scorer's layout) and every mode
    L = lib.LIB
    for dtype in (0, 1):
        c = ctypes.byref(_cache(lib, idx_k_dtype=dtype))
        for mode, pool_len, pool_blocks in ((0, 0, 0), (0, 0, 64), (1, 0, 0), (1, 512, 0), (2, 0, 0)):
            L.csa2_index_topk_workspace(c, mode, 0, 256, pool_len, pool_blocks)
        L.csa2_sparse_attn_workspace(c, 0, 64, 2048)
        P = ctypes.c_void_p
        lc = lib.csa2_local_cache(P(1), P(1), P(1), 2, 128, 128, 128)
        L.csa2_sparse_local_attn_workspace(c, ctypes.byref(lc), 0, 64, 2048)


def test_sparse_attn_validation(lib):
    L = lib.LIB
    P = ctypes.c_void_p
    c = ctypes.byref(_cache(lib))

    def call(n_heads=64, nq=2, top_k=64, q=P(1), ws=P(1), ws_bytes=1 << 40):
        return L.csa2_sparse_attn(c, q, n_heads, P(1), nq, P(1), top_k, 0.1, P(1), None, ws,
                                  ws_bytes, None)

    assert call(n_heads=24) == lib.CSA2_ERR_UNSUPPORTED
    assert call(n_heads=144) == lib.CSA2_ERR_UNSUPPORTED
    assert call(top_k=0) == lib.CSA2_ERR_SHAPE
    assert call(q=None) == lib.CSA2_ERR_NULL
    assert call(ws=None) == lib.CSA2_ERR_WORKSPACE
    assert call(ws_bytes=8) == lib.CSA2_ERR_WORKSPACE
    assert call(nq=0) == lib.CSA2_OK


def test_local_window_validation(lib):
    L = lib.LIB
    P = ctypes.c_void_p

    def lc(batch=2, window=128, dk=128, dv=128, k=P(1), v=P(1), pos=P(1)):
        return ctypes.byref(lib.csa2_local_cache(k, v, pos, batch, window, dk, dv))

    def app(c=None, n=4, k=P(1), seq=P(1)):
        return L.csa2_local_append(lc() if c is None else c, k, P(1), seq, P(1), n, None)

    def att(c=None, heads=64, nq=2, out=P(1), lse=P(1), qpos=P(1)):
        return L.csa2_local_attn(lc() if c is None else c, P(1), heads, P(1), qpos, nq, 0.1,
                                 out, lse, None)

    assert app(c=lc(k=None)) == lib.CSA2_ERR_NULL
    assert app(c=lc(pos=None)) == lib.CSA2_ERR_NULL
    assert app(c=lc(window=0)) == lib.CSA2_ERR_SHAPE
    assert app(c=lc(window=1025)) == lib.CSA2_ERR_SHAPE
    assert app(c=lc(batch=0)) == lib.CSA2_ERR_SHAPE
    assert app(c=lc(dk=64)) == lib.CSA2_ERR_UNSUPPORTED
    assert app(n=-1) == lib.CSA2_ERR_SHAPE
    assert app(n=0) == lib.CSA2_OK
    assert app(k=None) == lib.CSA2_ERR_NULL
    assert app(seq=None) == lib.CSA2_ERR_NULL
    assert att(heads=24) == lib.CSA2_ERR_UNSUPPORTED
    assert att(heads=144) == lib.CSA2_ERR_UNSUPPORTED
    assert att(nq=-1) == lib.CSA2_ERR_SHAPE
    assert att(nq=0) == lib.CSA2_OK
    assert att(lse=None) == lib.CSA2_ERR_NULL      # the merge needs the sparse lse
    assert att(out=None) == lib.CSA2_ERR_NULL
    assert att(qpos=None) == lib.CSA2_ERR_NULL


def test_persistent_image_sizes_and_validation(lib):
    L = lib.LIB
    P = ctypes.c_void_p
    c = _cache(lib)                       # 8 E4M3 index heads: tiles of 8 positions, 4 KB
    ref = ctypes.byref(c)
    assert L.csa2_kv_export_bytes(ref, 0) == 0
    assert L.csa2_kv_export_bytes(ref, 1) == 128 + 16 + 4096
    assert L.csa2_kv_export_bytes(ref, 8) == 8 * 144 + 4096
    assert L.csa2_kv_export_bytes(ref, 9) == 9 * 144 + 2 * 4096
    assert L.csa2_kv_export_bytes(ref, 4096) == 4096 * 144 + 512 * 4096
    assert L.csa2_kv_export_bytes(ref, 4097) == 0          # beyond capacity
    bf = ctypes.byref(_cache(lib, idx_heads=4, idx_k_dtype=0))   # bf16, 4 heads: 16 positions, 8 KB
    assert L.csa2_kv_export_bytes(bf, 17) == 17 * 144 + 2 * 8192
    n = L.csa2_kv_export_bytes(ref, 100)
    for fn in (L.csa2_kv_export, L.csa2_kv_import):
        assert fn(ref, 0, 0, None, 0, None) == lib.CSA2_OK        # empty prefix: nothing to copy
        assert fn(ref, 2, 100, P(1), n, None) == lib.CSA2_ERR_SHAPE
        assert fn(ref, -1, 100, P(1), n, None) == lib.CSA2_ERR_SHAPE
        assert fn(ref, 0, 4097, P(1), 1 << 30, None) == lib.CSA2_ERR_SHAPE
        assert fn(ref, 0, 100, None, n, None) == lib.CSA2_ERR_NULL
        assert fn(ref, 0, 100, P(1), n - 1, None) == lib.CSA2_ERR_WORKSPACE
        assert fn(ctypes.byref(_cache(lib, idx_k=None)), 0, 100, P(1), n, None) == lib.CSA2_ERR_NULL
    lc = lib.csa2_local_cache(P(1), P(1), P(1), 2, 128, 128, 128)
    assert L.csa2_local_clear(ctypes.byref(lc), 2, None) == lib.CSA2_ERR_SHAPE
    assert L.csa2_local_clear(ctypes.byref(lc), -1, None) == lib.CSA2_ERR_SHAPE


def test_proj_append_validation(lib):
    L = lib.LIB
    P = ctypes.c_void_p
    ref = ctypes.byref(_cache(lib))

    def call(c=ref, x=P(1), d=512, w=P(1), seq=P(1), n=4):
        return L.csa2_proj_append(c, x, d, w, seq, P(1), n, None)

    assert call(n=0) == lib.CSA2_OK
    assert call(n=-1) == lib.CSA2_ERR_SHAPE
    assert call(d=0) == lib.CSA2_ERR_SHAPE
    assert call(d=48) == lib.CSA2_ERR_SHAPE
    assert call(d=65536 + 32) == lib.CSA2_ERR_SHAPE
    assert call(x=None) == lib.CSA2_ERR_NULL
    assert call(w=None) == lib.CSA2_ERR_NULL
    assert call(seq=None) == lib.CSA2_ERR_NULL
    assert call(c=ctypes.byref(_cache(lib, idx_k=None))) == lib.CSA2_ERR_NULL
    assert call(c=ctypes.byref(_cache(lib, idx_heads=2))) == lib.CSA2_ERR_UNSUPPORTED
