"""ctypes binding of libcsa2.so: argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module checks
tensor shapes/dtypes/devices, passes raw device pointers and the current HIP
stream, and turns status codes into exceptions.  PyTorch provides device
memory and streams.  If the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# CSA2_LIBRARY names another build of the library (the sanitizer build of the
# host code); by default the in-tree libcsa2.so.
LIB_PATH = os.environ.get("CSA2_LIBRARY") or os.path.join(_HERE, "libcsa2.so")

CSA2_OK, CSA2_ERR_NULL, CSA2_ERR_SHAPE, CSA2_ERR_UNSUPPORTED, CSA2_ERR_WORKSPACE, CSA2_ERR_HIP, \
    CSA2_ERR_ARG = range(7)
CSA2_FULL, CSA2_REINDEX, CSA2_REUSE = 0, 1, 2
CSA2_BF16, CSA2_FP8_E4M3 = 0, 1
MODES = {"full": CSA2_FULL, "reindex": CSA2_REINDEX, "reuse": CSA2_REUSE}
DTYPES = {"bf16": CSA2_BF16, "fp8": CSA2_FP8_E4M3}


class csa2_cache(ctypes.Structure):
    _fields_ = [("kv_codes", ctypes.c_void_p), ("kv_scales", ctypes.c_void_p),
                ("idx_k", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
                ("idx_k_dtype", ctypes.c_int32)]


class csa2_local_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("window", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python sparse_attention_fp4_e2m1_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    C = ctypes.POINTER(csa2_cache)
    sig = {
        "csa2_kv_append": (I32, [C, P, P, P, P, P, I32, P]),
        "csa2_index_topk_workspace": (SZ, [C, I32, I32, I32, I32, I32]),
        "csa2_index_topk": (I32, [C, I32, P, I32, P, P, I32, I32, P, I32, I32, P, P, P, P, SZ, P]),
        "csa2_index_topk_append": (I32, [C, P, P, P, P, P, I32, I32, P, I32, P, P, I32, I32, P, I32,
                                         I32, P, P, P, P, SZ, P]),
        "csa2_sparse_attn_workspace": (SZ, [C, I32, I32, I32]),
        "csa2_sparse_attn": (I32, [C, P, I32, P, I32, P, I32, F32, P, P, P, SZ, P]),
        "csa2_sparse_attn_noalloc": (I32, [C, P, I32, P, I32, P, I32, F32, P, P, P]),
        "csa2_local_append": (I32, [ctypes.POINTER(csa2_local_cache), P, P, P, P, I32, P]),
        "csa2_local_attn": (I32, [ctypes.POINTER(csa2_local_cache), P, I32, P, P, I32, F32, P, P, P]),
        "csa2_proj_append": (I32, [C, P, I32, P, P, P, I32, P]),
        "csa2_sparse_local_attn_workspace": (SZ, [C, ctypes.POINTER(csa2_local_cache), I32, I32, I32]),
        "csa2_sparse_local_attn": (I32, [C, ctypes.POINTER(csa2_local_cache), P, I32, P, P, I32, P,
                                         I32, F32, P, P, P, SZ, P]),
        "csa2_kv_export_bytes": (SZ, [C, I32]),
        "csa2_kv_export": (I32, [C, I32, I32, P, SZ, P]),
        "csa2_kv_import": (I32, [C, I32, I32, P, SZ, P]),
        "csa2_local_clear": (I32, [ctypes.POINTER(csa2_local_cache), I32, P]),
        "csa2_profile_index_scan": (None, [P, P]),
        "csa2_strerror": (ctypes.c_char_p, [I32]),
        "csa2_abi_version": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


class Csa2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {LIB.csa2_strerror(status).decode()} (status {status})")
        self.status = status


def _check(status: int, where: str):
    if status != CSA2_OK:
        raise Csa2Error(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t, name, dtypes, shape=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")


_B16 = (torch.bfloat16, torch.int16, torch.uint16)
_I32 = (torch.int32,)


class Cache:
    """FP4 main-KV + index-key cache in device memory (the library's byte layout)."""

    def __init__(self, batch: int, capacity: int, idx_heads: int = 8, idx_k_dtype: str = "fp8",
                 dk: int = 128, dv: int = 128, idx_dim: int = 64, device="cuda"):
        self.batch, self.capacity = batch, capacity
        self.dk, self.dv, self.idx_heads, self.idx_dim = dk, dv, idx_heads, idx_dim
        self.idx_k_dtype = idx_k_dtype
        dev = torch.device(device)
        self.kv_codes = torch.zeros((batch, capacity, dk // 2 + dv // 2), dtype=torch.uint8, device=dev)
        self.kv_scales = torch.zeros((batch, capacity, dk // 16 + dv // 16), dtype=torch.uint8, device=dev)
        idt = torch.uint8 if idx_k_dtype == "fp8" else torch.int16
        self.idx_k = torch.zeros((batch, capacity, idx_heads, idx_dim), dtype=idt, device=dev)
        self.device = self.kv_codes.device
        self._c = csa2_cache(self.kv_codes.data_ptr(), self.kv_scales.data_ptr(),
                             self.idx_k.data_ptr(), batch, capacity, dk, dv, idx_heads, idx_dim,
                             DTYPES[idx_k_dtype])

    @property
    def ref(self):
        return ctypes.byref(self._c)

    def nbytes(self) -> int:
        return self.kv_codes.numel() + self.kv_scales.numel() + self.idx_k.numel() * self.idx_k.element_size()


def csa2_kv_append(cache: Cache, k, v, idx_k_in, seq, pos, stream=None) -> None:
    n = k.shape[0]
    d = cache.device
    _need(k, "k", _B16, (n, cache.dk), d)
    _need(v, "v", _B16, (n, cache.dv), d)
    if idx_k_in is not None:
        _need(idx_k_in, "idx_k_in", _B16, (n, cache.idx_heads, cache.idx_dim), d)
    _need(seq, "seq", _I32, (n,), d)
    _need(pos, "pos", _I32, (n,), d)
    _check(LIB.csa2_kv_append(cache.ref, _ptr(k), _ptr(v), _ptr(idx_k_in), _ptr(seq), _ptr(pos),
                              n, _stream(stream)), "csa2_kv_append")


def csa2_index_topk_workspace(cache: Cache, mode: str, nq: int, top_k: int, pool_len: int = 0,
                              pool_blocks: int = 0) -> int:
    return int(LIB.csa2_index_topk_workspace(cache.ref, MODES[mode], nq, top_k, pool_len, pool_blocks))


def csa2_index_topk(cache: Cache, mode: str, q_idx, q_seq, q_pos, top_k: int, q_dtype: str = "bf16",
                    pool_in=None, pool_blocks: int = 0, reuse_src=None, topk_out=None,
                    pool_out=None, workspace=None, stream=None, append=None):
    """Returns (topk_out [nq, top_k] int32, pool_out [nq, 8*pool_blocks] int32 or None).

    append: optional (k, v, idx_k_in, seq, pos), csa2_kv_append's rows, appended
    first in the same call (csa2_index_topk_append)."""
    d = cache.device
    if mode == "reuse":
        _need(reuse_src, "reuse_src", _I32, None, d)
        nq = reuse_src.shape[0]
        _need(reuse_src, "reuse_src", _I32, (nq, top_k), d)
    else:
        nq = q_idx.shape[0]
        _need(q_idx, "q_idx", _B16, (nq, cache.idx_heads, cache.idx_dim), d)
        _need(q_seq, "q_seq", _I32, (nq,), d)
        _need(q_pos, "q_pos", _I32, (nq,), d)
    pool_len = 0
    if pool_in is not None:
        pool_len = pool_in.shape[1]
        _need(pool_in, "pool_in", _I32, (nq, pool_len), d)
    if topk_out is None:
        topk_out = torch.empty((nq, top_k), dtype=torch.int32, device=d)
    _need(topk_out, "topk_out", _I32, (nq, top_k), d)
    if pool_blocks > 0 and pool_out is None:
        pool_out = torch.empty((nq, 8 * pool_blocks), dtype=torch.int32, device=d)
    if pool_out is not None:
        _need(pool_out, "pool_out", _I32, (nq, 8 * pool_blocks), d)
    ws_bytes = csa2_index_topk_workspace(cache, mode, nq, top_k, pool_len, pool_blocks)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=d)
    tail = (MODES[mode], _ptr(q_idx), DTYPES[q_dtype], _ptr(q_seq), _ptr(q_pos), nq, top_k,
            _ptr(pool_in), pool_len, pool_blocks, _ptr(pool_out), _ptr(reuse_src), _ptr(topk_out),
            _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream))
    if append is None:
        _check(LIB.csa2_index_topk(cache.ref, *tail), "csa2_index_topk")
    else:
        k, v, ik, seq, pos = append
        n = k.shape[0]
        _need(k, "k", _B16, (n, cache.dk), d)
        _need(v, "v", _B16, (n, cache.dv), d)
        if ik is not None:
            _need(ik, "idx_k_in", _B16, (n, cache.idx_heads, cache.idx_dim), d)
        _need(seq, "seq", _I32, (n,), d)
        _need(pos, "pos", _I32, (n,), d)
        _check(LIB.csa2_index_topk_append(cache.ref, _ptr(k), _ptr(v), _ptr(ik), _ptr(seq),
                                          _ptr(pos), n, *tail), "csa2_index_topk_append")
    return topk_out, pool_out


def csa2_index_topk_append(cache: Cache, k, v, idx_k_in, seq, pos, mode: str, q_idx, q_seq, q_pos,
                           top_k: int, **kw):
    """csa2_kv_append(cache, k, v, idx_k_in, seq, pos) then csa2_index_topk(cache,
    mode, q_idx, q_seq, q_pos, top_k, **kw) in one call; returns csa2_index_topk's."""
    return csa2_index_topk(cache, mode, q_idx, q_seq, q_pos, top_k,
                           append=(k, v, idx_k_in, seq, pos), **kw)


def csa2_sparse_attn_workspace(cache: Cache, nq: int, n_heads: int, top_k: int) -> int:
    return int(LIB.csa2_sparse_attn_workspace(cache.ref, nq, n_heads, top_k))


def csa2_sparse_attn(cache: Cache, q, q_seq, topk, softmax_scale: Optional[float] = None,
                     out=None, lse=None, want_lse: bool = True, workspace=None, stream=None):
    """Returns (out [nq, heads, dv] fp32, lse [nq, heads] fp32 or None)."""
    d = cache.device
    nq, n_heads = q.shape[0], q.shape[1]
    top_k = topk.shape[1]
    _need(q, "q", _B16, (nq, n_heads, cache.dk), d)
    _need(q_seq, "q_seq", _I32, (nq,), d)
    _need(topk, "topk", _I32, (nq, top_k), d)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(cache.dk)
    if out is None:
        out = torch.empty((nq, n_heads, cache.dv), dtype=torch.float32, device=d)
    _need(out, "out", (torch.float32,), (nq, n_heads, cache.dv), d)
    if lse is None and want_lse:
        lse = torch.empty((nq, n_heads), dtype=torch.float32, device=d)
    if lse is not None:
        _need(lse, "lse", (torch.float32,), (nq, n_heads), d)
    ws_bytes = csa2_sparse_attn_workspace(cache, nq, n_heads, top_k)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=d)
    _check(LIB.csa2_sparse_attn(cache.ref, _ptr(q), n_heads, _ptr(q_seq), nq, _ptr(topk), top_k,
                                float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                workspace.numel(), _stream(stream)), "csa2_sparse_attn")
    return out, lse


def csa2_sparse_attn_noalloc(cache: Cache, q, q_seq, topk, softmax_scale: Optional[float] = None,
                             out=None, lse=None, stream=None):
    """csa2_sparse_attn with the library's static scratch (no workspace); out
    and lse must be given (the call allocates nothing).  Returns (out, lse)."""
    d = cache.device
    nq, n_heads = q.shape[0], q.shape[1]
    top_k = topk.shape[1]
    _need(q, "q", _B16, (nq, n_heads, cache.dk), d)
    _need(q_seq, "q_seq", _I32, (nq,), d)
    _need(topk, "topk", _I32, (nq, top_k), d)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(cache.dk)
    _need(out, "out", (torch.float32,), (nq, n_heads, cache.dv), d)
    if lse is not None:
        _need(lse, "lse", (torch.float32,), (nq, n_heads), d)
    _check(LIB.csa2_sparse_attn_noalloc(cache.ref, _ptr(q), n_heads, _ptr(q_seq), nq, _ptr(topk),
                                        top_k, float(softmax_scale), _ptr(out), _ptr(lse),
                                        _stream(stream)), "csa2_sparse_attn_noalloc")
    return out, lse


class LocalCache:
    """One layer's local sliding-window KV: E4M3 codes in a ring of `window`
    slots per sequence, with the position each slot holds (-1 = none)."""

    def __init__(self, batch: int, window: int, dk: int = 128, dv: int = 128, device="cuda"):
        self.batch, self.window, self.dk, self.dv = batch, window, dk, dv
        dev = torch.device(device)
        self.k = torch.zeros((batch, window, dk), dtype=torch.uint8, device=dev)
        self.v = torch.zeros((batch, window, dv), dtype=torch.uint8, device=dev)
        self.pos = torch.full((batch, window), -1, dtype=torch.int32, device=dev)
        self.device = self.k.device
        self._c = csa2_local_cache(self.k.data_ptr(), self.v.data_ptr(), self.pos.data_ptr(), batch,
                                   window, dk, dv)

    @property
    def ref(self):
        return ctypes.byref(self._c)


def csa2_local_append(cache: LocalCache, k, v, seq, pos, stream=None) -> None:
    n = k.shape[0]
    d = cache.device
    _need(k, "k", _B16, (n, cache.dk), d)
    _need(v, "v", _B16, (n, cache.dv), d)
    _need(seq, "seq", _I32, (n,), d)
    _need(pos, "pos", _I32, (n,), d)
    _check(LIB.csa2_local_append(cache.ref, _ptr(k), _ptr(v), _ptr(seq), _ptr(pos), n,
                                 _stream(stream)), "csa2_local_append")


def csa2_local_attn(cache: LocalCache, q, q_seq, q_pos, out, lse,
                    softmax_scale: Optional[float] = None, stream=None):
    """Merges the window branch into (out, lse) of csa2_sparse_attn, in place."""
    d = cache.device
    nq, n_heads = q.shape[0], q.shape[1]
    _need(q, "q", _B16, (nq, n_heads, cache.dk), d)
    _need(q_seq, "q_seq", _I32, (nq,), d)
    _need(q_pos, "q_pos", _I32, (nq,), d)
    _need(out, "out", (torch.float32,), (nq, n_heads, cache.dv), d)
    _need(lse, "lse", (torch.float32,), (nq, n_heads), d)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(cache.dk)
    _check(LIB.csa2_local_attn(cache.ref, _ptr(q), n_heads, _ptr(q_seq), _ptr(q_pos), nq,
                               float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)),
           "csa2_local_attn")
    return out, lse


def csa2_kv_export_bytes(cache: Cache, length: int) -> int:
    return int(LIB.csa2_kv_export_bytes(cache.ref, int(length)))


def _image_buffer(t, name, nbytes):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or not t.is_contiguous():
        raise TypeError(f"{name}: a contiguous uint8 tensor is required")
    if t.device.type == "cpu" and not t.is_pinned():
        raise ValueError(f"{name}: host memory must be pinned (pin_memory=True)")
    if t.numel() < nbytes:
        raise ValueError(f"{name}: {t.numel()} bytes, {nbytes} needed")


def csa2_kv_export(cache: Cache, seq: int, length: int, dst=None, stream=None):
    """Persistent image of positions [0, length) of sequence seq, into dst (a
    uint8 tensor on the device or in pinned host memory; allocated on the
    device when None).  Ordered on the stream."""
    n = csa2_kv_export_bytes(cache, length)
    if dst is None:
        dst = torch.empty(max(n, 1), dtype=torch.uint8, device=cache.device)
    _image_buffer(dst, "dst", n)
    _check(LIB.csa2_kv_export(cache.ref, int(seq), int(length), _ptr(dst), dst.numel(),
                              _stream(stream)), "csa2_kv_export")
    return dst


def csa2_kv_import(cache: Cache, seq: int, length: int, src, stream=None) -> None:
    _image_buffer(src, "src", csa2_kv_export_bytes(cache, length))
    _check(LIB.csa2_kv_import(cache.ref, int(seq), int(length), _ptr(src), src.numel(),
                              _stream(stream)), "csa2_kv_import")


def csa2_local_clear(cache: LocalCache, seq: int, stream=None) -> None:
    _check(LIB.csa2_local_clear(cache.ref, int(seq), _stream(stream)), "csa2_local_clear")


def csa2_proj_append(cache: Cache, x, w, seq, pos, stream=None) -> None:
    """Projects hidden states x [n, d_model] with w [256 + idx_heads*64, d_model]
    (bf16 bits) and appends the K, V and index-key rows (include/csa2.h)."""
    n, d_model = x.shape[0], x.shape[1]
    d = cache.device
    _need(x, "x", _B16, (n, d_model), d)
    _need(w, "w", _B16, (256 + cache.idx_heads * 64, d_model), d)
    _need(seq, "seq", _I32, (n,), d)
    _need(pos, "pos", _I32, (n,), d)
    _check(LIB.csa2_proj_append(cache.ref, _ptr(x), d_model, _ptr(w), _ptr(seq), _ptr(pos), n,
                                _stream(stream)), "csa2_proj_append")


def csa2_sparse_local_attn(cache: Cache, local: LocalCache, q, q_seq, q_pos, topk,
                           softmax_scale: Optional[float] = None, out=None, lse=None,
                           workspace=None, stream=None):
    """Both branches in one pass (include/csa2.h); returns (out, lse)."""
    d = cache.device
    nq, n_heads = q.shape[0], q.shape[1]
    top_k = topk.shape[1]
    _need(q, "q", _B16, (nq, n_heads, cache.dk), d)
    _need(q_seq, "q_seq", _I32, (nq,), d)
    _need(q_pos, "q_pos", _I32, (nq,), d)
    _need(topk, "topk", _I32, (nq, top_k), d)
    if out is None:
        out = torch.empty((nq, n_heads, cache.dv), dtype=torch.float32, device=d)
    if lse is None:
        lse = torch.empty((nq, n_heads), dtype=torch.float32, device=d)
    _need(out, "out", (torch.float32,), (nq, n_heads, cache.dv), d)
    _need(lse, "lse", (torch.float32,), (nq, n_heads), d)
    ws = int(LIB.csa2_sparse_local_attn_workspace(cache.ref, local.ref, nq, n_heads, top_k))
    if workspace is None:
        workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=d)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(cache.dk)
    _check(LIB.csa2_sparse_local_attn(cache.ref, local.ref, _ptr(q), n_heads, _ptr(q_seq),
                                      _ptr(q_pos), nq, _ptr(topk), top_k, float(softmax_scale),
                                      _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                      _stream(stream)), "csa2_sparse_local_attn")
    return out, lse
