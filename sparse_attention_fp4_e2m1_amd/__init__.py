"""CSA2 sparse attention over an FP4 (E2M1) KV cache, for MI355X (gfx950).

The hot path lives in ``libcsa2.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/csa2.h``); ``csa2`` is its ctypes binding.  Importing the
binding raises if the library has not been built.
"""
from .csa2 import (  # noqa: F401
    Cache, Csa2Error, csa2_kv_append, csa2_index_topk, csa2_index_topk_append,
    csa2_index_topk_workspace,
    csa2_sparse_attn, csa2_sparse_attn_workspace, LocalCache, csa2_local_append, csa2_local_attn,
    csa2_local_clear, csa2_kv_export, csa2_kv_export_bytes, csa2_kv_import,
    csa2_proj_append, csa2_sparse_local_attn, csa2_sparse_attn_noalloc,
    CSA2_ERR_WORKSPACE, LIB, LIB_PATH,
)
