"""One CSA2 step over a stack of layers, as a sequence of C-ABI calls.

aiwiki "DeepSeek V4.1-Flash", section "Compressed Sparse Attention 2": every
layer has a static mode.  A Full layer scores the shared index keys and makes a
fresh Top-K (the decoder's first Full layer also builds the candidate pool); a
Reindex layer scores the pool (or everything visible) with its own query; a
Reuse layer recycles an earlier layer's Top-K.  Every layer then attends over
its Top-K rows of the shared FP4 main KV.

All buffers (Top-K lists, pools, outputs, workspaces) are allocated once in the
constructor, so a step only enqueues kernels and can be captured in a graph.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import csa2 as B


class LayerStack:
    def __init__(self, cache: B.Cache, layers: Sequence, nq: int, heads: int, top_k: int,
                 q_idx_dtype: str = "bf16", softmax_scale: Optional[float] = None):
        self.cache, self.layers, self.nq, self.heads, self.top_k = cache, list(layers), nq, heads, top_k
        self.q_idx_dtype = q_idx_dtype
        # K of each layer: its own (a layer's top_k > 0), else the stack's;
        # a Reuse layer has its source's
        self.k = []
        for L in self.layers:
            if L.mode == "reuse":
                self.k.append(self.k[L.reuse_from])
            else:
                self.k.append(getattr(L, "top_k", 0) or top_k)
        self.softmax_scale = softmax_scale
        d = cache.device
        # a Reuse layer's list is its source's list itself (an alias: the
        # indices are unchanged, so no copy is enqueued; csa2_index_topk's
        # Reuse mode is the copying form for callers that need their own buffer)
        self.topk = []
        for li, L in enumerate(self.layers):
            if L.mode == "reuse":
                self.topk.append(self.topk[L.reuse_from])
            else:
                self.topk.append(torch.full((nq, self.k[li]), -1, dtype=torch.int32, device=d))
        self.pool = [torch.full((nq, 8 * L.pool_blocks), -1, dtype=torch.int32, device=d)
                     if (L.mode == "full" and L.pool_blocks > 0) else None for L in self.layers]
        self.out = [torch.zeros((nq, heads, cache.dv), dtype=torch.float32, device=d) for _ in self.layers]
        self.lse = [torch.zeros((nq, heads), dtype=torch.float32, device=d) for _ in self.layers]
        ws, wa = 0, 0
        for li, L in enumerate(self.layers):
            pool_len = 8 * self.layers[L.pool_from].pool_blocks if (L.mode == "reindex" and L.pool_from >= 0) else 0
            ws = max(ws, B.csa2_index_topk_workspace(cache, L.mode, nq, self.k[li], pool_len,
                                                     L.pool_blocks if L.mode == "full" else 0))
            wa = max(wa, B.csa2_sparse_attn_workspace(cache, nq, heads, self.k[li]))
        self.ws_topk = torch.empty(max(ws, 256), dtype=torch.uint8, device=d)
        self.ws_attn = torch.empty(max(wa, 256), dtype=torch.uint8, device=d)

    def run(self, q: Sequence[torch.Tensor], q_idx: Sequence[torch.Tensor], q_seq: torch.Tensor,
            q_pos: torch.Tensor, append: Optional[tuple] = None, stream=None,
            scan_events: Optional[tuple] = None, mark=None):
        """Enqueue one step: optional append (k, v, idx_k, seq, pos), then every layer
        (the append rides in the first index layer's call, csa2_index_topk_append).

        scan_events: optional (before, after) hipEvent_t handles recorded around the
        index scoring of the first Full layer (csa2_profile_index_scan).
        mark: optional callable, called with ("attn", layer, "before" / "after")
        right before and after each layer's attention call is enqueued (a
        caller records its own events there)."""
        # the step's append goes into the first index layer's call (one launch
        # fewer where the scorer can take it), else on its own
        if append is not None and self.layers[0].mode == "reuse":
            k, v, ik, seq, pos = append
            B.csa2_kv_append(self.cache, k, v, ik, seq, pos, stream=stream)
            append = None
        for li, L in enumerate(self.layers):
            if L.mode == "reuse":
                pass   # self.topk[li] is self.topk[L.reuse_from]
            elif L.mode == "full":
                if scan_events is not None:
                    B.LIB.csa2_profile_index_scan(scan_events[0], scan_events[1])
                try:
                    B.csa2_index_topk(self.cache, "full", q_idx[li], q_seq, q_pos, self.k[li],
                                      q_dtype=self.q_idx_dtype, pool_blocks=L.pool_blocks,
                                      topk_out=self.topk[li], pool_out=self.pool[li],
                                      workspace=self.ws_topk, stream=stream, append=append)
                finally:
                    if scan_events is not None:
                        B.LIB.csa2_profile_index_scan(None, None)
                        scan_events = None
            else:
                pool_in = self.pool[L.pool_from] if L.pool_from >= 0 else None
                B.csa2_index_topk(self.cache, "reindex", q_idx[li], q_seq, q_pos, self.k[li],
                                  q_dtype=self.q_idx_dtype, pool_in=pool_in,
                                  topk_out=self.topk[li], workspace=self.ws_topk, stream=stream,
                                  append=append)
            if L.mode != "reuse":
                append = None
            if mark is not None:
                mark("attn", li, "before")
            B.csa2_sparse_attn(self.cache, q[li], q_seq, self.topk[li],
                               softmax_scale=self.softmax_scale, out=self.out[li],
                               lse=self.lse[li], workspace=self.ws_attn, stream=stream)
            if mark is not None:
                mark("attn", li, "after")
