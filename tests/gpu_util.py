"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the library through its binding, and run the oracle on the same inputs."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import synth
from oracle import csa2 as O

DEV = torch.device("cuda:0")


def announce(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def lib():
    import sparse_attention_fp4_e2m1_amd as m
    return m


def dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def filled_caches(wl: synth.Workload, capacity=None, seqs=None):
    """GPU cache filled through csa2_kv_append and the oracle cache filled by the oracle,
    from the same seeded bf16 rows (every row of every sequence)."""
    m = lib()
    cap = capacity or wl.context
    gc = m.Cache(wl.batch, cap, idx_heads=wl.idx_heads, idx_k_dtype=wl.idx_k_dtype)
    oc = O.OracleCache(wl.batch, cap, idx_heads=wl.idx_heads, idx_k_dtype=wl.idx_k_dtype)
    data = synth.gen_batch(wl)
    for b in range(wl.batch) if seqs is None else seqs:
        seq = np.full(wl.context, b, np.int32)
        pos = np.arange(wl.context, dtype=np.int32)
        m.csa2_kv_append(gc, dev_u16(data.k[b]), dev_u16(data.v[b]), dev_u16(data.ik[b]),
                         dev_i32(seq), dev_i32(pos))
        oc.append(data.k[b], data.v[b], data.ik[b], seq, pos)
    torch.cuda.synchronize()
    return gc, oc, data


def untile_idx(raw: np.ndarray, heads: int, dtype) -> np.ndarray:
    """Index keys from the library's tiled layout (include/csa2.h) to
    [batch][capacity][heads][64] in `dtype` (uint8 E4M3 codes or uint16 bf16 bits)."""
    esz = np.dtype(dtype).itemsize
    raw = np.ascontiguousarray(raw).view(np.uint8)
    b = raw.shape[0]
    t = 64 // heads
    chunks = 4 * esz
    r = raw.reshape(b, -1, chunks, t, heads, 16)          # [b][tile][chunk][pos][head][16]
    r = r.transpose(0, 1, 3, 4, 2, 5)                     # [b][tile][pos][head][chunk][16]
    return np.ascontiguousarray(r).reshape(b, -1, heads, 64 * esz).view(dtype).reshape(b, -1, heads, 64)


def attn_errors(out, lse, ref_out, ref_lse):
    """Per (query, head) row: max_c |delta| / max_c |ref|, and |delta lse|."""
    out = np.asarray(out, np.float64)
    ref_out = np.asarray(ref_out, np.float64)
    den = np.abs(ref_out).max(axis=-1)
    num = np.abs(out - ref_out).max(axis=-1)
    rel = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    lse = np.asarray(lse, np.float64)
    ref_lse = np.asarray(ref_lse, np.float64)
    both_inf = np.isneginf(lse) & np.isneginf(ref_lse)
    dl = np.where(both_inf, 0.0, np.abs(lse - ref_lse))
    return rel, dl


ATTN_TOL = 2e-3
DEFAULT_SCALE = float(np.float32(1.0 / math.sqrt(128)))


# ---------------------------------------------------------------------------
# Relaxed index-set rule, for the matrix-core scorer (E4M3 index queries
# against E4M3 keys over all visible positions): its fp32 sums follow the
# matrix core's order, so scores near the K-th one may swap places with the
# oracle's fixed-order scores.  A GPU set G is accepted against the oracle set
# O when |G| = |O|, G is ascending, distinct and made of candidates, and every
# element of G xor O has an exact score within 2 * 512 * 2^-24 * (sum|q||k|
# of it + of the oracle's K-th element) of the oracle's K-th element's exact
# score.  Everything away from the boundary must agree exactly.
# ---------------------------------------------------------------------------
GAMMA_512 = 512 * 2.0 ** -24


def matrix_core_layer(wl, layer) -> bool:
    """Whether the library scores this layer on matrix cores."""
    if wl.q_idx_dtype != "fp8" or wl.idx_k_dtype != "fp8":
        return False
    if layer.mode == "full":
        return layer.pool_blocks == 0
    return layer.mode == "reindex" and layer.pool_from < 0


def relaxed_topk_check(got, want, cand, canon, exact, mag) -> int:
    """got, want: [K] rows (ascending, -1 padded); cand: the candidate positions
    (ascending); canon, exact, mag: the oracle's fp32 score, exact score and
    magnitude sum per candidate.  Returns the number of swapped pairs; raises
    AssertionError if the rule fails."""
    got = np.asarray(got)
    want = np.asarray(want)
    g = got[got >= 0]
    w = want[want >= 0]
    assert np.all(got[len(g):] == -1), "padding"
    assert len(g) == len(w), (len(g), len(w))
    assert np.all(np.diff(g) > 0), "ascending and distinct"
    cand = np.asarray(cand)
    gi = np.searchsorted(cand, g)
    assert np.all(gi < len(cand)) and np.array_equal(cand[gi], g), "members are candidates"
    diff = np.setxor1d(g, w)
    if len(diff) == 0:
        return 0
    wi = np.searchsorted(cand, w)
    ws = np.asarray(canon, np.float64)[wi]
    kth = wi[np.lexsort((-w, ws))[0]]            # smallest score; among equals the highest position
    di = np.searchsorted(cand, diff)
    tol = 2 * GAMMA_512 * (np.asarray(mag)[di] + mag[kth])
    far = np.abs(np.asarray(exact)[di] - exact[kth]) > tol
    assert not far.any(), f"swapped elements away from the K-th score: {diff[far][:8]}"
    return len(diff) // 2


def check_stack(wl, oc, stack, ref, qs, rows, log=None):
    """Checks a LayerStack's results for sampled queries against the oracle.

    rows: (query index on the GPU, row of `ref`, the query's sequence in `oc`).
    Top-K: bit-exact, except on matrix-core layers (relaxed rule); Reuse: the
    GPU source layer's rows unchanged; pools bit-exact; attention within
    ATTN_TOL of the oracle on the same index rows (recomputed by the oracle
    where a relaxed set differs from its own)."""
    qpos = wl.query_pos()
    topks = [host(t) for t in stack.topk]
    for li, layer in enumerate(wl.layers):
        tk = topks[li]
        out, lse = host(stack.out[li]), host(stack.lse[li])
        pool = host(stack.pool[li]) if ref[li]["pool"] is not None else None
        swaps, worst = 0, 0.0
        for i, r, b in rows:
            p = int(qpos[i])
            if layer.mode == "reuse":
                # the oracle's list of the Reuse layer (its source's list), unless
                # the GPU's source list differs from the oracle's (a matrix-core
                # source, judged there by the relaxed rule): then the GPU's source
                src = layer.reuse_from
                same_src = np.array_equal(topks[src][i], ref[src]["topk"][r])
                want = ref[li]["topk"][r] if same_src else topks[src][i]
                assert np.array_equal(tk[i], want), f"layer {li} reuse"
            elif matrix_core_layer(wl, layer):
                qi = O.query_index_values(qs[li].q_idx[i], "fp8")
                cand = np.arange(p + 1)
                keys = oc.index_key_values(b, cand)
                exact, mag = O.index_scores_exact(qi, keys)
                swaps += relaxed_topk_check(tk[i], ref[li]["topk"][r], cand,
                                            O.index_scores(qi, keys), exact, mag)
            else:
                assert np.array_equal(tk[i], ref[li]["topk"][r]), f"layer {li} Top-K of query {i}"
            if pool is not None:
                assert np.array_equal(pool[i], ref[li]["pool"][r]), f"layer {li} pool of query {i}"
            if np.array_equal(tk[i], ref[li]["topk"][r]):
                ro, rl = ref[li]["out"][r], ref[li]["lse"][r]
            else:
                ro, rl = O.sparse_attention(qs[li].q[i], oc, b, tk[i])
            rel, dl = attn_errors(out[i], lse[i], ro, rl)
            assert rel.max() <= ATTN_TOL and dl.max() <= ATTN_TOL, (li, i, rel.max(), dl.max())
            worst = max(worst, float(rel.max()))
        if log is not None:
            log(f"  layer {li} ({layer.mode}) ok: max rel err {worst:.2e}"
                + (f", {swaps} swaps at the K-th score" if matrix_core_layer(wl, layer) else ""))
