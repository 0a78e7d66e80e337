"""CSA2 hot path, written out plainly on the CPU (test infrastructure only).

Steps, in the pages' order (aiwiki "DeepSeek V4.1-Flash", section "Compressed
Sparse Attention 2"; model card, Introduction, CSA2 paragraph):

1. quantize-and-append of main K/V into the FP4 cache (E2M1 codes, one E4M3
   scale per 16 channels) and storage of the index keys;
2. index scoring of every causally visible candidate against the layer's index
   query, and per-query Top-K, in Full, Reindex or Reuse mode, with the
   decoder's candidate pool of 8-position blocks ranked by their maximum score;
3. gather and dequantization of the selected rows;
4. softmax attention of every query head over those rows.

Cache layout (the library's main-KV layout, so parity compares raw bytes):
    kv_codes  [batch][capacity][dk/2 + dv/2]  uint8: K codes then V codes;
              channel 2i in the low nibble of byte i, 2i+1 in the high nibble
    kv_scales [batch][capacity][dk/16 + dv/16] uint8 E4M3: K scales then V
    idx_k     [batch][capacity][idx_heads][idx_dim]: bf16 bits (uint16) or
              E4M3 codes (uint8), in logical order (the library tiles them)
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .formats import (bf16_value, e2m1_encode, e2m1_value, e4m3_encode, e4m3_encode_ratio,
                      e4m3_value, fma_f32)

BLOCK = 16          # channels per E4M3 scale
POOL_BLOCK = 8      # positions per candidate-pool block


# ---------------------------------------------------------------------------
# Step 1: quantize-and-append
# ---------------------------------------------------------------------------

def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., 2n] 4-bit codes -> [..., n] bytes; even channel in the low nibble (reading)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def quantize_rows(x_bits: np.ndarray):
    """FP4 quantization of bf16 rows [n, d] (d a multiple of 16).

    Model card, Introduction, CSA2 paragraph: E2M1 values with one E4M3 scale
    per 16 channels.  Reading (the pages give no rule): the scale of a block is
    the E4M3 value nearest amax/6 (amax = largest |x| in the block, 6 = largest
    E2M1 magnitude), RNE, saturating at 448; each element takes the E2M1 code
    nearest x/scale, RNE, saturating at 6, keeping x's sign.

    Returns (packed codes [n, d/2] uint8, scale codes [n, d/16] uint8).
    """
    x = bf16_value(x_bits)
    n, d = x.shape
    blocks = x.reshape(n, d // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=2)
    sc = e4m3_encode_ratio(amax, 6.0)
    s = e4m3_value(sc)
    codes = e2m1_encode(blocks, s[:, :, None]).reshape(n, d)
    return pack_nibbles(codes), sc


def dequantize_rows(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Value of FP4 rows: E2M1(code) * E4M3(scale), float64 (exact)."""
    codes = unpack_nibbles(packed)
    n, d = codes.shape
    v = e2m1_value(codes).reshape(n, d // BLOCK, BLOCK) * e4m3_value(scales)[:, :, None]
    return v.reshape(n, d)


# E4M3 of every bf16 bit pattern and the value of every E4M3 code: the same
# functions evaluated once per distinct input, so large caches decode fast.
_E4M3_OF_BF16 = None
_E4M3_VALUE = None


def _e4m3_tables():
    global _E4M3_OF_BF16, _E4M3_VALUE
    if _E4M3_OF_BF16 is None:
        bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
        with np.errstate(invalid="ignore"):
            vals = bf16_value(bits)
        finite = np.isfinite(vals)
        enc = np.zeros(1 << 16, np.uint8)
        enc[finite] = e4m3_encode(vals[finite])
        _E4M3_OF_BF16 = enc
        _E4M3_VALUE = e4m3_value(np.arange(256)).astype(np.float32)
    return _E4M3_OF_BF16, _E4M3_VALUE


class OracleCache:
    """Host copy of the FP4 main-KV cache and the index-key cache (logical layout).

    lazy=True keeps the appended bf16 K/V rows and quantizes a row only when
    it is read (kv_values), for contexts too long to quantize whole; the index
    keys are always stored.
    """

    def __init__(self, batch, capacity, dk=128, dv=128, idx_heads=8, idx_dim=64, idx_k_dtype="fp8",
                 lazy=False):
        self.batch, self.capacity = batch, capacity
        self.dk, self.dv, self.idx_heads, self.idx_dim = dk, dv, idx_heads, idx_dim
        self.idx_k_dtype = idx_k_dtype
        self.lazy = lazy
        if lazy:
            self.raw_k = [None] * batch     # per sequence: list of (pos, K bits, V bits)
            self.kv_codes = self.kv_scales = None
        else:
            self.kv_codes = np.zeros((batch, capacity, dk // 2 + dv // 2), np.uint8)
            self.kv_scales = np.zeros((batch, capacity, dk // BLOCK + dv // BLOCK), np.uint8)
        ik_t = np.uint8 if idx_k_dtype == "fp8" else np.uint16
        self.idx_k = np.zeros((batch, capacity, idx_heads, idx_dim), ik_t)

    def bytes_per_token(self) -> dict:
        """Bytes one cached position occupies (main KV and index keys)."""
        main = self.kv_codes.shape[2] + self.kv_scales.shape[2]
        idx = self.idx_k.shape[2] * self.idx_k.shape[3] * self.idx_k.itemsize
        return {"main_kv": main, "index_keys": idx}

    def append(self, k_bits, v_bits, ik_bits, seq, pos):
        """Quantize and store rows r at (seq[r], pos[r]).

        Index keys are stored verbatim (bf16 cache) or cast to E4M3 with RNE,
        saturating (fp8 cache).  The pages say index keys come from main-KV
        entries (aiwiki, "Compressed Sparse Attention 2") without giving the map;
        here they arrive as an input, as the learned projection needs weights.
        """
        seq = np.asarray(seq)
        pos = np.asarray(pos)
        if self.lazy:
            for b in np.unique(seq):
                m = seq == b
                entry = (pos[m], np.asarray(k_bits)[m], np.asarray(v_bits)[m])
                self.raw_k[b] = (self.raw_k[b] or []) + [entry]
        else:
            kc, ks = quantize_rows(k_bits)
            vc, vs = quantize_rows(v_bits)
            self.kv_codes[seq, pos] = np.concatenate([kc, vc], axis=1)
            self.kv_scales[seq, pos] = np.concatenate([ks, vs], axis=1)
        if ik_bits is not None:
            if self.idx_k_dtype == "fp8":
                self.idx_k[seq, pos] = _e4m3_tables()[0][np.asarray(ik_bits, np.uint16)]
            else:
                self.idx_k[seq, pos] = np.asarray(ik_bits, np.uint16)

    def index_key_values(self, b, rows) -> np.ndarray:
        """Decoded index keys of sequence b at `rows`, float32 [n, idx_heads, idx_dim]."""
        raw = self.idx_k[b, rows]
        if self.idx_k_dtype == "fp8":
            return _e4m3_tables()[1][raw]
        return bf16_value(raw).astype(np.float32)

    def _rows_bits(self, b, rows):
        """bf16 K and V bits of sequence b at `rows` (lazy mode; latest append wins)."""
        k = np.zeros((len(rows), self.dk), np.uint16)
        v = np.zeros((len(rows), self.dv), np.uint16)
        for pos, kb, vb in self.raw_k[b] or []:
            where = np.full(self.capacity, -1, np.int64)
            where[pos] = np.arange(len(pos))
            idx = where[rows]
            hit = idx >= 0
            k[hit] = kb[idx[hit]]
            v[hit] = vb[idx[hit]]
        return k, v

    def kv_values(self, b, rows):
        """Dequantized (K, V) of sequence b at `rows`, float64 [n, dk], [n, dv]."""
        if self.lazy:
            kb, vb = self._rows_bits(b, np.asarray(rows))
            kc, ks = quantize_rows(kb)
            vc, vs = quantize_rows(vb)
            return dequantize_rows(kc, ks), dequantize_rows(vc, vs)
        codes = self.kv_codes[b, rows]
        scales = self.kv_scales[b, rows]
        hk, sk = self.dk // 2, self.dk // BLOCK
        k = dequantize_rows(codes[:, :hk], scales[:, :sk])
        v = dequantize_rows(codes[:, hk:], scales[:, sk:])
        return k, v


# ---------------------------------------------------------------------------
# Step 2: index scoring, Top-K, candidate pool, modes
# ---------------------------------------------------------------------------

def query_index_values(q_idx_bits, dtype: str) -> np.ndarray:
    """Index query as float32 values: bf16 as given, or cast to E4M3 (RNE, saturating)."""
    v = bf16_value(q_idx_bits)
    if dtype == "fp8":
        v = e4m3_value(e4m3_encode(v))
    return v.astype(np.float32)


def index_scores(q: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Index score of every candidate: sum over indexer heads of q_h . k_h, in fp32.

    Source: aiwiki "Compressed Sparse Attention 2" (Full and Reindex layers
    score candidate positions with a new index query against the shared index
    keys).  The pages do not give the score's form.  Reading: the plain sum over
    heads of the head dot products, no activation or head weights, accumulated
    in fp32 the plain way, left to right, so that the Top-K decision is
    reproducible:
      * per head h: acc_h = 0, then acc_h = fma(q[h][c], k[h][c], acc_h) for
        c = 0, 1, ..., D-1 (one chain of fused multiply-adds, a single rounding
        per step);
      * over heads: s = acc_0, then s = s + acc_h for h = 1, ..., H-1.

    q: float32 [H, D]; keys: float32 [n, H, D]; returns float32 [n].
    Pins: exact rational evaluation of this order on cancelling inputs, exact
    integer cases, and the fp32 error bound against the exact dot product
    (tests/test_oracle_scores.py).
    """
    q = np.asarray(q, np.float32)
    keys = np.asarray(keys, np.float32)
    n = keys.shape[0]
    H, D = q.shape
    acc = np.zeros((n, H), np.float32)
    for c in range(D):
        acc = fma_f32(q[None, :, c], keys[:, :, c], acc)
    s = acc[:, 0].copy()
    for h in range(1, H):
        s = (s + acc[:, h]).astype(np.float32)
    return s


def index_scores_exact(q: np.ndarray, keys: np.ndarray):
    """The index score of every candidate without rounding, and its magnitude sum.

    Same sum as index_scores (every head, every channel: sum_h q_h . k_h) taken
    in float64, with sum_h |q_h| . |k_h| beside it (the scale of the fp32
    rounding error of any summation order: n terms in any order stay within
    n * 2^-24 times that sum).  For E4M3 queries against E4M3 keys the result
    is exact: an E4M3 value is a multiple of 2^-9 below 2^9, so each product is
    a multiple of 2^-18 below 2^18 and a sum of 512 of them needs at most 45
    bits; float64 carries 53, in any order.

    q: float32 [H, D]; keys: float32 [n, H, D]; returns (float64 [n], float64 [n]).
    Used to check index sets of a scorer whose fp32 sums follow another order.
    """
    q = np.asarray(q, np.float64).reshape(-1)
    k = np.asarray(keys, np.float64).reshape(len(keys), -1)
    return k @ q, np.abs(k) @ np.abs(q)


def topk_select(scores: np.ndarray, positions: np.ndarray, k: int) -> np.ndarray:
    """The k candidates with the largest scores, as positions in ascending order, -1 padded.

    Source: model card, CSA2 paragraph and aiwiki "Compressed Sparse Attention 2"
    (each indexing layer makes a fresh Top-K selection).  Readings: ties in
    score go to the lower position; -0 and +0 are equal; fewer than k
    candidates leaves -1 padding at the end.
    """
    s = np.asarray(scores, np.float32).astype(np.float64) + 0.0   # -0.0 -> +0.0
    positions = np.asarray(positions, np.int64)
    order = np.lexsort((positions, -s))             # score descending, then position ascending
    chosen = np.sort(positions[order[:k]])
    out = np.full(k, -1, np.int32)
    out[:len(chosen)] = chosen
    return out


def build_pool(scores: np.ndarray, pool_blocks: int) -> np.ndarray:
    """Candidate pool of the first Full layer, from scores of positions 0..n-1.

    Source: aiwiki "Compressed Sparse Attention 2" (the first Full-mode decoder
    layer scores every visible position, ranks blocks of eight positions by
    their maximum index score and keeps a fixed number of blocks as the shared
    pool).  Readings: blocks are aligned to position 0; a partial last block
    uses its visible members; block ties go to the lower block; the pool lists
    the kept positions in ascending order, -1 padded to 8 * pool_blocks.
    """
    s = np.asarray(scores, np.float32)
    n = len(s)
    nblk = (n + POOL_BLOCK - 1) // POOL_BLOCK
    padded = np.full(nblk * POOL_BLOCK, -np.inf, np.float32)   # absent members never win a max
    padded[:n] = s
    bmax = padded.reshape(nblk, POOL_BLOCK).max(axis=1)
    blocks = topk_select(bmax, np.arange(nblk), pool_blocks)
    pos = [p for b in blocks if b >= 0
           for p in range(b * POOL_BLOCK, min(n, (b + 1) * POOL_BLOCK))]
    out = np.full(POOL_BLOCK * pool_blocks, -1, np.int32)
    out[:len(pos)] = pos
    return out


def index_topk(mode: str, cache: OracleCache, seq: int, q_pos: int, q_idx: np.ndarray, top_k: int,
               pool_in: Optional[np.ndarray] = None, pool_blocks: int = 0,
               reuse_src: Optional[np.ndarray] = None):
    """One query's Top-K in the given mode; returns (topk, pool or None, scores, candidates).

    Source: aiwiki "Compressed Sparse Attention 2":
      * full: score every causally visible position [0, q_pos]; optionally
        build the candidate pool;
      * reindex: new index query over an earlier layer's index keys, searching
        only the pool (pool_in; entries -1 or beyond q_pos are skipped), or all
        visible positions when no pool is given;
      * reuse: the earlier layer's Top-K indices, unchanged.
    q_idx: float32 [idx_heads, idx_dim] (see query_index_values).
    """
    if mode == "reuse":
        return np.array(reuse_src, np.int32).copy(), None, None, None
    if mode == "full" or pool_in is None:
        cand = np.arange(q_pos + 1)
    elif mode == "reindex":
        p = np.asarray(pool_in, np.int64)
        cand = p[(p >= 0) & (p <= q_pos)]
    else:
        raise ValueError(mode)
    # candidates are scored independently; chunks only bound the memory
    chunk = 1 << 16
    scores = np.concatenate([index_scores(q_idx, cache.index_key_values(seq, cand[i:i + chunk]))
                             for i in range(0, len(cand), chunk)] or [np.zeros(0, np.float32)])
    topk = topk_select(scores, cand, top_k)
    pool = build_pool(scores, pool_blocks) if (mode == "full" and pool_blocks > 0) else None
    return topk, pool, scores, cand


# ---------------------------------------------------------------------------
# Steps 3-4: gather, dequantize, softmax attention
# ---------------------------------------------------------------------------

def sparse_attention(q_bits: np.ndarray, cache: OracleCache, seq: int, topk: np.ndarray,
                     scale: Optional[float] = None):
    """Softmax attention of every head over the selected rows, in float64.

    Source: model card, CSA2 paragraph and aiwiki "Compressed Sparse Attention
    2" (each layer attends over its Top-K positions of the shared FP4 main KV,
    one KV head shared by all query heads).  For head h:
        z_j = scale * (q_h . K_j),  o_h = sum_j softmax(z)_j V_j,
        lse_h = ln sum_j exp(z_j),
    over the entries j of `topk` that are >= 0 (each entry counts once).
    Readings: no positional term, no sink, sparse rows only; scale defaults to
    1/sqrt(dk); an empty selection gives o = 0 and lse = -inf.

    q_bits: bf16 bits [heads, dk].  Returns (out [heads, dv], lse [heads]).
    """
    q = bf16_value(q_bits)
    H = q.shape[0]
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(cache.dk)))
    rows = np.asarray(topk, np.int64)
    rows = rows[rows >= 0]
    if len(rows) == 0:
        return np.zeros((H, cache.dv)), np.full(H, -np.inf)
    k, v = cache.kv_values(seq, rows)
    z = (q @ k.T) * scale
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    ell = p.sum(axis=1, keepdims=True)
    out = (p @ v) / ell
    lse = (m + np.log(ell))[:, 0]
    return out, lse


# ---------------------------------------------------------------------------
# The local sliding-window branch
# ---------------------------------------------------------------------------

class OracleLocalCache:
    """One layer's local sliding-window K and V in FP8: a ring of `window`
    slots per sequence, position p in slot p % window, with the position each
    slot holds (-1 = none).

    Source: aiwiki "DeepSeek V4.1-Flash", section "Compressed Sparse Attention
    2" (every CSA2 layer creates its own local sliding-window keys and values)
    and section "KV-cache formats and bounded replay" (the local window KV is
    stored in FP8).  Readings (the pages give no format detail): each bf16
    element becomes its OCP E4M3 code (round to nearest even, saturating at
    448, sign kept), with no scale; the window of a query at position p is
    positions max(0, p - window + 1) .. p.
    """

    def __init__(self, batch, window, dk=128, dv=128):
        self.batch, self.window, self.dk, self.dv = batch, window, dk, dv
        self.k = np.zeros((batch, window, dk), np.uint8)
        self.v = np.zeros((batch, window, dv), np.uint8)
        self.pos = np.full((batch, window), -1, np.int64)

    def append(self, k_bits, v_bits, seq, pos):
        enc = _e4m3_tables()[0]
        k_bits = np.asarray(k_bits, np.uint16)
        v_bits = np.asarray(v_bits, np.uint16)
        for r, (b, p) in enumerate(zip(np.asarray(seq), np.asarray(pos))):
            s = int(p) % self.window
            self.k[b, s] = enc[k_bits[r]]
            self.v[b, s] = enc[v_bits[r]]
            self.pos[b, s] = int(p)

    def window_rows(self, b, q_pos):
        """(positions, K, V) of the window of a query at q_pos in sequence b:
        the positions whose slot holds them, ascending; K, V float64."""
        val = _e4m3_tables()[1]
        want = np.arange(max(0, q_pos - self.window + 1), q_pos + 1)
        slots = want % self.window
        have = self.pos[b, slots] == want
        sl = slots[have]
        return want[have], val[self.k[b, sl]].astype(np.float64), val[self.v[b, sl]].astype(np.float64)


def attention_with_window(q_bits: np.ndarray, cache: OracleCache, seq: int, topk: np.ndarray,
                          local: OracleLocalCache, q_pos: int, scale: Optional[float] = None):
    """Softmax attention of every head over the selected FP4 rows and the
    layer's FP8 window rows together, in float64.

    Source: as sparse_attention for the selected rows; aiwiki "Compressed
    Sparse Attention 2" for the local window every layer also attends over.
    One softmax over both sets: z_j = scale * (q_h . K_j) for the entries of
    `topk` (>= 0) and the window rows, o_h = sum_j softmax(z)_j V_j,
    lse_h = ln sum_j exp(z_j).  Reading: the two sets are different cached
    values (the shared FP4 global KV, the layer's own FP8 window) side by side,
    so a position in both counts twice; no positional term.

    q_bits: bf16 bits [heads, dk].  Returns (out [heads, dv], lse [heads]).
    """
    q = bf16_value(q_bits)
    H = q.shape[0]
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(cache.dk)))
    rows = np.asarray(topk, np.int64)
    rows = rows[rows >= 0]
    ks, vs = [], []
    if len(rows):
        k, v = cache.kv_values(seq, rows)
        ks.append(k)
        vs.append(v)
    _, kl, vl = local.window_rows(seq, q_pos)
    if len(kl):
        ks.append(kl)
        vs.append(vl)
    if not ks:
        return np.zeros((H, cache.dv)), np.full(H, -np.inf)
    k = np.concatenate(ks)
    v = np.concatenate(vs)
    z = (q @ k.T) * scale
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    ell = p.sum(axis=1, keepdims=True)
    return (p @ v) / ell, (m + np.log(ell))[:, 0]


# ---------------------------------------------------------------------------
# A whole step over a layer stack
# ---------------------------------------------------------------------------

def run_layers(cache: OracleCache, layers: Sequence, q_seq, q_pos, queries, top_k: int,
               q_idx_dtype: str, scale: Optional[float] = None, only=None):
    """Index Top-K and attention for every layer of a stack, per query.

    layers: objects with .mode, .pool_blocks, .pool_from, .reuse_from (and
    optionally .top_k: a layer's own K; 0 or absent means top_k)
    queries: per layer, objects with .q [nq, heads, dk] and .q_idx [nq, H_I, D] bf16 bits.
    only: optional list of query indices to compute (others are skipped).
    Returns per layer a dict with 'topk' [nq, K], 'pool' (or None), 'out', 'lse'.
    """
    nq = len(q_seq)
    sel = range(nq) if only is None else list(only)
    results = []
    for li, layer in enumerate(layers):
        qd = queries[li]
        # this layer's K: a Reuse layer keeps its source's list; otherwise the
        # layer's own top_k when it has one (> 0), else the stack's
        if layer.mode == "reuse":
            k_li = results[layer.reuse_from]["topk"].shape[1]
        else:
            k_li = getattr(layer, "top_k", 0) or top_k
        res = {"topk": np.full((nq, k_li), -1, np.int32), "pool": None,
               "out": np.zeros((nq, qd.q.shape[1], cache.dv)),
               "lse": np.full((nq, qd.q.shape[1]), -np.inf)}
        if layer.mode == "full" and layer.pool_blocks > 0:
            res["pool"] = np.full((nq, POOL_BLOCK * layer.pool_blocks), -1, np.int32)
        for i in sel:
            b, p = int(q_seq[i]), int(q_pos[i])
            pool_in = None
            if layer.mode == "reindex" and layer.pool_from >= 0:
                pool_in = results[layer.pool_from]["pool"][i]
            reuse = results[layer.reuse_from]["topk"][i] if layer.mode == "reuse" else None
            qi = query_index_values(qd.q_idx[i], q_idx_dtype)
            topk, pool, _, _ = index_topk(layer.mode, cache, b, p, qi, k_li, pool_in=pool_in,
                                          pool_blocks=layer.pool_blocks, reuse_src=reuse)
            res["topk"][i] = topk
            if pool is not None:
                res["pool"][i] = pool
            res["out"][i], res["lse"][i] = sparse_attention(qd.q[i], cache, b, topk, scale)
        results.append(res)
    return results


def bf16_round_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bits of finite float64 values rounded to nearest, ties to even
    (8 significant bits; the exponent range of float32, with its subnormals
    spaced 2^-133).  Values are assumed to lie within bf16's finite range."""
    v = np.asarray(v, np.float64)
    _, e = np.frexp(v)                                  # |v| = m 2^e, 0.5 <= m < 1
    step = np.ldexp(1.0, np.maximum(e, -125) - 8)       # spacing of bf16 values near v
    r = np.rint(v / step) * step                        # np.rint: ties to even
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def project_rows(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """The encoder-side projection of hidden states to the rows csa2 appends.

    Source: aiwiki "DeepSeek V4.1-Flash", section "Causal Encoder-Decoder": a
    decoder layer's global keys and values are projected from the final
    causal-encoder hidden states with that layer's own weights.  Readings (the
    pages give no precision or layout): y = W x per token, taken exactly (the
    float64 sum of bf16 products, exact when the products and partial sums
    fit 53 bits) and rounded once to bf16; W has one row per output channel:
    K channels 0..127, V 128..255, then the index keys head by head.

    x_bits [n, d_model], w_bits [channels, d_model] bf16 bits.  Returns the
    bf16 bits of y [n, channels].
    """
    x = bf16_value(x_bits).astype(np.float64)
    w = bf16_value(w_bits).astype(np.float64)
    return bf16_round_bits(x @ w.T)


def project_and_append(cache: OracleCache, x_bits, w_bits, seq, pos):
    """project_rows, then the cache's own quantize-and-append of the K, V and
    index-key parts of the projected rows."""
    y = project_rows(x_bits, w_bits)
    H, D = cache.idx_k.shape[2], cache.idx_k.shape[3]
    n = y.shape[0]
    cache.append(y[:, :cache.dk], y[:, cache.dk:cache.dk + cache.dv],
                 y[:, cache.dk + cache.dv:].reshape(n, H, D), seq, pos)
    return y
