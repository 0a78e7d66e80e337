"""Workload presets and seeded input generation for the CSA2 hot path.

The shapes follow the pages' statement of the problem (the model card
"DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression", section
Introduction, CSA2 paragraph; the aiwiki article "DeepSeek V4.1-Flash",
sections "Compressed Sparse Attention 2" and "KV-cache formats and bounded
replay"): one shared FP4 main-KV head with K and V of 128 channels each, a
multi-head indexer, per-query Top-K, a decoder candidate pool of 8-position
blocks, contexts up to 1,048,576 tokens.  The pages publish no data, so every
value here is synthetic and seeded.

Everything in this module is random-number drawing and layout.  The only
numeric transform is rounding float32 draws to bfloat16 (round to nearest
even), which is how the bf16 inputs of the path are produced.

Seeds (numpy ``SeedSequence(seed, spawn_key=...)``, PCG64 generators):
    spawn_key (0,)          structure draws (outlier channels / channel
                            log-scales / outlier tokens)
    spawn_key (t, b, c)     rows [c*ROW_CHUNK, (c+1)*ROW_CHUNK) of sequence b
                            for tensor t = 1 main K, 2 main V, 3 index keys
    spawn_key (4, layer, j) queries of one layer: j = 0 attention query,
                            j = 1 index query
    Each key names its draw, so any sequence (or chunk) regenerates on its own
    and chunks can be drawn in parallel.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

ROW_CHUNK = 1 << 16


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 values (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Layer:
    mode: str                 # "full" | "reindex" | "reuse"
    pool_blocks: int = 0      # full: number of 8-position blocks kept in the pool (0: no pool)
    pool_from: int = -1       # reindex: layer whose pool is searched (-1: no pool, all visible)
    reuse_from: int = -1      # reuse: layer whose Top-K indices are recycled
    top_k: int = 0            # full / reindex: this layer's K (0: the workload's); reuse: its source's


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int                # sequences in the cache
    context: int              # rows per sequence after the step's append
    heads: int                # attention query heads sharing the one KV head
    idx_heads: int            # indexer heads
    idx_k_dtype: str          # "bf16" | "fp8": storage type of the index keys
    q_idx_dtype: str          # "bf16" | "fp8": precision the index query is scored in
    top_k: int
    layers: tuple
    keys: str                 # value structure, see gen_structure
    prefill: int = 0          # >0: this many new causal query tokens (one sequence)
    idx_dim: int = 64
    dk: int = 128
    dv: int = 128

    @property
    def nq(self) -> int:
        return self.prefill if self.prefill else self.batch

    @property
    def appended(self) -> int:
        """Rows appended per sequence by one step (decode: 1, prefill: the chunk)."""
        return self.prefill if self.prefill else 1

    def query_seq(self) -> np.ndarray:
        if self.prefill:
            return np.zeros(self.prefill, np.int32)
        return np.arange(self.batch, dtype=np.int32)

    def query_pos(self) -> np.ndarray:
        """Position of each query; it sees cache rows [0, pos]."""
        if self.prefill:
            return np.arange(self.context - self.prefill, self.context, dtype=np.int32)
        return np.full(self.batch, self.context - 1, np.int32)

    def n_row_chunks(self) -> int:
        return (self.context + ROW_CHUNK - 1) // ROW_CHUNK

    def idx_bytes_per_token(self) -> int:
        return self.idx_heads * self.idx_dim * (1 if self.idx_k_dtype == "fp8" else 2)


def _full(pool_blocks=0):
    return Layer("full", pool_blocks=pool_blocks)


WORKLOADS = {
    # batch 1, 4096 context, 16 heads, indexer 4x64 bf16, Top-K 256, one Full layer;
    # N(0,1) values, main K and V each with 4 outlier channels scaled x8.
    "tiny_4k": Workload("tiny_4k", seed=0, batch=1, context=4096, heads=16, idx_heads=4,
                        idx_k_dtype="bf16", q_idx_dtype="bf16", top_k=256,
                        layers=(_full(),), keys="outlier_channels"),
    # batch 32, 65536 context, 64 heads, indexer 8x64 fp8 keys, Top-K 2048, Full mode;
    # main K and index keys N(0,1) times a per-channel log-normal scale.
    "decode_64k_b32": Workload("decode_64k_b32", seed=1, batch=32, context=65536, heads=64,
                               idx_heads=8, idx_k_dtype="fp8", q_idx_dtype="bf16",
                               top_k=2048, layers=(_full(),), keys="lognormal_channels"),
    # batch 8, 262144 context; layer 0 Full building a 1024-block (8192-position) pool,
    # layers 1-3 Reindex over it, layers 4-7 Reuse layer 3's indices.
    "chain8_256k_b8": Workload("chain8_256k_b8", seed=2, batch=8, context=262144, heads=64,
                               idx_heads=8, idx_k_dtype="fp8", q_idx_dtype="bf16",
                               top_k=2048,
                               layers=(_full(1024),
                                       Layer("reindex", pool_from=0),
                                       Layer("reindex", pool_from=0),
                                       Layer("reindex", pool_from=0),
                                       Layer("reuse", reuse_from=3),
                                       Layer("reuse", reuse_from=3),
                                       Layer("reuse", reuse_from=3),
                                       Layer("reuse", reuse_from=3)),
                               keys="plain"),
    # batch 1, 1,048,576 context; Full over every token building a 2048-block
    # (16384-position) pool, then Reindex over the pool; 1% of tokens have keys x10.
    "decode_1m": Workload("decode_1m", seed=3, batch=1, context=1 << 20, heads=64,
                          idx_heads=8, idx_k_dtype="fp8", q_idx_dtype="bf16", top_k=2048,
                          layers=(_full(2048), Layer("reindex", pool_from=0)),
                          keys="outlier_tokens"),
    # the released pool setting: batch 8, 262144 context; layer 0 Full (K 2048)
    # building a 2048-block (16384-position) pool, layers 1-3 Reindex over the
    # pool selecting 512 each, layers 4-7 Reuse layer 3's 512 indices.
    "released_256k_b8": Workload("released_256k_b8", seed=5, batch=8, context=262144, heads=64,
                                 idx_heads=8, idx_k_dtype="fp8", q_idx_dtype="bf16", top_k=2048,
                                 layers=(_full(2048),
                                         Layer("reindex", pool_from=0, top_k=512),
                                         Layer("reindex", pool_from=0, top_k=512),
                                         Layer("reindex", pool_from=0, top_k=512),
                                         Layer("reuse", reuse_from=3),
                                         Layer("reuse", reuse_from=3),
                                         Layer("reuse", reuse_from=3),
                                         Layer("reuse", reuse_from=3)),
                                 keys="plain"),
    # encoder side (no candidate pool): 4096 new causal query tokens on a
    # 131072-row cache; layer 0 Full (K 2048), layer 1 Reindex over every
    # visible position selecting 512, layer 2 Reuse layer 1's indices.
    "encoder_4k_on_128k": Workload("encoder_4k_on_128k", seed=6, batch=1, context=131072 + 4096,
                                   heads=64, idx_heads=8, idx_k_dtype="fp8", q_idx_dtype="fp8",
                                   top_k=2048,
                                   layers=(_full(), Layer("reindex", top_k=512),
                                           Layer("reuse", reuse_from=1)),
                                   keys="plain", prefill=4096),
    # 4096 new causal query tokens appended to a 131072-row cache; fp8 indexer
    # scoring, per-query causal Top-K 2048, 64-head sparse attention.
    "prefill_4k_on_128k": Workload("prefill_4k_on_128k", seed=4, batch=1, context=131072 + 4096,
                                   heads=64, idx_heads=8, idx_k_dtype="fp8", q_idx_dtype="fp8",
                                   top_k=2048, layers=(_full(),), keys="plain", prefill=4096),
}


def workload(name: str, **overrides) -> Workload:
    """A preset, optionally with fields replaced (e.g. a smaller context for tests)."""
    wl = WORKLOADS[name]
    return dataclasses.replace(wl, **overrides) if overrides else wl


def _seed(wl: Workload, *key):
    return np.random.SeedSequence(wl.seed, spawn_key=tuple(key))


@dataclasses.dataclass
class Structure:
    k_outlier_channels: Optional[np.ndarray] = None   # main-K channels scaled x8
    v_outlier_channels: Optional[np.ndarray] = None   # main-V channels scaled x8
    k_channel_scale: Optional[np.ndarray] = None      # [dk] float32 exp(g)
    ik_channel_scale: Optional[np.ndarray] = None     # [idx_heads, idx_dim] float32 exp(g)
    outlier_tokens: Optional[list] = None             # per sequence: sorted row indices scaled x10


def gen_structure(wl: Workload) -> Structure:
    rng = np.random.Generator(np.random.PCG64(_seed(wl, 0)))
    st = Structure()
    if wl.keys == "outlier_channels":
        st.k_outlier_channels = np.sort(rng.choice(wl.dk, 4, replace=False))
        st.v_outlier_channels = np.sort(rng.choice(wl.dv, 4, replace=False))
    elif wl.keys == "lognormal_channels":
        st.k_channel_scale = np.exp(rng.standard_normal(wl.dk)).astype(np.float32)
        st.ik_channel_scale = np.exp(rng.standard_normal((wl.idx_heads, wl.idx_dim))).astype(np.float32)
    elif wl.keys == "outlier_tokens":
        st.outlier_tokens = [np.sort(rng.choice(wl.context, wl.context // 100, replace=False))
                             for _ in range(wl.batch)]
    elif wl.keys != "plain":
        raise ValueError(wl.keys)
    return st


@dataclasses.dataclass
class SequenceData:
    k: np.ndarray    # [rows, dk] uint16 bf16 bits
    v: np.ndarray    # [rows, dv] uint16 bf16 bits
    ik: np.ndarray   # [rows, idx_heads, idx_dim] uint16 bf16 bits


def _draw_rows(seed_seq, shape):
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    out = np.empty(shape, np.float32)
    rng.standard_normal(dtype=np.float32, out=out)
    return out


def _fill_chunk(wl, st, b, c, seeds, out):
    lo = c * ROW_CHUNK
    hi = min(wl.context, lo + ROW_CHUNK)
    n = hi - lo
    k = _draw_rows(seeds[0], (n, wl.dk))
    v = _draw_rows(seeds[1], (n, wl.dv))
    ik = _draw_rows(seeds[2], (n, wl.idx_heads, wl.idx_dim))
    if st.k_outlier_channels is not None:
        k[:, st.k_outlier_channels] *= np.float32(8.0)
        v[:, st.v_outlier_channels] *= np.float32(8.0)
    if st.k_channel_scale is not None:
        k *= st.k_channel_scale[None, :]
        ik *= st.ik_channel_scale[None, :, :]
    if st.outlier_tokens is not None:
        rows = st.outlier_tokens[b]
        rows = rows[(rows >= lo) & (rows < hi)] - lo
        k[rows] *= np.float32(10.0)
        ik[rows] *= np.float32(10.0)
    out.k[lo:hi] = f32_to_bf16_bits(k)
    out.v[lo:hi] = f32_to_bf16_bits(v)
    out.ik[lo:hi] = f32_to_bf16_bits(ik)


def gen_sequence(wl: Workload, b: int, threads: int = 8, st: Optional[Structure] = None) -> SequenceData:
    """All `context` rows of sequence b (bf16 bits)."""
    st = st if st is not None else gen_structure(wl)
    nchunk = wl.n_row_chunks()
    out = SequenceData(np.empty((wl.context, wl.dk), np.uint16),
                       np.empty((wl.context, wl.dv), np.uint16),
                       np.empty((wl.context, wl.idx_heads, wl.idx_dim), np.uint16))
    tasks = [(c, tuple(_seed(wl, t, b, c) for t in (1, 2, 3))) for c in range(nchunk)]
    if threads <= 1 or nchunk == 1:
        for c, seeds in tasks:
            _fill_chunk(wl, st, b, c, seeds, out)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda t: _fill_chunk(wl, st, b, t[0], t[1], out), tasks))
    return out


def gen_batch(wl: Workload, threads: int = 8) -> SequenceData:
    """Rows of every sequence, stacked: k [batch, context, dk], v, ik likewise."""
    st = gen_structure(wl)
    nchunk = wl.n_row_chunks()
    k = np.empty((wl.batch, wl.context, wl.dk), np.uint16)
    v = np.empty((wl.batch, wl.context, wl.dv), np.uint16)
    ik = np.empty((wl.batch, wl.context, wl.idx_heads, wl.idx_dim), np.uint16)
    views = [SequenceData(k[b], v[b], ik[b]) for b in range(wl.batch)]
    tasks = [(b, c) for b in range(wl.batch) for c in range(nchunk)]

    def run(t):
        b, c = t
        _fill_chunk(wl, st, b, c, tuple(_seed(wl, t, b, c) for t in (1, 2, 3)), views[b])

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(run, tasks))
    return SequenceData(k, v, ik)


@dataclasses.dataclass
class QueryData:
    q: np.ndarray       # [nq, heads, dk] uint16 bf16 bits
    q_idx: np.ndarray   # [nq, idx_heads, idx_dim] uint16 bf16 bits


def gen_queries(wl: Workload, layer: int) -> QueryData:
    """The attention query and index query of every query token, for one layer."""
    q = _draw_rows(_seed(wl, 4, layer, 0), (wl.nq, wl.heads, wl.dk))
    qi = _draw_rows(_seed(wl, 4, layer, 1), (wl.nq, wl.idx_heads, wl.idx_dim))
    return QueryData(f32_to_bf16_bits(q), f32_to_bf16_bits(qi))
