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
