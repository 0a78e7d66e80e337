"""GPU parity of csa2_proj_append (the encoder-side projection fused into
quantize-and-append) against the oracle's project_and_append.

Bit-exact on hidden states and weights drawn from a coarse grid (x in
{-1, -3/4, .., 1}, w in {-1/2, -3/8, .., 1/2}): every product and partial sum
is a multiple of 2^-5 of magnitude at most d_model / 2 <= 2^15 (20
significant bits), exact in fp32 in any order, so the matrix
cores' sums equal the oracle's exact ones and the bf16 rounding, codes, scales
and index keys agree byte for byte.  On random normal inputs the fp32
accumulation order differs from the exact sum, so a value that lands next to
a bf16 rounding boundary may round the other way: there every byte must be the
encoding of a value within the fp32 error bound of the exact sum
(tests/proj_rule.py, itself checked on the CPU with planted mistakes).  The
contraction order does not depend on the call's size: the same rows give the
same bytes alone and inside a larger call."""
import numpy as np
import pytest
import torch

import synth
from oracle import csa2 as O
from gpu_util import announce, dev_i32, dev_u16, host, lib, untile_idx
from proj_rule import check_projection_bytes

pytestmark = pytest.mark.gpu


def _run(heads, dtype, n, d_model, grid=True, seed=0, capacity=512):
    m = lib()
    rng = np.random.default_rng(seed)
    ch = 256 + heads * 64
    if grid:
        x = synth.f32_to_bf16_bits(rng.integers(-4, 5, (n, d_model)).astype(np.float32) / 4)
        w = synth.f32_to_bf16_bits(rng.integers(-4, 5, (ch, d_model)).astype(np.float32) / 8)
    else:
        x = synth.f32_to_bf16_bits(rng.standard_normal((n, d_model)).astype(np.float32))
        w = synth.f32_to_bf16_bits((rng.standard_normal((ch, d_model)) / np.sqrt(d_model)).astype(np.float32))
    # rows scattered over two sequences, positions in no particular order
    slots = rng.permutation(2 * capacity)[:n]
    seq, pos = (slots // capacity).astype(np.int32), (slots % capacity).astype(np.int32)
    gc = m.Cache(2, capacity, idx_heads=heads, idx_k_dtype=dtype)
    m.csa2_proj_append(gc, dev_u16(x), dev_u16(w), dev_i32(seq), dev_i32(pos))
    torch.cuda.synchronize()
    oc = O.OracleCache(2, capacity, idx_heads=heads, idx_k_dtype=dtype)
    O.project_and_append(oc, x, w, seq, pos)
    gidx = untile_idx(host(gc.idx_k), heads, oc.idx_k.dtype)
    got = (host(gc.kv_codes), host(gc.kv_scales), gidx)
    want = (oc.kv_codes, oc.kv_scales, oc.idx_k)
    if grid:
        return got, want
    # per row, in call order: the inputs and the row's bytes
    return (x, w), tuple(a[seq, pos] for a in got)


@pytest.mark.parametrize("heads,dtype", [(8, "fp8"), (4, "bf16")])
@pytest.mark.parametrize("n,d_model", [(1, 32), (100, 512), (200, 1056), (64, 4096), (257, 96),
                                       (300, 512), (1000, 1056), (600, 96), (1024, 4096),
                                       (1, 65536), (520, 65536)])
def test_proj_append_bit_exact_on_exact_sums(heads, dtype, n, d_model):
    announce(f"proj append heads={heads} idx={dtype} n={n} d={d_model}")
    got, want = _run(heads, dtype, n, d_model, seed=n + d_model)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)


@pytest.mark.parametrize("heads,dtype", [(8, "fp8"), (4, "bf16")])
@pytest.mark.parametrize("n,d_model", [(300, 2048), (40, 4096), (7, 1056), (700, 2080)])
def test_proj_append_random_inputs_per_element(heads, dtype, n, d_model):
    # every launch shape (below 256 tokens, from 256, from 512)
    announce(f"proj append random inputs heads={heads} idx={dtype} n={n} d={d_model}")
    (x, w), (codes, scales, idx) = _run(heads, dtype, n, d_model, grid=False, seed=11 + n)
    amb = check_projection_bytes(x, w, heads, dtype, codes, scales, idx)
    announce(f"  {amb} of {n * (256 + heads * 64)} values next to a bf16 rounding boundary")


def test_proj_append_bytes_do_not_depend_on_the_call():
    # 32 random rows projected alone (small-call tiles), at offsets 0, 5 and
    # 261 inside 300-row calls (64 x 64 tiles) and at offsets 0 and 600 inside
    # 700-row calls (128 x 128 tiles): identical bytes
    m = lib()
    rng = np.random.default_rng(7)
    d_model, heads = 2048, 8
    ch = 256 + heads * 64
    rows = synth.f32_to_bf16_bits(rng.standard_normal((32, d_model)).astype(np.float32))
    w = dev_u16(synth.f32_to_bf16_bits((rng.standard_normal((ch, d_model)) / np.sqrt(d_model)).astype(np.float32)))
    results = []
    for off, n in ((0, 32), (0, 300), (5, 300), (261, 300), (0, 700), (600, 700)):
        announce(f"proj append rows at offset {off} of a {n}-row call")
        x = synth.f32_to_bf16_bits(rng.standard_normal((n, d_model)).astype(np.float32))
        x[off:off + 32] = rows
        gc = m.Cache(1, 1024, idx_heads=heads, idx_k_dtype="fp8")
        m.csa2_proj_append(gc, dev_u16(x), w, dev_i32(np.zeros(n)), dev_i32(np.arange(n)))
        torch.cuda.synchronize()
        sl = slice(off, off + 32)
        results.append((host(gc.kv_codes)[0, sl], host(gc.kv_scales)[0, sl],
                        untile_idx(host(gc.idx_k), heads, np.uint8)[0, sl]))
    for r in results[1:]:
        for a, b in zip(results[0], r):
            assert np.array_equal(a, b)


def test_proj_append_empty_is_a_no_op():
    m = lib()
    gc = m.Cache(1, 64, idx_heads=8, idx_k_dtype="fp8")
    e = torch.empty((0, 64), dtype=torch.int16, device="cuda")
    w = torch.zeros((256 + 512, 64), dtype=torch.int16, device="cuda")
    z = torch.empty(0, dtype=torch.int32, device="cuda")
    m.csa2_proj_append(gc, e, w, z, z)
    torch.cuda.synchronize()
    assert int(host(gc.kv_codes).sum()) == 0
