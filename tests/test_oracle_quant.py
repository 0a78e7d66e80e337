"""Pins of the oracle's quantize-and-append: known-answer blocks, layout, invariants."""
import os

import numpy as np
import pytest

import synth
from oracle import csa2 as O
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _known_answers():
    out = []
    for line in open(os.path.join(GOLDEN, "fp4_block_known_answers.txt")):
        if line.startswith("#") or not line.strip():
            continue
        vals, sc, packed = [p.strip() for p in line.split("|")]
        out.append(([float(v) for v in vals.split()], int(sc, 16), bytes.fromhex(packed)))
    return out


@pytest.mark.parametrize("case", _known_answers(), ids=lambda c: f"scale{c[1]:02x}")
def test_known_answer_blocks(case):
    vals, sc, packed = case
    x = np.array(vals, np.float32)
    bits = synth.f32_to_bf16_bits(x)
    assert np.array_equal(synth.bf16_bits_to_f32(bits), x), "fixture values must be exact bf16"
    codes, scales = O.quantize_rows(bits[None, :])
    assert scales[0, 0] == sc
    assert bytes(codes[0]) == packed


def test_bytes_per_token_layout():
    want = {}
    for line in open(os.path.join(GOLDEN, "kv_bytes_per_token.txt")):
        if not line.startswith("#"):
            k, v = line.split()
            want[k] = int(v)
    c8 = O.OracleCache(1, 8, idx_heads=8, idx_k_dtype="fp8")
    c16 = O.OracleCache(1, 8, idx_heads=4, idx_k_dtype="bf16")
    assert c8.bytes_per_token()["main_kv"] == want["main_kv"]
    assert c8.bytes_per_token()["index_keys"] == want["index_keys_fp8_8x64"]
    assert c16.bytes_per_token()["index_keys"] == want["index_keys_bf16_4x64"]


def test_exactly_representable_rows_roundtrip():
    # Rows built as code * scale with a block amax of exactly 6*scale quantize back losslessly.
    rng = np.random.default_rng(1)
    for _ in range(50):
        sc = int(rng.integers(8, 0x70))
        s = float(F.E4M3_NONNEG[sc])
        codes = rng.integers(0, 16, 16)
        codes[rng.integers(0, 16)] = 7 | (8 * int(rng.integers(0, 2)))   # one +-6 sets amax
        x = F.e2m1_value(codes) * s
        bits = synth.f32_to_bf16_bits(x.astype(np.float32))
        assert np.array_equal(synth.bf16_bits_to_f32(bits), x.astype(np.float32))
        packed, scales = O.quantize_rows(bits[None])
        assert scales[0, 0] == sc
        back = O.dequantize_rows(packed, scales)[0]
        assert np.array_equal(back, x)


def test_dequant_error_bounded_and_exact_in_half_precision():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((256, 128)).astype(np.float32) * np.float32(3)
    bits = synth.f32_to_bf16_bits(x)
    xv = F.bf16_value(bits)
    packed, scales = O.quantize_rows(bits)
    y = O.dequantize_rows(packed, scales)
    s = np.repeat(F.e4m3_value(scales), 16, axis=1)
    # nearest E2M1 point: error at most half the widest gap (2 at the top) times the scale,
    # unless the block saturated its scale (not at these magnitudes)
    assert np.all(np.abs(y - xv) <= 1.0 * s + 1e-30)
    # Every dequantized value is exact in fp16 and bf16.
    assert np.array_equal(y.astype(np.float16).astype(np.float64), y)
    yb = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(y.astype(np.float32))).astype(np.float64)
    assert np.array_equal(yb, y)


def test_append_layout_and_chunking():
    wl = synth.workload("tiny_4k", context=64)
    seq = synth.gen_sequence(wl, 0)
    a = O.OracleCache(1, 64, idx_heads=4, idx_k_dtype="bf16")
    a.append(seq.k, seq.v, seq.ik, np.zeros(64, int), np.arange(64))
    b = O.OracleCache(1, 64, idx_heads=4, idx_k_dtype="bf16")
    for lo in range(0, 64, 16):   # chunked append = one-shot append (quantization is per row)
        b.append(seq.k[lo:lo + 16], seq.v[lo:lo + 16], seq.ik[lo:lo + 16],
                 np.zeros(16, int), np.arange(lo, lo + 16))
    assert np.array_equal(a.kv_codes, b.kv_codes) and np.array_equal(a.kv_scales, b.kv_scales)
    assert np.array_equal(a.idx_k, b.idx_k)
    # K occupies bytes 0..63 and scales 0..7; V the rest
    kc, ks = O.quantize_rows(seq.k)
    vc, vs = O.quantize_rows(seq.v)
    assert np.array_equal(a.kv_codes[0, :, :64], kc) and np.array_equal(a.kv_codes[0, :, 64:], vc)
    assert np.array_equal(a.kv_scales[0, :, :8], ks) and np.array_equal(a.kv_scales[0, :, 8:], vs)
    # fp8 index keys are the E4M3 cast of the bf16 values
    c = O.OracleCache(1, 64, idx_heads=4, idx_k_dtype="fp8")
    c.append(seq.k, seq.v, seq.ik, np.zeros(64, int), np.arange(64))
    assert np.array_equal(c.idx_k[0], F.e4m3_encode(F.bf16_value(seq.ik)))


def test_lazy_cache_and_tables_match_direct_quantization():
    wl = synth.workload("decode_64k_b32", context=96, batch=2)
    data = synth.gen_batch(wl)
    eager = O.OracleCache(2, 96)
    lazy = O.OracleCache(2, 96, lazy=True)
    for b in range(2):
        seq, pos = np.full(96, b), np.arange(96)
        eager.append(data.k[b], data.v[b], data.ik[b], seq, pos)
        lazy.append(data.k[b], data.v[b], data.ik[b], seq, pos)
    # index keys through the lookup table equal the encoder applied directly
    assert np.array_equal(eager.idx_k, F.e4m3_encode(F.bf16_value(data.ik)))
    assert np.array_equal(lazy.idx_k, eager.idx_k)
    assert np.array_equal(eager.index_key_values(1, np.arange(96)),
                          F.e4m3_value(eager.idx_k[1]).astype(np.float32))
    rows = np.array([5, 0, 95, 40])
    for b in range(2):
        ke, ve = eager.kv_values(b, rows)
        kl, vl = lazy.kv_values(b, rows)
        assert np.array_equal(ke, kl) and np.array_equal(ve, vl)
    # a later append to the same position wins in both
    newk = data.k[0, :1].copy() ^ np.uint16(0x8000)
    eager.append(newk, data.v[0, :1], None, [1], [40])
    lazy.append(newk, data.v[0, :1], None, [1], [40])
    assert np.array_equal(eager.kv_values(1, rows)[0], lazy.kv_values(1, rows)[0])
