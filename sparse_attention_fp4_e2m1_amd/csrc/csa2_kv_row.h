// Quantize-and-append of one cache row (device code shared by the append
// kernel and the index scorer's fused append).
//
// Model card "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression",
// Introduction, CSA2 paragraph: the main KV is cached in FP4, E2M1 values with
// one E4M3 scale per 16 channels.  Rounding rules (the pages give none):
// scale = E4M3 nearest amax/6, element = E2M1 nearest x/scale, ties to even,
// saturating, sign kept; index keys stored as bf16 or cast to E4M3 (nearest
// even, saturating at 448, sign kept).
#pragma once

#include "csa2_internal.h"

namespace csa2 {

// E2M1 magnitude code of |x| under decoded scale s > 0: the count of midpoints
// (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) * s below |x|; a value exactly on a
// midpoint moves up only when the upper neighbour's code is even.  Every
// midpoint * s is exact in fp32 (<= 3 significant bits times <= 4).
static __device__ __forceinline__ uint32_t e2m1_mag(float ax, float s) {
  uint32_t c = 0;
  c += (ax > 0.25f * s);
  c += (ax >= 0.75f * s);   // tie -> code 2 (even)
  c += (ax > 1.25f * s);
  c += (ax >= 1.75f * s);   // tie -> code 4
  c += (ax > 2.5f * s);
  c += (ax >= 3.5f * s);    // tie -> code 6
  c += (ax > 5.0f * s);
  return c;
}

// One 16-channel block: E4M3 scale code (returned) and the 16 E2M1 codes,
// channel i in nibble i of (lo, hi).
static __device__ __forceinline__ uint32_t quant_block16(const float (&x)[16], uint32_t &lo,
                                                  uint32_t &hi) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  // amax is a bf16 value; the correctly rounded quotient never lands on an
  // E4M3 midpoint unless the exact quotient does, so rounding it to E4M3
  // equals rounding the exact amax/6.
  const uint32_t sc = e4m3_from_f32_nonneg(amax / 6.0f);
  const float s = e4m3_to_f32(sc);
  lo = 0;
  hi = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t c = s > 0.0f ? e2m1_mag(fabsf(x[i]), s) : 0u;
    c |= (__float_as_uint(x[i]) >> 28) & 8u;   // sign bit, -0 kept
    if (i < 8) lo |= c << (4 * i);
    else hi |= c << (4 * (i - 8));
  }
  return sc;
}

// Eight consecutive index-key channels (bf16 bits in a) of head h at
// position p into the tiled layout (tiles of 64/H positions;
// [chunk][position-in-tile][head][16 B]), as bf16 or cast to E4M3.
static __device__ __forceinline__ void store_idx8(uint8_t *seq_idx, int H, int esz, int64_t p, int h,
                                           int ch, uint4 a) {
  const int T = kWave / H;
  uint8_t *tile = seq_idx + (p / T) * (64 * 64 * esz);
  const int byte = ch * esz;                         // byte of channel ch within the head
  uint8_t *dst = tile + (byte / 16) * 1024 + ((p % T) * H + h) * 16 + byte % 16;
  if (esz == 1) {
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
    uint32_t out[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t hb = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
      const float f = __uint_as_float(hb << 16);
      const uint32_t c = e4m3_from_f32_nonneg(fabsf(f)) | ((hb >> 8) & 0x80u);
      out[i >> 2] |= c << (8 * (i & 3));
    }
    *reinterpret_cast<uint2 *>(dst) = make_uint2(out[0], out[1]);
  } else {
    *reinterpret_cast<uint4 *>(dst) = a;
  }
}

// Row `row` by one wave.  Every load of the row is issued first, with no
// branch around it (a load under a lane-dependent branch is waited for before
// the branch closes), so a decode step's handful of rows costs one memory
// round trip: lanes 0..15 quantize one 16-channel block each (K blocks 0..7,
// then V), and every lane stores eight channels of the index keys.
static __device__ __forceinline__ void append_row(const AppendRows &A, int row, int lane) {
  const int32_t sq = A.seq[row];
  const int32_t ps = A.pos[row];
  // K / V block (lanes 16..63 load lane % 16's block again, unused)
  const bool is_v = (lane & 8) != 0;
  const int blk = lane & 7;
  const uint4 *s4 =
      reinterpret_cast<const uint4 *>((is_v ? A.v : A.k) + (int64_t)row * 128 + blk * 16);
  const uint4 a = s4[0], b = s4[1];
  // index keys: 8 channels per lane (lanes past the row's H * 64 channels
  // load the last group again, unused; without index keys the row's K
  // channels stand in, unused)
  const int e = min(lane * 8, A.idx_elems - 8);
  const uint16_t *isrc = A.idx_in != nullptr ? A.idx_in + (int64_t)row * A.idx_elems + e
                                             : A.k + (int64_t)row * 128;
  const uint4 ik = *reinterpret_cast<const uint4 *>(isrc);
  const int64_t slot = (int64_t)sq * A.capacity + ps;

  if (lane < 16) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float x[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    uint32_t lo, hi;
    const uint32_t sc = quant_block16(x, lo, hi);
    uint2 *dst = reinterpret_cast<uint2 *>(A.kv_codes + slot * 128 + (is_v ? 64 : 0) + blk * 8);
    *dst = make_uint2(lo, hi);
    A.kv_scales[slot * 16 + (is_v ? 8 : 0) + blk] = (uint8_t)sc;
  }

  if (A.idx_in != nullptr && lane * 8 < A.idx_elems) {
    const int H = A.idx_elems / 64;
    const int esz = A.idx_fp8 ? 1 : 2;
    const int64_t seq_bytes = (int64_t)A.capacity * A.idx_elems * esz;
    uint8_t *seq_idx = static_cast<uint8_t *>(A.idx_k) + (int64_t)sq * seq_bytes;
    store_idx8(seq_idx, H, esz, ps, e / 64, e % 64, ik);
  }
}

// An index key element as the cache holds it, as a float: bf16 bits b cast
// to E4M3 (fp8) or kept.
static __device__ __forceinline__ float idx_key_value(uint32_t b, bool fp8) {
  const float f = __uint_as_float(b << 16);
  if (!fp8) return f;
  return e4m3_to_f32(e4m3_from_f32_nonneg(fabsf(f)) | ((b >> 8) & 0x80u));
}

}  // namespace csa2
