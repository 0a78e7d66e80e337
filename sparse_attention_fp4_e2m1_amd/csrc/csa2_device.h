// Device helpers shared by the CSA2 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// OCP E4M3FN code -> float (exact).  0x7F/0xFF never reach here (finite data).
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  uint32_t e = (code >> 3) & 15u;
  uint32_t m = code & 7u;
  float mag = e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (code & 0x80u) ? -mag : mag;
}

// Non-negative finite float -> E4M3 code, round to nearest even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_from_f32_nonneg(float y) {
  if (!(y < 448.0f)) return 0x7Eu;                     // saturate (also y == 448)
  if (y < 0x1p-6f) {                                    // subnormal range: multiples of 2^-9
    return (uint32_t)__builtin_rintf(y * 512.0f);      // exact scaling; rint = ties to even
  }
  uint32_t u = __float_as_uint(y);
  // keep 3 mantissa bits: round the low 20 bits to nearest even (carry may bump the exponent)
  uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;
  uint32_t e = (r >> 3) - 120u;                         // rebias 127 -> 7
  uint32_t code = (e << 3) | (r & 7u);
  return code > 0x7Eu ? 0x7Eu : code;
}

// Byte offset, within one sequence, of the 16-B chunk `chunk` of head h of
// position p in the tiled index-key layout: tiles of 64/H positions, each
// tile [chunk][position-in-tile][head][16 B].  esz = bytes per element.
template <int H, int kEsz>
__device__ __forceinline__ int64_t idx_chunk_offset(int64_t p, int h, int chunk) {
  constexpr int T = kWave / H;
  return (p / T) * (64 * 64 * kEsz) + chunk * 1024 + ((p % T) * H + h) * 16;
}

// Order-preserving key of an fp32 score; -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ uint32_t shfl_xor_u(uint32_t v, int mask) {
  return (uint32_t)__shfl_xor((int)v, mask, kWave);
}

// x + (x of the lane selected by the DPP control kCtrl); lanes without a
// source, or in rows outside kRowMask, add 0.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_add(uint32_t x) {
  return x + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, kRowMask, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes of a wave, in DPP moves: shifts by
// 1, 2, 4, 8 within each row of 16 lanes, then row 0's total into row 1 and
// row 2's into row 3 (row_bcast:15), then rows 0-1's total into rows 2-3
// (row_bcast:31).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v = dpp_add<0x111, 0xF>(v);   // row_shr:1
  v = dpp_add<0x112, 0xF>(v);   // row_shr:2
  v = dpp_add<0x114, 0xF>(v);   // row_shr:4
  v = dpp_add<0x118, 0xF>(v);   // row_shr:8
  v = dpp_add<0x142, 0xA>(v);   // row_bcast:15 into rows 1, 3
  v = dpp_add<0x143, 0xC>(v);   // row_bcast:31 into rows 2, 3
  return v;
}

// Exclusive prefix sum over the block; `scratch` holds >= blockDim/64 + 1 words.
// Returns the exclusive prefix, writes the block total.  Two barriers; every
// thread adds the wave totals before its own (at most 16).
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *scratch,
                                                         uint32_t &total) {
  constexpr int kMaxWaves = 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  const uint32_t inc = wave_inclusive_scan(v);
  __syncthreads();   // scratch free: readers of a previous scan are done
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kMaxWaves; ++w) {
    if (w < nwaves) {
      const uint32_t t = scratch[w];
      all += t;
      before += w < wave ? t : 0u;
    }
  }
  total = all;
  return before + inc - v;
}

}  // namespace csa2
