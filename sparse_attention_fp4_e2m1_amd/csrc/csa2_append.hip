// Quantize-and-append into the FP4 main-KV cache and the index-key cache.
//
// Model card "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression",
// Introduction, CSA2 paragraph: the main KV is cached in FP4, E2M1 values with
// one E4M3 scale per 16 channels.  aiwiki "DeepSeek V4.1-Flash", "KV-cache
// formats and bounded replay": the runtime global KV stays in accelerator
// memory.  Rounding rules (the pages give none): scale = E4M3 nearest amax/6,
// element = E2M1 nearest x/scale, ties to even, saturating, sign kept.
//
// One wave per appended row.  Lanes 0..15 each own one 16-channel block
// (8 K blocks, then 8 V blocks): 32 B of bf16 in, 8 B of codes + 1 scale byte
// out.  All 64 lanes then move the row's index keys (bf16 copy or E4M3 cast).
//
// aiwiki "DeepSeek V4.1-Flash", "Compressed Sparse Attention 2" and "KV-cache
// formats and bounded replay": each layer's own local sliding-window K and V
// are kept in FP8; local_append_kernel casts them to E4M3 into a ring of
// window slots per sequence.
#include "csa2_internal.h"

namespace csa2 {
namespace {

// E2M1 magnitude code of |x| under decoded scale s > 0: the count of midpoints
// (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) * s below |x|; a value exactly on a
// midpoint moves up only when the upper neighbour's code is even.  Every
// midpoint * s is exact in fp32 (<= 3 significant bits times <= 4).
__device__ __forceinline__ uint32_t e2m1_mag(float ax, float s) {
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

__global__ void __launch_bounds__(256) kv_append_kernel(
    uint8_t *__restrict__ kv_codes, uint8_t *__restrict__ kv_scales, void *__restrict__ idx_k,
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const uint16_t *__restrict__ idx_in, const int32_t *__restrict__ seq,
    const int32_t *__restrict__ pos, int32_t n, int32_t capacity, int32_t idx_elems,
    int32_t idx_fp8) {
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= n) return;
  const int64_t slot = (int64_t)seq[row] * capacity + pos[row];

  if (lane < 16) {
    const bool is_v = lane >= 8;
    const int blk = lane & 7;
    const uint16_t *src = (is_v ? v : k) + (int64_t)row * 128 + blk * 16;
    const uint4 *s4 = reinterpret_cast<const uint4 *>(src);
    uint4 a = s4[0], b = s4[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float x[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
    // amax is a bf16 value; the correctly rounded quotient never lands on an
    // E4M3 midpoint unless the exact quotient does, so rounding it to E4M3
    // equals rounding the exact amax/6.
    const uint32_t sc = e4m3_from_f32_nonneg(amax / 6.0f);
    const float s = e4m3_to_f32(sc);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t c = s > 0.0f ? e2m1_mag(fabsf(x[i]), s) : 0u;
      c |= (__float_as_uint(x[i]) >> 28) & 8u;   // sign bit, -0 kept
      if (i < 8) lo |= c << (4 * i);
      else hi |= c << (4 * (i - 8));
    }
    uint2 *dst = reinterpret_cast<uint2 *>(kv_codes + slot * 128 + (is_v ? 64 : 0) + blk * 8);
    *dst = make_uint2(lo, hi);
    kv_scales[slot * 16 + (is_v ? 8 : 0) + blk] = (uint8_t)sc;
  }

  if (idx_in != nullptr) {
    // idx_elems = H * 64 bf16 values: 8 per lane-step, stored in the tiled
    // layout (tiles of 64/H positions; [chunk][position-in-tile][head][16 B]).
    const int H = idx_elems / 64;
    const int T = kWave / H;
    const int esz = idx_fp8 ? 1 : 2;
    const int64_t p = pos[row];
    const int64_t seq_bytes = (int64_t)capacity * idx_elems * esz;
    uint8_t *tile = static_cast<uint8_t *>(idx_k) + (int64_t)seq[row] * seq_bytes +
                    (p / T) * (64 * 64 * esz);
    const int64_t slot16 = (p % T) * H;
    const uint16_t *src = idx_in + (int64_t)row * idx_elems;
    for (int e = lane * 8; e < idx_elems; e += kWave * 8) {
      const uint4 a = *reinterpret_cast<const uint4 *>(src + e);
      const int h = e / 64;
      const int ch = e % 64;
      const int byte = ch * esz;                         // byte of channel ch within the head
      uint8_t *dst = tile + (byte / 16) * 1024 + (slot16 + h) * 16 + byte % 16;
      if (idx_fp8) {
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
  }
}

// Local window rows: E4M3 codes of every bf16 element (no scale), into slot
// pos % window; one wave per row, two elements per lane per tensor.
__global__ void __launch_bounds__(256) local_append_kernel(
    uint8_t *__restrict__ lk, uint8_t *__restrict__ lv, int32_t *__restrict__ lpos,
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ seq, const int32_t *__restrict__ pos, int32_t n, int32_t window) {
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= n) return;
  const int32_t p = pos[row];
  const int64_t slot = (int64_t)seq[row] * window + p % window;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint16_t *src = (t == 0 ? k : v) + (int64_t)row * 128 + 2 * lane;
    const uint32_t w = *reinterpret_cast<const uint32_t *>(src);
    uint32_t codes = 0u;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t hb = (w >> (16 * i)) & 0xFFFFu;
      const float f = __uint_as_float(hb << 16);
      codes |= (e4m3_from_f32_nonneg(fabsf(f)) | ((hb >> 8) & 0x80u)) << (8 * i);
    }
    uint8_t *dst = (t == 0 ? lk : lv) + slot * 128 + 2 * lane;
    *reinterpret_cast<uint16_t *>(dst) = (uint16_t)codes;
  }
  if (lane == 0) lpos[slot] = p;
}

// Empties one sequence's window: every slot's position becomes -1.
__global__ void __launch_bounds__(256) local_clear_kernel(int32_t *__restrict__ lpos, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) lpos[i] = -1;
}

}  // namespace

hipError_t launch_local_clear(const csa2_local_cache &c, int32_t seq, hipStream_t stream) {
  hipLaunchKernelGGL(local_clear_kernel, dim3((c.window + 255) / 256), dim3(256), 0, stream,
                     c.pos + (int64_t)seq * c.window, c.window);
  return hipGetLastError();
}

hipError_t launch_local_append(const csa2_local_cache &c, const uint16_t *k, const uint16_t *v,
                               const int32_t *seq, const int32_t *pos, int32_t n,
                               hipStream_t stream) {
  const int rows_per_block = 4;
  hipLaunchKernelGGL(local_append_kernel, dim3((n + rows_per_block - 1) / rows_per_block),
                     dim3(rows_per_block * kWave), 0, stream, c.k, c.v, c.pos, k, v, seq, pos, n,
                     c.window);
  return hipGetLastError();
}

hipError_t launch_kv_append(const csa2_cache &c, const uint16_t *k, const uint16_t *v,
                            const uint16_t *idx_in, const int32_t *seq, const int32_t *pos,
                            int32_t n, hipStream_t stream) {
  const int rows_per_block = 4;
  dim3 grid((n + rows_per_block - 1) / rows_per_block);
  const int32_t idx_elems = c.idx_heads * c.idx_dim;
  hipLaunchKernelGGL(kv_append_kernel, grid, dim3(rows_per_block * kWave), 0, stream, c.kv_codes,
                     c.kv_scales, c.idx_k, k, v, idx_in, seq, pos, n, c.capacity, idx_elems,
                     (int32_t)(c.idx_k_dtype == CSA2_FP8_E4M3));
  return hipGetLastError();
}

}  // namespace csa2
