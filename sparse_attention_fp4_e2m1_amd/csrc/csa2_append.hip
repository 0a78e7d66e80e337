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

// One 16-channel block: E4M3 scale code (returned) and the 16 E2M1 codes,
// channel i in nibble i of (lo, hi).
__device__ __forceinline__ uint32_t quant_block16(const float (&x)[16], uint32_t &lo,
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
__device__ __forceinline__ void store_idx8(uint8_t *seq_idx, int H, int esz, int64_t p, int h,
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
    uint32_t lo, hi;
    const uint32_t sc = quant_block16(x, lo, hi);
    uint2 *dst = reinterpret_cast<uint2 *>(kv_codes + slot * 128 + (is_v ? 64 : 0) + blk * 8);
    *dst = make_uint2(lo, hi);
    kv_scales[slot * 16 + (is_v ? 8 : 0) + blk] = (uint8_t)sc;
  }

  if (idx_in != nullptr) {
    // idx_elems = H * 64 bf16 values: 8 per lane-step
    const int H = idx_elems / 64;
    const int esz = idx_fp8 ? 1 : 2;
    const int64_t seq_bytes = (int64_t)capacity * idx_elems * esz;
    uint8_t *seq_idx = static_cast<uint8_t *>(idx_k) + (int64_t)seq[row] * seq_bytes;
    const uint16_t *src = idx_in + (int64_t)row * idx_elems;
    for (int e = lane * 8; e < idx_elems; e += kWave * 8)
      store_idx8(seq_idx, H, esz, pos[row], e / 64, e % 64,
                 *reinterpret_cast<const uint4 *>(src + e));
  }
}

// The encoder-side projection fused into quantize-and-append (aiwiki "DeepSeek
// V4.1-Flash", section "Causal Encoder-Decoder": the decoder's global keys and
// values are projected from the final causal-encoder hidden states).  One
// workgroup computes a tile of 16 kRT tokens x 16 kCT output channels of
// Y = X W^T on matrix cores (bf16 operands, fp32 accumulation).  Its kW
// waves split the contraction (wave w takes k-steps w, w + kW, ...) and each
// holds the whole tile, so every operand fragment feeds kRT or kCT products;
// the kW partial tiles are summed in LDS in wave order, rounded to bf16 and
// quantized exactly as kv_append_kernel does.  Output channels: K 0..127,
// V 128..255, index keys 256.. (head-major).
// Operand fragments of v_mfma_f32_16x16x32_bf16: lane l supplies row l % 16
// and contraction indices k0 + 8 (l / 16) .. +7 of both X and W (16 B each,
// straight from memory); the result lane holds rows 4 (l / 16) + 0..3 of
// column l % 16.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int kRT, int kCT, int kW>
__global__ void __launch_bounds__(64 * kW) proj_append_kernel(
    uint8_t *__restrict__ kv_codes, uint8_t *__restrict__ kv_scales, uint8_t *__restrict__ idx_k,
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int32_t d_model,
    const int32_t *__restrict__ seq, const int32_t *__restrict__ pos, int32_t n,
    int32_t capacity, int32_t H, int32_t esz) {
  constexpr int kRows = 16 * kRT, kCols = 16 * kCT, kPitch = kCols + 4;
  __shared__ float tile[kRows * kPitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int kg = lane >> 4;
  const int r0 = blockIdx.x * kRows;
  const int c0 = blockIdx.y * kCols;
  const uint16_t *xa[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)   // rows past n read row n - 1, never stored
    xa[rt] = x + (int64_t)min(r0 + 16 * rt + l16, n - 1) * d_model + 8 * kg;
  const uint16_t *wb = w + (int64_t)(c0 + l16) * d_model + 8 * kg;
  const int64_t tstride = (int64_t)16 * d_model;

  f32x4 acc[kRT][kCT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) acc[rt][ct] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 2
  for (int k0 = 32 * wave; k0 < d_model; k0 += 32 * kW) {
    bf16x8 a[kRT];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
      a[rt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(xa[rt] + k0));
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      const bf16x8 b =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(wb + ct * tstride + k0));
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rt], b, acc[rt][ct], 0, 0, 0);
    }
  }
  // sum of the four partial tiles, wave 0 first
  for (int wv = 0; wv < kW; ++wv) {
    if (wave == wv) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float *t = tile + (16 * rt + 4 * kg + i) * kPitch + 16 * ct + l16;
            *t = wv == 0 ? acc[rt][ct][i] : *t + acc[rt][ct][i];
          }
    }
    __syncthreads();
  }

  // (token, 16-channel block): K or V block -> E4M3 scale and E2M1 codes;
  // index-key block -> two groups of 8 channels, bf16 or E4M3
  const int64_t seq_bytes = (int64_t)capacity * H * 64 * esz;
  for (int item = tid; item < kRows * kCT; item += 64 * kW) {
    const int r = item / kCT, j = item % kCT;
    const int row = r0 + r;
    if (row >= n) continue;
    const float *src = tile + r * kPitch + 16 * j;
    const int c = c0 + 16 * j;
    if (c < 256) {
      float xv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) xv[i] = __uint_as_float(bf16_rne(src[i]) << 16);
      uint32_t lo, hi;
      const uint32_t sc = quant_block16(xv, lo, hi);
      const int64_t slot = (int64_t)seq[row] * capacity + pos[row];
      const int half = c >> 7, blk = (c & 127) >> 4;
      *reinterpret_cast<uint2 *>(kv_codes + slot * 128 + 64 * half + 8 * blk) = make_uint2(lo, hi);
      kv_scales[slot * 16 + 8 * half + blk] = (uint8_t)sc;
    } else {
      uint8_t *seq_idx = idx_k + (int64_t)seq[row] * seq_bytes;
      const int ci = c - 256;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        uint32_t q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          q[i] = bf16_rne(src[8 * g + 2 * i]) | (bf16_rne(src[8 * g + 2 * i + 1]) << 16);
        store_idx8(seq_idx, H, esz, pos[row], ci / 64, ci % 64 + 8 * g,
                   make_uint4(q[0], q[1], q[2], q[3]));
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

hipError_t launch_proj_append(const csa2_cache &c, const uint16_t *x, int32_t d_model,
                              const uint16_t *w, const int32_t *seq, const int32_t *pos,
                              int32_t n, hipStream_t stream) {
  // 64 x 64 tiles, four waves (a wave holds 16 accumulators: three waves per
  // SIMD); below 256 tokens 16 x 64 tiles and eight waves, which give more
  // workgroups and shorter contraction loops.  Measured at d_model 4096:
  // 64 x 64 beats 64 x 128 by 1.4x at 4096 tokens; at 32 tokens the small
  // tiles take 21.9 us against 25.4 us for 32 x 64 with four waves.
  const int cols = 256 + 64 * c.idx_heads;
  const int32_t esz = c.idx_k_dtype == CSA2_FP8_E4M3 ? 1 : 2;
  uint8_t *ik = static_cast<uint8_t *>(c.idx_k);
  if (n >= 256) {
    hipLaunchKernelGGL((proj_append_kernel<4, 4, 4>), dim3((n + 63) / 64, cols / 64), dim3(256), 0,
                       stream, c.kv_codes, c.kv_scales, ik, x, w, d_model, seq, pos, n,
                       c.capacity, c.idx_heads, esz);
  } else {
    hipLaunchKernelGGL((proj_append_kernel<1, 4, 8>), dim3((n + 15) / 16, cols / 64), dim3(512), 0,
                       stream, c.kv_codes, c.kv_scales, ik, x, w, d_model, seq, pos, n,
                       c.capacity, c.idx_heads, esz);
  }
  return hipGetLastError();
}

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
