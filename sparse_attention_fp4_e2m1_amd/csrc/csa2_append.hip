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
#include "csa2_kv_row.h"

namespace csa2 {
namespace {

// One wave per row (append_row).
__global__ void __launch_bounds__(256) kv_append_kernel(const AppendRows A) {
  const int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= A.n) return;
  append_row(A, row, threadIdx.x & (kWave - 1));
}

// The encoder-side projection fused into quantize-and-append (aiwiki "DeepSeek
// V4.1-Flash", section "Causal Encoder-Decoder": the decoder's global keys and
// values are projected from the final causal-encoder hidden states).  One
// workgroup computes a tile of 16 kRT tokens x 16 kCT kCG output channels of
// Y = X W^T on matrix cores (bf16 operands, fp32 accumulation).  Four waves
// per group of 16 kCT channels split the contraction and each holds the
// group's whole tile, so every operand fragment feeds kRT or kCT products;
// the partial tiles are summed in LDS in wave order, rounded to bf16 and
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

// The contraction is split over four waves in every launch shape: wave ks of
// a channel group takes k-steps ks, ks + 4, ks + 8, ... (32 channels of
// d_model each) in order, and the four partial tiles are added in wave order,
// ((p0 + p1) + p2) + p3.  So the fp32 order of every output element depends on
// d_model only, not on the call's token count or the tile shape, and a row
// projects to the same bytes whichever call carries it.
constexpr int kProjSplit = 4;

template <int kRT, int kCT, int kCG>   // 16 kRT rows x 16 kCT columns per wave, kCG column groups
__global__ void __launch_bounds__(64 * kProjSplit * kCG) proj_append_kernel(
    uint8_t *__restrict__ kv_codes, uint8_t *__restrict__ kv_scales, uint8_t *__restrict__ idx_k,
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int32_t d_model,
    const int32_t *__restrict__ seq, const int32_t *__restrict__ pos, int32_t n,
    int32_t capacity, int32_t H, int32_t esz) {
  constexpr int kW = kProjSplit * kCG;
  constexpr int kRows = 16 * kRT, kCols = 16 * kCT * kCG, kPitch = kCols + 4;
  __shared__ float tile[kRows * kPitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ks = wave % kProjSplit;   // contraction slice
  const int cg = wave / kProjSplit;   // column group
  const int l16 = lane & 15;
  const int kg = lane >> 4;
  const int r0 = blockIdx.x * kRows;
  const int c0 = blockIdx.y * kCols + cg * 16 * kCT;
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
  for (int k0 = 32 * ks; k0 < d_model; k0 += 32 * kProjSplit) {
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
  // sum of the four partial tiles of each column group, slice 0 first
  for (int sv = 0; sv < kProjSplit; ++sv) {
    if (ks == sv) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float *t = tile + (16 * rt + 4 * kg + i) * kPitch + cg * 16 * kCT + 16 * ct + l16;
            *t = sv == 0 ? acc[rt][ct][i] : *t + acc[rt][ct][i];
          }
    }
    __syncthreads();
  }

  // (token, 16-channel block): K or V block -> E4M3 scale and E2M1 codes;
  // index-key block -> two groups of 8 channels, bf16 or E4M3
  const int64_t seq_bytes = (int64_t)capacity * H * 64 * esz;
  constexpr int kBlocks = kCols / 16;   // 16-channel blocks per row of the tile
  for (int item = tid; item < kRows * kBlocks; item += 64 * kW) {
    const int r = item / kBlocks, j = item % kBlocks;
    const int row = r0 + r;
    if (row >= n) continue;
    const float *src = tile + r * kPitch + 16 * j;
    const int c = blockIdx.y * kCols + 16 * j;
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
  // SIMD); below 256 tokens 16 x 64 tiles of two column groups (eight waves),
  // which give more workgroups.  Both split the contraction over four waves
  // the same way.  Measured at d_model 4096: 64 x 64 beats 64 x 128 by 1.4x at
  // 4096 tokens.
  const int cols = 256 + 64 * c.idx_heads;
  const int32_t esz = c.idx_k_dtype == CSA2_FP8_E4M3 ? 1 : 2;
  uint8_t *ik = static_cast<uint8_t *>(c.idx_k);
  if (n >= 256) {
    hipLaunchKernelGGL((proj_append_kernel<4, 4, 1>), dim3((n + 63) / 64, cols / 64), dim3(256), 0,
                       stream, c.kv_codes, c.kv_scales, ik, x, w, d_model, seq, pos, n,
                       c.capacity, c.idx_heads, esz);
  } else {
    hipLaunchKernelGGL((proj_append_kernel<1, 2, 2>), dim3((n + 15) / 16, cols / 64), dim3(512), 0,
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

AppendRows append_rows(const csa2_cache &c, const uint16_t *k, const uint16_t *v,
                       const uint16_t *idx_in, const int32_t *seq, const int32_t *pos, int32_t n) {
  return AppendRows{static_cast<uint8_t *>(c.kv_codes), static_cast<uint8_t *>(c.kv_scales),
                    c.idx_k, k, v, idx_in, seq, pos, n, c.capacity, c.idx_heads * c.idx_dim,
                    (int32_t)(c.idx_k_dtype == CSA2_FP8_E4M3)};
}

hipError_t launch_kv_append(const csa2_cache &c, const uint16_t *k, const uint16_t *v,
                            const uint16_t *idx_in, const int32_t *seq, const int32_t *pos,
                            int32_t n, hipStream_t stream) {
  const int rows_per_block = 4;
  dim3 grid((n + rows_per_block - 1) / rows_per_block);
  hipLaunchKernelGGL(kv_append_kernel, grid, dim3(rows_per_block * kWave), 0, stream,
                     append_rows(c, k, v, idx_in, seq, pos, n));
  return hipGetLastError();
}

}  // namespace csa2
