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
#include <type_traits>

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

// One fp32 order for every launch shape: the T = d_model / 32 k-steps (32
// channels of d_model each) fall into four contiguous quarters, quarter s
// being k-steps [proj_bound(T, s), proj_bound(T, s + 1)) -- whole groups of
// four k-steps, G = ceil(T / 4) groups split as evenly as that allows; each
// quarter is one chain of matrix-core products in k-step order from 0, and
// the four partial sums are added as ((p0 + p1) + p2) + p3.  So every output
// element depends on d_model only, not on the call's token count or the tile
// shape, and a row projects to the same bytes whichever call carries it.
constexpr int kProjSplit = 4;
__device__ __forceinline__ int proj_bound(int T, int s) {
  return min(T, 4 * ((s * ((T + 3) / 4)) >> 2));
}

// The epilogue of one (token, 16-channel block) of fp32 sums src[0..15]:
// rounded to bf16, then a K or V block -> E4M3 scale and E2M1 codes, an
// index-key block -> two groups of 8 channels, bf16 or E4M3.
__device__ __forceinline__ void proj_store_block(const float *src, int row, int c,
                                                 uint8_t *kv_codes, uint8_t *kv_scales,
                                                 uint8_t *idx_k, const int32_t *seq,
                                                 const int32_t *pos, int32_t capacity, int32_t H,
                                                 int32_t esz) {
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
    const int64_t seq_bytes = (int64_t)capacity * H * 64 * esz;
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

// 16 kRT rows x 16 kCT columns per wave, kCG column groups; kUnroll k-steps per loop trip
template <int kRT, int kCT, int kCG, int kUnroll>
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int T = d_model / 32;
  const int t_end = proj_bound(T, ks + 1);
  // one k-step: loads (into a, b) and products, in k order
  auto load = [&](int t, bf16x8 (&a)[kRT], bf16x8 (&b)[kCT]) {
    const int k0 = 32 * t;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
      a[rt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(xa[rt] + k0));
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct)
      b[ct] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(wb + ct * tstride + k0));
  };
  auto mul = [&](const bf16x8 (&a)[kRT], const bf16x8 (&b)[kCT]) {
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rt], b[ct], acc[rt][ct], 0, 0, 0);
  };
  // kUnroll k-steps per trip, all their loads first, so that they are in
  // flight together (a wave's chain is a row of dependent round trips
  // otherwise); the products still run in k order
  int t = proj_bound(T, ks);
  for (; t + kUnroll <= t_end; t += kUnroll) {
    bf16x8 a[kUnroll][kRT], b[kUnroll][kCT];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) load(t + u, a[u], b[u]);
    __builtin_amdgcn_sched_barrier(0);   // the compiler would interleave them again
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) mul(a[u], b[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (; t < t_end; ++t) {
    bf16x8 a[kRT], b[kCT];
    load(t, a, b);
    mul(a, b);
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

  constexpr int kBlocks = kCols / 16;   // 16-channel blocks per row of the tile
  for (int item = tid; item < kRows * kBlocks; item += 64 * kW) {
    const int r = item / kBlocks, j = item % kBlocks;
    const int row = r0 + r;
    if (row >= n) continue;
    proj_store_block(tile + r * kPitch + 16 * j, row, blockIdx.y * kCols + 16 * j, kv_codes,
                     kv_scales, idx_k, seq, pos, capacity, H, esz);
  }
}

// Large calls: tiles of 128 tokens x kBN channels (96 where the channel count
// allows it: 8 x 32 workgroups fill 256 CUs at 4096 tokens; else 128), four
// waves in 2 x 2, each with 64 x kBN / 2 of the tile (products of 16 x 16,
// same operand layout as above).  Operands go from global memory straight
// into LDS, 128 contraction channels (four k-steps) per stage: a stage holds
// 128 token rows and then kBN weight rows of 256 B, and 16-B chunk c of row r
// sits in slot c ^ (r % 16), so that a fragment read (16 consecutive rows,
// one chunk) hits 16 distinct slots.  Two stages alternate; the next stage's
// loads are spread over the current stage's k-steps, and each k-step's
// fragments are read from LDS while the previous k-step's products run.
// Each wave runs the four contraction quarters one after another, each as
// its own chain (P), and adds them up in order into S (from -0, which adds
// exactly): the arithmetic of the four-wave split above.  Quarters start at
// stage starts.  Workgroup b runs on XCD b % 8; the column tiles of a row
// tile go to one XCD, so that its L2 serves their shared token rows.
constexpr int kPT = 128;                          // tile rows (tokens)
constexpr int kPK = 128;                          // contraction channels per stage
constexpr int kPKSteps = kPK / 32;                // k-steps per stage
constexpr int kProjTileMin = 512;                 // tokens from which calls take these tiles

template <int kBN>   // tile columns (channels): 96 or 128
__global__ void __launch_bounds__(256) proj_tile_kernel(
    uint8_t *__restrict__ kv_codes, uint8_t *__restrict__ kv_scales, uint8_t *__restrict__ idx_k,
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int32_t d_model,
    const int32_t *__restrict__ seq, const int32_t *__restrict__ pos, int32_t n,
    int32_t capacity, int32_t H, int32_t esz, int32_t nrt, int32_t nct) {
  constexpr int kWN = kBN / 2;                            // columns per wave
  constexpr int kCT = kWN / 16;                           // 16-column tiles per wave
  constexpr int kPStageBytes = (kPT + kBN) * kPK * 2;     // 56 or 64 KB
  constexpr int kPLoads = kPStageBytes / 16 / 256;        // 16-B pieces per thread per stage
  constexpr int kPPitch = kBN + 4;                        // epilogue: fp32 rows (64 at a time)
  static_assert(kBN % 32 == 0 && kPStageBytes % 4096 == 0, "tile shape");
  static_assert(kPLoads <= 4 * kPKSteps, "a stage's pieces fit the k-steps' issue slots");
  static_assert(64 * kPPitch * 4 <= kPStageBytes, "the epilogue's rows fit one stage");
  // separate LDS objects, so that reads of one stage never wait on the loads
  // into the other
  __shared__ __attribute__((aligned(16))) uint8_t stageA[kPStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stageB[kPStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, kg = lane >> 4;
  const int m8 = blockIdx.x >> 3;
  const int rt = (m8 / nct) * 8 + (blockIdx.x & 7), ct = m8 % nct;
  if (rt >= nrt) return;   // the grid's row tiles are rounded up to a multiple of 8
  const int r0 = rt * kPT, c0 = ct * kBN;
  const int T = d_model / 32;                 // k-steps
  const int nst = (d_model + kPK - 1) / kPK;  // stages (the last one may hold fewer k-steps)

  // Piece k of thread tid is piece k * 256 + tid of the stage, at LDS byte
  // 16 (k * 256 + tid): row 16 k + tid / 16 (128 token rows, then weight rows),
  // slot tid % 16, holding chunk (tid % 16) ^ ((tid / 16) % 16) of the row.
  const int prow = tid >> 4;
  const int pchunk = (tid & 15) ^ (prow & 15);
  const bool full_rows = r0 + kPT <= n;
  // piece k of stage st into dst; whole: the stage lies inside the contraction
  auto dma = [&](auto whole, uint8_t *dst, int st, int k) {
    if (!decltype(whole)::value && kPK * st + 8 * pchunk >= d_model) return;   // past the end
    const uint16_t *g;
    if (k < kPT / 16) {
      const int row = r0 + 16 * k + prow;
      g = x + (int64_t)(full_rows ? row : min(row, n - 1)) * d_model;
    } else {
      g = w + (int64_t)(c0 + 16 * (k - kPT / 16) + prow) * d_model;
    }
    __builtin_amdgcn_global_load_lds(
        reinterpret_cast<const uint32_t *>(g + kPK * st + 8 * pchunk),
        reinterpret_cast<uint32_t *>(dst + k * 4096 + wave * 1024), 16, 0, 0);
  };
  f32x4 S[4][kCT], P[4][kCT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < kCT; ++jj) {
      S[i][jj] = {-0.0f, -0.0f, -0.0f, -0.0f};
      P[i][jj] = {0.0f, 0.0f, 0.0f, 0.0f};
    }
  int snext = 1;   // the next quarter whose start is still ahead
  auto fold = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < kCT; ++jj) {
        S[i][jj] += P[i][jj];
        P[i][jj] = {0.0f, 0.0f, 0.0f, 0.0f};
      }
    ++snext;
  };
  // kFast: this stage has all its k-steps and the next one exists and is
  // whole too (every stage but the last one or two): no branch in the loop,
  // which keeps the compiler's LDS waits exact.  Otherwise the general path.
  auto compute = [&](auto fast, const uint8_t *cur, uint8_t *nxt, int st) {
    constexpr bool kFast = decltype(fast)::value;
    const bool more = kFast || st + 1 < nst;
    const int nk = kFast ? kPKSteps : min(kPKSteps, T - st * kPKSteps);   // uniform
    // fragments in two register sets: after each row tile's four products of
    // k-step j come two of k-step j + 1's LDS reads and one of the next
    // stage's loads, so that the reads run while the matrix cores work (the
    // fences keep the compiler from moving them)
    bf16x8 fa[2][4], fb[2][4];   // fb[.][jj], jj < kCT
    // one fragment: lane row l16 of the 16 rows from op_row (row % 16 == l16),
    // chunk 4 j + kg of k-step j
    auto frag1 = [&](int op_row, int j) -> bf16x8 {
      const int off = l16 * 256 + 16 * ((4 * j + kg) ^ l16);
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(cur + op_row * 256 + off));
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[0][i] = frag1(64 * wm + 16 * i, 0);
      if (i < kCT) fb[0][i] = frag1(kPT + kWN * wn + 16 * i, 0);
    }
#pragma unroll
    for (int j = 0; j < kPKSteps; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (kFast || j < nk) {
#pragma unroll
          for (int jj = 0; jj < kCT; ++jj)
            P[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[j & 1][i], fb[j & 1][jj],
                                                               P[i][jj], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (j + 1 < kPKSteps && (kFast || j + 1 < nk)) {
          fa[(j + 1) & 1][i] = frag1(64 * wm + 16 * i, j + 1);
          if (i < kCT) fb[(j + 1) & 1][i] = frag1(kPT + kWN * wn + 16 * i, j + 1);
        }
        if (more && 4 * j + i < kPLoads) dma(fast, nxt, st + 1, 4 * j + i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto run_stage = [&](const uint8_t *cur, uint8_t *nxt, int st) {
    if (st + 1 < nst && (st + 2 < nst || d_model % kPK == 0))
      compute(std::true_type{}, cur, nxt, st);
    else
      compute(std::false_type{}, cur, nxt, st);
  };



#pragma unroll
  for (int k = 0; k < kPLoads; ++k) dma(std::false_type{}, stageA, 0, k);
  // two stages per trip, so that each buffer has its own copy of the code
  for (int st = 0; st < nst; st += 2) {
    while (snext <= 3 && proj_bound(T, snext) <= st * kPKSteps) fold();
    __syncthreads();   // this stage's loads done; the other buffer no longer read
    run_stage(stageA, stageB, st);
    if (st + 1 < nst) {
      while (snext <= 3 && proj_bound(T, snext) <= (st + 1) * kPKSteps) fold();
      __syncthreads();
      run_stage(stageB, stageA, st + 1);
    }
  }
  while (snext <= 4) fold();
  __syncthreads();   // every wave is done with the stages: stage A holds the epilogue rows

  float *tile = reinterpret_cast<float *>(stageA);   // 64 x kPPitch fp32
  for (int h = 0; h < 2; ++h) {   // rows 64 h .. 64 h + 63 of the tile: wave row wm = h
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < kCT; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            tile[(16 * i + 4 * kg + e) * kPPitch + kWN * wn + 16 * jj + l16] = S[i][jj][e];
    }
    __syncthreads();
    for (int item = tid; item < 64 * (kBN / 16); item += 256) {
      const int r = item / (kBN / 16), jb = item % (kBN / 16);
      const int row = r0 + 64 * h + r;
      if (row < n)
        proj_store_block(tile + r * kPPitch + 16 * jb, row, c0 + 16 * jb, kv_codes, kv_scales,
                         idx_k, seq, pos, capacity, H, esz);
    }
    __syncthreads();
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
  // Launch shapes by token count, measured at d_model 4096 (kernel trace):
  // from 512 tokens the 128-row tiles (45-50 us from 512 to 4096 tokens);
  // 256..511 64 x 64 tiles (34 us); 192..255 16 x 64 tiles of two column
  // groups (25 us); below 192 16 x 16 tiles, whose many workgroups spread
  // the weight stream over more CUs (11 us at 32 tokens, 19 us at 128).
  // Every shape sums in the same order.
  const int cols = 256 + 64 * c.idx_heads;
  const int32_t esz = c.idx_k_dtype == CSA2_FP8_E4M3 ? 1 : 2;
  uint8_t *ik = static_cast<uint8_t *>(c.idx_k);
  if (n >= kProjTileMin) {
    const int nrt = (n + kPT - 1) / kPT;
    const int nrt8 = (nrt + 7) / 8 * 8;
    if (cols % 96 == 0)   // 768 channels: 96-wide tiles
      hipLaunchKernelGGL(proj_tile_kernel<96>, dim3((unsigned)(nrt8 * (cols / 96))), dim3(256),
                         0, stream, c.kv_codes, c.kv_scales, ik, x, w, d_model, seq, pos, n,
                         c.capacity, c.idx_heads, esz, nrt, cols / 96);
    else                  // 512 channels
      hipLaunchKernelGGL(proj_tile_kernel<128>, dim3((unsigned)(nrt8 * (cols / 128))), dim3(256),
                         0, stream, c.kv_codes, c.kv_scales, ik, x, w, d_model, seq, pos, n,
                         c.capacity, c.idx_heads, esz, nrt, cols / 128);
  } else if (n >= 256) {
    hipLaunchKernelGGL((proj_append_kernel<4, 4, 1, 2>), dim3((n + 63) / 64, cols / 64), dim3(256), 0,
                       stream, c.kv_codes, c.kv_scales, ik, x, w, d_model, seq, pos, n,
                       c.capacity, c.idx_heads, esz);
  } else if (n >= 192) {
    hipLaunchKernelGGL((proj_append_kernel<1, 2, 2, 8>), dim3((n + 15) / 16, cols / 64), dim3(512),
                       0, stream, c.kv_codes, c.kv_scales, ik, x, w, d_model, seq, pos, n,
                       c.capacity, c.idx_heads, esz);
  } else {
    hipLaunchKernelGGL((proj_append_kernel<1, 1, 1, 8>), dim3((n + 15) / 16, cols / 16), dim3(256),
                       0, stream, c.kv_codes, c.kv_scales, ik, x, w, d_model, seq, pos, n,
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
