// Gather + dequantization of the selected FP4 rows and softmax attention.
//
// Model card "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression",
// Introduction, CSA2 paragraph, and aiwiki "DeepSeek V4.1-Flash", section
// "Compressed Sparse Attention 2": each layer attends over its Top-K positions
// of the shared FP4 main KV (E2M1 values, one E4M3 scale per 16 channels).
// All query heads share the one KV head, so per query the work is a dense
// [heads x 128] x [128 x rows] contraction -- it runs on matrix cores.
//
// attn_partial_kernel: one workgroup per (query, split of 64 selected rows),
// one wave per 16 query heads.
//   * K rows are gathered straight into MFMA A-operand registers: lane l owns
//     row l%16 and channels 32g..32g+31 (g = l/16): 16 B of codes + 2 scale
//     bytes, dequantized exactly to bf16.  The contraction index is permuted
//     (k-slice s, lane group g <-> channels 32g + 8s .. +7) identically for Q.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (fp32 accumulation), exp2-based
//     softmax statistics per head over the split, P rounded to fp16.
//   * V rows are dequantized once per workgroup into LDS, transposed
//     [channel][row] in fp16 (exact), and O = P V runs on
//     v_mfma_f32_16x16x32_f16.  Partial (max, sum, O) go to the workspace.
// attn_combine_kernel: merges the splits of each (query, head).
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kRowsPerSplit = 64;
constexpr int kVtPitch = kRowsPerSplit + 4;    // fp16 elements per LDS row of V^T
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// E2M1 code (4 bits, bit 3 sign) times a decoded scale; exact in fp32.
// Placing the code's 3 magnitude bits at fp32 bits 24..22 gives the value
// scaled by 2^-126 (code 1 lands on the subnormal 0.5 * 2^-126), so one
// multiply by 2^126 restores it.
__device__ __forceinline__ float e2m1_times(uint32_t code, float s) {
  const float tiny = __uint_as_float(((code & 8u) << 28) | ((code & 7u) << 22));
  return (tiny * 0x1p126f) * s;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // values here have <= 6 significant bits: truncation is exact
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

template <int kWaves>
__global__ void __launch_bounds__(kWaves * 64) attn_partial_kernel(
    const uint8_t *__restrict__ kv_codes, const uint8_t *__restrict__ kv_scales,
    int64_t capacity, const uint16_t *__restrict__ qg, int32_t n_heads,
    const int32_t *__restrict__ q_seq, const int32_t *__restrict__ topk, int32_t top_k,
    float scale_log2, float *__restrict__ part_acc, float2 *__restrict__ part_ml,
    int32_t splits) {
  __shared__ int32_t rows[kRowsPerSplit];
  __shared__ _Float16 vt[128 * kVtPitch];

  const int split = blockIdx.x;
  const int q = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t seq_base = (int64_t)q_seq[q] * capacity;

  if (tid < kRowsPerSplit) {
    const int r = split * kRowsPerSplit + tid;
    rows[tid] = r < top_k ? topk[(int64_t)q * top_k + r] : -1;
  }
  __syncthreads();

  // --- V rows -> LDS, transposed, fp16 (64 rows x 8 blocks of 16 channels)
  for (int item = tid; item < kRowsPerSplit * 8; item += kWaves * 64) {
    const int r = item >> 3;
    const int blk = item & 7;
    const int32_t row = rows[r];
    uint2 codes = make_uint2(0, 0);
    float s = 0.0f;
    if (row >= 0) {
      const int64_t slot = seq_base + row;
      codes = *reinterpret_cast<const uint2 *>(kv_codes + slot * 128 + 64 + blk * 8);
      s = e4m3_to_f32(kv_scales[slot * 16 + 8 + blk]);
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const uint32_t word = c < 8 ? codes.x : codes.y;
      const uint32_t code = (word >> (4 * (c & 7))) & 0xFu;
      vt[(blk * 16 + c) * kVtPitch + r] = (_Float16)e2m1_times(code, s);
    }
  }

  // --- Q fragment (B operand): head 16*wave + lane%16, channels 32g..32g+31
  const int g = lane >> 4;
  const int l16 = lane & 15;
  bf16x8 qf[4];
  {
    const uint16_t *qp = qg + ((int64_t)q * n_heads + wave * 16 + l16) * 128 + 32 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 v = *reinterpret_cast<const uint4 *>(qp + 8 * s);
      qf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // --- S^T tiles: rows 16t + 4g + i, head l16
  f32x4 st[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int32_t row = rows[16 * t + l16];
    uint4 codes = make_uint4(0, 0, 0, 0);
    uint32_t sc2 = 0;
    if (row >= 0) {
      const int64_t slot = seq_base + row;
      codes = *reinterpret_cast<const uint4 *>(kv_codes + slot * 128 + 16 * g);
      sc2 = *reinterpret_cast<const uint16_t *>(kv_scales + slot * 16 + 2 * g);
    }
    const float s0 = e4m3_to_f32(sc2 & 0xFFu);
    const float s1 = e4m3_to_f32(sc2 >> 8);
    const uint32_t w[4] = {codes.x, codes.y, codes.z, codes.w};
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // channels 32g + 8s .. +7 = code word s; scale block 2g + (s >= 2)
      const float sc = s < 2 ? s0 : s1;
      const uint32_t cw = w[s];
      uint32_t packed[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        packed[e] = pack_bf16x2(e2m1_times((cw >> (8 * e)) & 0xFu, sc),
                                e2m1_times((cw >> (8 * e + 4)) & 0xFu, sc));
      const bf16x8 kf = __builtin_bit_cast(bf16x8, make_uint4(packed[0], packed[1], packed[2], packed[3]));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], acc, 0, 0, 0);
    }
    st[t] = acc;
  }

  // --- softmax statistics over this split for head 16*wave + l16
  float z[16];
  float m = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = rows[16 * t + 4 * g + i] >= 0;
      const float v = ok ? st[t][i] * scale_log2 : -INFINITY;
      z[4 * t + i] = v;
      m = fmaxf(m, v);
    }
  m = fmaxf(m, shfl_xor_f(m, 16));
  m = fmaxf(m, shfl_xor_f(m, 32));
  _Float16 p16[16];
  float lsum = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float p = (m == -INFINITY) ? 0.0f : exp2f(z[k] - m);
    p16[k] = (_Float16)p;
    lsum += (float)p16[k];
  }
  lsum += shfl_xor_f(lsum, 16);
  lsum += shfl_xor_f(lsum, 32);

  __syncthreads();   // V^T complete

  // --- O = P V: k-slice sigma covers tiles 2 sigma, 2 sigma + 1;
  // lane group g holds rows 32 sigma + 4g + 0..3 and 32 sigma + 16 + 4g + 0..3.
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {
    f16x8 pa;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pa[i] = p16[4 * (2 * sg) + i];
      pa[4 + i] = p16[4 * (2 * sg + 1) + i];
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const _Float16 *vrow = vt + (dt * 16 + l16) * kVtPitch + 32 * sg + 4 * g;
      const uint2 a = *reinterpret_cast<const uint2 *>(vrow);
      const uint2 b = *reinterpret_cast<const uint2 *>(vrow + 16);
      const f16x8 vb = __builtin_bit_cast(f16x8, make_uint4(a.x, a.y, b.x, b.y));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb, o[dt], 0, 0, 0);
    }
  }

  // --- partial results: O rows = heads 16*wave + 4g + i, column d = 16 dt + l16
  const int64_t pbase = ((int64_t)q * splits + split) * n_heads;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = wave * 16 + 4 * g + i;
      part_acc[(pbase + head) * 128 + dt * 16 + l16] = o[dt][i];
    }
  if (g == 0) part_ml[pbase + wave * 16 + l16] = make_float2(m, lsum);
}

__global__ void __launch_bounds__(128) attn_combine_kernel(
    const float *__restrict__ part_acc, const float2 *__restrict__ part_ml, int32_t n_heads,
    int32_t splits, float *__restrict__ out, float *__restrict__ lse) {
  const int h = blockIdx.x;
  const int q = blockIdx.y;
  const int d = threadIdx.x;
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s)
    mx = fmaxf(mx, part_ml[((int64_t)q * splits + s) * n_heads + h].x);
  float acc = 0.0f, tot = 0.0f;
  if (mx != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const int64_t pi = ((int64_t)q * splits + s) * n_heads + h;
      const float2 ml = part_ml[pi];
      if (ml.x == -INFINITY) continue;
      const float w = exp2f(ml.x - mx);
      tot += w * ml.y;
      acc += w * part_acc[pi * 128 + d];
    }
  }
  const int64_t oi = ((int64_t)q * n_heads + h);
  out[oi * 128 + d] = tot > 0.0f ? acc / tot : 0.0f;
  if (lse != nullptr && d == 0) lse[oi] = tot > 0.0f ? (mx + log2f(tot)) * kLn2 : -INFINITY;
}

}  // namespace

AttnWorkspace attn_workspace_layout(const csa2_cache &c, int32_t nq, int32_t n_heads,
                                    int32_t top_k) {
  AttnWorkspace w;
  w.splits = (top_k + kRowsPerSplit - 1) / kRowsPerSplit;
  const size_t units = (size_t)nq * w.splits * n_heads;
  w.part_acc = 0;
  w.part_ml = align256(units * c.dv * sizeof(float));
  w.total = align256(w.part_ml + units * sizeof(float2));
  return w;
}

hipError_t launch_sparse_attn(const csa2_cache &c, const uint16_t *q, int32_t n_heads,
                              const int32_t *q_seq, int32_t nq, const int32_t *topk,
                              int32_t top_k, float softmax_scale, float *out, float *lse,
                              uint8_t *ws, const AttnWorkspace &L, hipStream_t s) {
  float *acc = reinterpret_cast<float *>(ws + L.part_acc);
  float2 *ml = reinterpret_cast<float2 *>(ws + L.part_ml);
  const float scale_log2 = softmax_scale * kLog2e;
  dim3 grid((unsigned)L.splits, (unsigned)nq);
  const int waves = n_heads / 16;
#define CSA2_ATTN_CASE(W)                                                                        \
  case W:                                                                                        \
    hipLaunchKernelGGL(attn_partial_kernel<W>, grid, dim3(W * 64), 0, s, c.kv_codes, c.kv_scales, \
                       (int64_t)c.capacity, q, n_heads, q_seq, topk, top_k, scale_log2, acc, ml, \
                       L.splits);                                                                \
    break;
  switch (waves) {
    CSA2_ATTN_CASE(1)
    CSA2_ATTN_CASE(2)
    CSA2_ATTN_CASE(3)
    CSA2_ATTN_CASE(4)
    CSA2_ATTN_CASE(5)
    CSA2_ATTN_CASE(6)
    CSA2_ATTN_CASE(7)
    CSA2_ATTN_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef CSA2_ATTN_CASE
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)n_heads, (unsigned)nq), dim3(128), 0, s,
                     acc, ml, n_heads, L.splits, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
