// Gather + dequantization of the selected FP4 rows and softmax attention.
//
// Model card "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression",
// Introduction, CSA2 paragraph, and aiwiki "DeepSeek V4.1-Flash", section
// "Compressed Sparse Attention 2": each layer attends over its Top-K positions
// of the shared FP4 main KV (E2M1 values, one E4M3 scale per 16 channels).
// All query heads share the one KV head, so per query the work is a dense
// [heads x 128] x [128 x rows] contraction -- it runs on matrix cores.
//
// attn_partial_kernel: one workgroup per (query, split of the selected rows),
// one wave per 16 query heads; the split is walked in sub-chunks of 64 rows
// with an online softmax, and the gathers of the next sub-chunk are in flight
// while the current one is computed.
//   * K rows are gathered straight into MFMA A-operand registers: lane l owns
//     row l%16 and channels 32g..32g+31 (g = l/16): 16 B of codes + 2 scale
//     bytes, dequantized exactly to bf16.  The contraction index is permuted
//     (k-slice s, lane group g <-> channels 32g + 8s .. +7) identically for Q.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (fp32 accumulation); exp2-based
//     softmax statistics per head; P rounded to fp16.
//   * V rows are dequantized into LDS, transposed [channel][row] in fp16
//     (exact), double-buffered, and O += P V runs on v_mfma_f32_16x16x32_f16.
// attn_combine_kernel: merges the splits of each (query, head).
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kSub = 64;                      // rows per sub-chunk
constexpr int kVtPitch = kSub + 4;            // fp16 elements per LDS row of V^T
constexpr int kMaxRowsPerSplit = 256;
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

// Gathered codes of one sub-chunk held in registers between prefetch and use.
template <int kWaves>
struct SubChunk {
  // (row, 16-channel block) items of V per thread; the last round may be partial
  static constexpr int kVItems = (kSub * 8 + kWaves * 64 - 1) / (kWaves * 64);
  uint4 kc[4];          // K codes of rows 16t + l16, channels 32g..32g+31
  uint32_t ks[4];       // their two scale bytes
  uint2 vc[kVItems];
  uint32_t vs[kVItems];
};

template <int kWaves>
__device__ __forceinline__ void gather(SubChunk<kWaves> &sc, const int32_t *rows, int base,
                                       const uint8_t *__restrict__ kv_codes,
                                       const uint8_t *__restrict__ kv_scales, int64_t seq_base,
                                       int l16, int g, int tid) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int32_t row = rows[base + 16 * t + l16];
    const int64_t slot = seq_base + (row >= 0 ? row : 0);
    sc.kc[t] = *reinterpret_cast<const uint4 *>(kv_codes + slot * 128 + 16 * g);
    sc.ks[t] = *reinterpret_cast<const uint16_t *>(kv_scales + slot * 16 + 2 * g);
  }
#pragma unroll
  for (int v = 0; v < SubChunk<kWaves>::kVItems; ++v) {
    const int item = min(tid + v * kWaves * 64, kSub * 8 - 1);
    const int32_t row = rows[base + (item >> 3)];
    const int64_t slot = seq_base + (row >= 0 ? row : 0);
    sc.vc[v] = *reinterpret_cast<const uint2 *>(kv_codes + slot * 128 + 64 + (item & 7) * 8);
    sc.vs[v] = kv_scales[slot * 16 + 8 + (item & 7)];
  }
}

// One sub-chunk of 64 rows: V to LDS, S^T on matrix cores, online softmax,
// O += P V.  Contains one barrier.
template <int kWaves>
__device__ __forceinline__ void attend_sub(const SubChunk<kWaves> &sc, const int32_t *rows, int base,
                                           _Float16 *vbuf, const bf16x8 (&qf)[4], float scale_log2,
                                           int g, int l16, int tid, float &m_run, float &l_run,
                                           f32x4 (&o)[8]) {
  constexpr int kVItems = SubChunk<kWaves>::kVItems;
    // V of this sub-chunk -> LDS, transposed, fp16 (exact)
#pragma unroll
    for (int v = 0; v < kVItems; ++v) {
      const int item = tid + v * kWaves * 64;
      if (item >= kSub * 8) break;
      const int r = item >> 3;
      const int blk = item & 7;
      const bool ok = rows[base + r] >= 0;
      const float s = ok ? e4m3_to_f32(sc.vs[v]) : 0.0f;
#pragma unroll
      for (int cc = 0; cc < 16; ++cc) {
        const uint32_t word = cc < 8 ? sc.vc[v].x : sc.vc[v].y;
        const uint32_t code = (word >> (4 * (cc & 7))) & 0xFu;
        vbuf[(blk * 16 + cc) * kVtPitch + r] = (_Float16)e2m1_times(code, s);
      }
    }

    // S^T tiles: rows base + 16t + 4g + i, head l16
    f32x4 st[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float s0 = e4m3_to_f32(sc.ks[t] & 0xFFu);
      const float s1 = e4m3_to_f32((sc.ks[t] >> 8) & 0xFFu);
      const uint32_t w[4] = {sc.kc[t].x, sc.kc[t].y, sc.kc[t].z, sc.kc[t].w};
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

    // online softmax for head 16*wave + l16
    float z[16];
    float mc = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = rows[base + 16 * t + 4 * g + i] >= 0;
        const float v = ok ? st[t][i] * scale_log2 : -INFINITY;
        z[4 * t + i] = v;
        mc = fmaxf(mc, v);
      }
    mc = fmaxf(mc, shfl_xor_f(mc, 16));
    mc = fmaxf(mc, shfl_xor_f(mc, 32));
    const float m_new = fmaxf(m_run, mc);
    const float alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
    _Float16 p16[16];
    float lsum = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float p = (m_new == -INFINITY) ? 0.0f : exp2f(z[k] - m_new);
      p16[k] = (_Float16)p;
      lsum += (float)p16[k];
    }
    lsum += shfl_xor_f(lsum, 16);
    lsum += shfl_xor_f(lsum, 32);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    // O rows are heads 16*wave + 4g + i: fetch their alpha from lane 4g + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt][i] *= a;
    }

    __syncthreads();   // V^T of this sub-chunk complete (and the other buffer free)

    // O += P V: k-slice sg covers tiles 2sg, 2sg+1; lane group g holds rows
    // 32sg + 4g + 0..3 and 32sg + 16 + 4g + 0..3
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
        const _Float16 *vrow = vbuf + (dt * 16 + l16) * kVtPitch + 32 * sg + 4 * g;
        const uint2 a = *reinterpret_cast<const uint2 *>(vrow);
        const uint2 b = *reinterpret_cast<const uint2 *>(vrow + 16);
        const f16x8 vb = __builtin_bit_cast(f16x8, make_uint4(a.x, a.y, b.x, b.y));
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb, o[dt], 0, 0, 0);
      }
    }
}

template <int kWaves>
__global__ void __launch_bounds__(kWaves * 64) attn_partial_kernel(
    const uint8_t *__restrict__ kv_codes, const uint8_t *__restrict__ kv_scales,
    int64_t capacity, const uint16_t *__restrict__ qg, int32_t n_heads,
    const int32_t *__restrict__ q_seq, const int32_t *__restrict__ topk, int32_t top_k,
    int32_t rows_per_split, float scale_log2, float *__restrict__ part_acc,
    float2 *__restrict__ part_ml, int32_t splits) {
  __shared__ int32_t rows[kMaxRowsPerSplit + 2 * kSub];   
  __shared__ _Float16 vt[2][128 * kVtPitch];

  const int split = blockIdx.x;
  const int q = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int64_t seq_base = (int64_t)q_seq[q] * capacity;
  const int row0 = split * rows_per_split;
  const int nrows = min(rows_per_split, top_k - row0);
  const int nsub = (nrows + kSub - 1) / kSub;

  for (int r = tid; r < (nsub + 2) * kSub; r += kWaves * 64)
    rows[r] = r < nrows ? topk[(int64_t)q * top_k + row0 + r] : -1;

  // Q fragment (B operand): head 16*wave + l16, channels 32g..32g+31
  bf16x8 qf[4];
  {
    const uint16_t *qp = qg + ((int64_t)q * n_heads + wave * 16 + l16) * 128 + 32 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qp + 8 * s));
  }
  __syncthreads();

  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = {0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY;   // for head 16*wave + l16 (same in all four lane groups)
  float l_run = 0.0f;

  SubChunk<kWaves> bufA, bufB;
  gather(bufA, rows, 0, kv_codes, kv_scales, seq_base, l16, g, tid);
  // ping-pong: the gathers of sub-chunk c+1 are issued before sub-chunk c is
  // computed, with no branch around them and no register copy between buffers
  // (either would make the compiler wait for the prefetch)
  for (int c = 0; c < nsub; c += 2) {
    gather(bufB, rows, (c + 1) * kSub, kv_codes, kv_scales, seq_base, l16, g, tid);
    attend_sub<kWaves>(bufA, rows, c * kSub, vt[0], qf, scale_log2, g, l16, tid, m_run, l_run, o);
    if (c + 1 >= nsub) break;
    gather(bufA, rows, (c + 2) * kSub, kv_codes, kv_scales, seq_base, l16, g, tid);
    attend_sub<kWaves>(bufB, rows, (c + 1) * kSub, vt[1], qf, scale_log2, g, l16, tid, m_run, l_run, o);
  }

  // partial results: O rows = heads 16*wave + 4g + i, column d = 16 dt + l16
  const int64_t pbase = ((int64_t)q * splits + split) * n_heads;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = wave * 16 + 4 * g + i;
      part_acc[(pbase + head) * 128 + dt * 16 + l16] = o[dt][i];
    }
  if (g == 0) part_ml[pbase + wave * 16 + l16] = make_float2(m_run, l_run);
}

// One workgroup per (query, 4 heads): thread (head, d) merges every split.
__global__ void __launch_bounds__(512) attn_combine_kernel(
    const float *__restrict__ part_acc, const float2 *__restrict__ part_ml, int32_t n_heads,
    int32_t splits, float *__restrict__ out, float *__restrict__ lse) {
  constexpr int kHeadsPer = 4;
  __shared__ float mx_sh[kHeadsPer];
  __shared__ float inv_sh[kHeadsPer];
  __shared__ float lse_sh[kHeadsPer];
  const int q = blockIdx.y;
  const int hl = threadIdx.x >> 7;
  const int h = blockIdx.x * kHeadsPer + hl;
  const int d = threadIdx.x & 127;
  const float2 *ml = part_ml + (int64_t)q * splits * n_heads + h;
  if (d < 64) {
    // the split statistics of head h: overall max and normalizer
    float mx = -INFINITY;
    for (int s = d; s < splits; s += 64) mx = fmaxf(mx, ml[(int64_t)s * n_heads].x);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float tot = 0.0f;
    for (int s = d; s < splits; s += 64) {
      const float2 v = ml[(int64_t)s * n_heads];
      if (v.x != -INFINITY) tot += exp2f(v.x - mx) * v.y;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o, 64);
    if (d == 0) {
      mx_sh[hl] = mx;
      inv_sh[hl] = tot > 0.0f ? 1.0f / tot : 0.0f;
      lse_sh[hl] = tot > 0.0f ? (mx + log2f(tot)) * kLn2 : -INFINITY;
    }
  }
  __syncthreads();
  const float mx = mx_sh[hl];
  float acc = 0.0f;
  if (mx != -INFINITY) {
    const float *pa = part_acc + ((int64_t)q * splits * n_heads + h) * 128 + d;
    const int64_t sstride = (int64_t)n_heads * 128;
    int s = 0;
    for (; s + 4 <= splits; s += 4) {
      float a[4], w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = pa[(s + u) * sstride];
        const float m = ml[(int64_t)(s + u) * n_heads].x;
        w[u] = (m == -INFINITY) ? 0.0f : exp2f(m - mx);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += w[u] * a[u];
    }
    for (; s < splits; ++s) {
      const float m = ml[(int64_t)s * n_heads].x;
      if (m != -INFINITY) acc += exp2f(m - mx) * pa[s * sstride];
    }
  }
  const int64_t oi = (int64_t)q * n_heads + h;
  out[oi * 128 + d] = acc * inv_sh[hl];
  if (lse != nullptr && d == 0) lse[oi] = lse_sh[hl];
}

// Rows per split: enough workgroups to fill the chip (>= 256 when the batch
// allows), at most kMaxRowsPerSplit, a multiple of the sub-chunk.
int32_t rows_per_split(int32_t nq, int32_t top_k) {
  const int32_t subs = (top_k + kSub - 1) / kSub;
  int32_t per = kMaxRowsPerSplit / kSub;
  while (per > 1 && (int64_t)nq * ((subs + per - 1) / per) < 256) per /= 2;
  return per * kSub;
}

}  // namespace

AttnWorkspace attn_workspace_layout(const csa2_cache &c, int32_t nq, int32_t n_heads,
                                    int32_t top_k) {
  AttnWorkspace w;
  const int32_t rps = rows_per_split(nq, top_k);
  w.splits = (top_k + rps - 1) / rps;
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
  const int32_t rps = rows_per_split(nq, top_k);
  dim3 grid((unsigned)L.splits, (unsigned)nq);
  const int waves = n_heads / 16;
#define CSA2_ATTN_CASE(W)                                                                        \
  case W:                                                                                        \
    hipLaunchKernelGGL(attn_partial_kernel<W>, grid, dim3(W * 64), 0, s, c.kv_codes, c.kv_scales, \
                       (int64_t)c.capacity, q, n_heads, q_seq, topk, top_k, rps, scale_log2, acc, \
                       ml, L.splits);                                                            \
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
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(n_heads / 4), (unsigned)nq), dim3(512),
                     0, s, acc, ml, n_heads, L.splits, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
