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
// with an online softmax.
//   * The workgroup gathers a sub-chunk's codes two sub-chunks ahead (one in
//     the four-per-CU form that large 64-head grids take) and dequantizes
//     them once into LDS, shared by every head wave: K^ in fp16 as
//     MFMA A fragments (the contraction index permuted, k-slice s and lane
//     group g <-> channels 32g + 8s .. +7, identically for Q), V^ in fp16
//     transposed [channel][row].  E2M1 codes go through the hardware FP4
//     conversion; every value is exact (E2M1 times E4M3 has at most 6
//     significant bits and lies in [2^-10, 2688]).
//   * Q is rounded once to fp16 (exact for bf16 values of magnitude 2^-14 to
//     65504; smaller ones move by less than 2^-25).
//   * S^T = K Q^T with v_mfma_f32_16x16x32_f16 (fp32 accumulation); exp2-based
//     softmax statistics per head; P rounded to fp16; O^T += V^T P^T with
//     v_mfma_f32_16x16x32_f16 (a lane's output column is its own head, so the
//     softmax rescale and normalization need no cross-lane moves).
// attn_combine_kernel: merges the splits of each (query, head).
#include <algorithm>
#include <mutex>

#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kSub = 64;                      // rows per sub-chunk
constexpr int kVtPitch = kSub + 8;            // fp16 elements per LDS row of V^T (16-B aligned rows)

// Where row r (0..63) of a sub-chunk sits in an LDS row of V^T: in each half
// of 32 rows, the rows one lane group of the PV product reads (4g..4g+3 and
// 16+4g..16+4g+3) are adjacent, so that its operand is one 16-byte read.
// Rows 2p and 2p + 1 stay adjacent.
__device__ __forceinline__ int vt_col(int r) {
  return (r & 32) + 8 * ((r >> 2) & 3) + 4 * ((r >> 4) & 1) + (r & 3);
}
constexpr int kMaxRowsPerSplit = 2048;
constexpr int kTargetGroups = 256;            // workgroups aimed for (one per CU)
constexpr int kTwoSubMinGroups = 128;         // see rows_per_split
constexpr int64_t kDenseMinGroups = 768;      // 64 heads: the four-per-CU form from this many workgroups
constexpr int kMaxSplits = 256;               // splits of one query, at most
constexpr int kCombineBatch = 32;            // split outputs per round of combine loads
constexpr int kLocalRowsPerSplit = 128;       // window rows per split of the fused call
static_assert(kTargetGroups <= kMaxSplits && (65536 + kMaxRowsPerSplit - 1) / kMaxRowsPerSplit <= kMaxSplits,
              "every accepted top_k fits the combine's split table");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// Two E2M1 codes (byte kByte of w) times s (given as an fp16 pair), as fp16:
// E2M1 and E4M3 values and their products are exact in fp16.
template <int kByte>
__device__ __forceinline__ f16x2 fp4x2_f16(uint32_t w, f16x2 s2) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, kByte) * s2;
}

// Gathered codes of one sub-chunk, held in registers between load and dequant.
//   K item (tile t, lane l): row 16t + l%16, channels 32g..32g+31 (g = l/16):
//     16 B of codes and their two scale bytes.
//   V item (row pair p, block b): rows 2p, 2p+1, channels 16b..16b+15: 8 B of
//     codes and one scale byte per row.
template <int kThreads>
struct Gathered {
  static constexpr int kItems = (4 * 64 + kThreads - 1) / kThreads;   // of each kind
  uint4 kc[kItems];
  uint32_t ks[kItems];
  uint2 vc[kItems][2];
  uint32_t vs[kItems];
};

// codes / scales: the query's sequence (row 0); row offsets fit 32 bits.
template <int kThreads>
__device__ __forceinline__ void gather(Gathered<kThreads> &gd, const int32_t *rows, int base,
                                       const uint8_t *__restrict__ codes,
                                       const uint8_t *__restrict__ scales, int tid) {
#pragma unroll
  for (int it = 0; it < Gathered<kThreads>::kItems; ++it) {
    const int item = min(tid + it * kThreads, 4 * 64 - 1);
    {
      const int g = (item & 63) >> 4;
      const uint32_t row = (uint32_t)max(rows[base + 16 * (item >> 6) + (item & 15)], 0);
      gd.kc[it] = *reinterpret_cast<const uint4 *>(codes + row * 128u + 16u * g);
      gd.ks[it] = *reinterpret_cast<const uint16_t *>(scales + row * 16u + 2u * g);
    }
    {
      const int pr = item & 31, b = item >> 5;
      uint32_t sc = 0u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t row = (uint32_t)max(rows[base + 2 * pr + h], 0);
        gd.vc[it][h] = *reinterpret_cast<const uint2 *>(codes + row * 128u + 64u + 8u * b);
        sc |= (uint32_t)scales[row * 16u + 8u + b] << (8 * h);
      }
      gd.vs[it] = sc;
    }
  }
}

// Dequantizes one gathered sub-chunk into LDS: K^ as fp16 MFMA A fragments
// kq[tile][k-step][lane] (16 B each: k-step s of lane group g is channels
// 32g + 8s .. +7), V^ transposed as fp16 vt[channel][row].
template <int kThreads, int kPitch>
__device__ __forceinline__ void dequant(const Gathered<kThreads> &gd, uint4 *kq, _Float16 *vt,
                                        int tid) {
#pragma unroll
  for (int it = 0; it < Gathered<kThreads>::kItems; ++it) {
    const int item = tid + it * kThreads;
    if (Gathered<kThreads>::kItems * kThreads > 4 * 64 && item >= 4 * 64) break;
    {
      // E4M3 scales of the two 16-channel blocks, by the hardware OCP E4M3
      // conversion (exact in fp16)
      const f16x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(gd.ks[it], 1.0f, false);
      const _Float16 s0 = s01[0], s1 = s01[1];
      const uint32_t w[4] = {gd.kc[it].x, gd.kc[it].y, gd.kc[it].z, gd.kc[it].w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f16x2 sc = s < 2 ? f16x2{s0, s0} : f16x2{s1, s1};
        kq[((item >> 6) * 4 + s) * 64 + (item & 63)] =
            make_uint4(__builtin_bit_cast(uint32_t, fp4x2_f16<0>(w[s], sc)),
                       __builtin_bit_cast(uint32_t, fp4x2_f16<1>(w[s], sc)),
                       __builtin_bit_cast(uint32_t, fp4x2_f16<2>(w[s], sc)),
                       __builtin_bit_cast(uint32_t, fp4x2_f16<3>(w[s], sc)));
      }
    }
    {
      const int pr = item & 31, b = item >> 5;
      const f16x2 sab = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(gd.vs[it], 1.0f, false);
      const _Float16 sa = sab[0], sb = sab[1];
      const f16x2 s2a = {sa, sa}, s2b = {sb, sb};
      uint32_t *dst = reinterpret_cast<uint32_t *>(vt + (16 * b) * kPitch + vt_col(2 * pr));
#pragma unroll
      for (int hw = 0; hw < 2; ++hw) {
        const uint32_t wa = hw ? gd.vc[it][0].y : gd.vc[it][0].x;
        const uint32_t wb = hw ? gd.vc[it][1].y : gd.vc[it][1].x;
        f16x2 ra[4], rb[4];
        ra[0] = fp4x2_f16<0>(wa, s2a), ra[1] = fp4x2_f16<1>(wa, s2a);
        ra[2] = fp4x2_f16<2>(wa, s2a), ra[3] = fp4x2_f16<3>(wa, s2a);
        rb[0] = fp4x2_f16<0>(wb, s2b), rb[1] = fp4x2_f16<1>(wb, s2b);
        rb[2] = fp4x2_f16<2>(wb, s2b), rb[3] = fp4x2_f16<3>(wb, s2b);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t a = __builtin_bit_cast(uint32_t, ra[e]);
          const uint32_t c = __builtin_bit_cast(uint32_t, rb[e]);
          // channel 8hw + 2e: (row 2pr, row 2pr+1); channel 8hw + 2e + 1 likewise
          dst[((8 * hw + 2 * e) * kPitch) / 2] = __builtin_amdgcn_perm(c, a, 0x05040100u);
          dst[((8 * hw + 2 * e + 1) * kPitch) / 2] = __builtin_amdgcn_perm(c, a, 0x07060302u);
        }
      }
    }
  }
}

// Cross-row reductions with gfx950's lane swaps (VALU, no LDS round trip):
// with both operands x, permlane16_swap leaves a lane's own value and that of
// lane ^ 16 in the two results (permlane32_swap: lane ^ 32), in an order that
// depends on the lane; the operations are commutative, so every lane of a
// pair gets the same bits.
__device__ __forceinline__ float xor16_partner_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_partner_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lane_pair_sum16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float lane_pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One sub-chunk of 64 rows from LDS: S^T on matrix cores, online softmax,
// O^T += V^T P^T.  scale_log2 = |softmax scale| * log2(e) (a negative scale was
// folded into Q), so the running maximum of the scaled scores is the scaled
// maximum of the raw ones.
template <int kPitch>
__device__ __forceinline__ void attend_sub(const uint4 *kq, const _Float16 *vbuf,
                                           const int32_t *rows, int base, const f16x8 (&qf)[4],
                                           float scale_log2, int g, int l16, int lane,
                                           float &m_run, float &l_run, f32x4 (&o)[8]) {
  // S^T tiles: rows base + 16t + 4g + i, head l16
  f32x4 st[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f16x8 kf = __builtin_bit_cast(f16x8, kq[(t * 4 + s) * 64 + lane]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[s], acc, 0, 0, 0);
    }
    st[t] = acc;
  }

  // online softmax for head 16*wave + l16; rows marked -1 (bit set in `bad`)
  // take no weight
  const uint64_t bad = __ballot(rows[base + lane] < 0);
  // this lane's rows: bit 4t + i <-> row 16t + 4g + i
  uint32_t mine = 0u;
  float mc = -INFINITY;
  if (bad != 0ull) {
#pragma unroll
    for (int t = 0; t < 4; ++t) mine |= ((uint32_t)(bad >> (16 * t + 4 * g)) & 0xFu) << (4 * t);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) st[t][i] = ((mine >> (4 * t + i)) & 1u) ? -INFINITY : st[t][i];
  }
  // max as med3(x, y, +inf), as a tree: no NaN canonicalization of the
  // matrix-core results (none is NaN: -1 rows hold -inf)
  float m4[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    m4[t] = __builtin_amdgcn_fmed3f(__builtin_amdgcn_fmed3f(st[t][0], st[t][1], INFINITY),
                                    __builtin_amdgcn_fmed3f(st[t][2], st[t][3], INFINITY), INFINITY);
  mc = __builtin_amdgcn_fmed3f(__builtin_amdgcn_fmed3f(m4[0], m4[1], INFINITY),
                               __builtin_amdgcn_fmed3f(m4[2], m4[3], INFINITY), INFINITY);
  mc = xor16_partner_max(mc);
  mc = xor32_partner_max(mc);
  // (fmaxf drops the NaN of -inf * 0 for a zero scale)
  const float m_new = fmaxf(m_run, mc * scale_log2);
  // exp2 straight on the hardware instruction: arguments are <= 0 and the
  // results go to fp16, so results below the fp32 normal range do not matter
  const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
  f16x2 p2[8];
  if (bad == 0ull) {
    // every row valid: m_new is finite
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int t = k >> 1, i = 2 * (k & 1);
      const f32x2 e = {__builtin_amdgcn_exp2f(fmaf(st[t][i], scale_log2, -m_new)),
                       __builtin_amdgcn_exp2f(fmaf(st[t][i + 1], scale_log2, -m_new))};
      p2[k] = __builtin_convertvector(e, f16x2);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int t = k >> 1, i = 2 * (k & 1);
      f32x2 e = {__builtin_amdgcn_exp2f(fmaf(st[t][i], scale_log2, -m_new)),
                 __builtin_amdgcn_exp2f(fmaf(st[t][i + 1], scale_log2, -m_new))};
      // no weight when nothing is visible yet, or for a -1 row (also with a
      // zero scale, where the exponent is NaN)
      e[0] = (m_new == -INFINITY || ((mine >> (4 * t + i)) & 1u)) ? 0.0f : e[0];
      e[1] = (m_new == -INFINITY || ((mine >> (4 * t + i + 1)) & 1u)) ? 0.0f : e[1];
      p2[k] = __builtin_convertvector(e, f16x2);
    }
  }
  // the normalizer sums the fp16 weights the PV product uses
  const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
  float ls[2] = {0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 8; ++k) ls[k & 1] = __builtin_amdgcn_fdot2(p2[k], one2, ls[k & 1], false);
  float lsum = ls[0] + ls[1];
  lsum = lane_pair_sum16(lsum);
  lsum = lane_pair_sum32(lsum);
  l_run = l_run * alpha + lsum;
  m_run = m_new;
  // O^T columns are this lane's head.  Once the running maxima settle, alpha
  // is 1 everywhere and O is left alone.
  if (__ballot(alpha != 1.0f) != 0ull) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
  }

  // O^T += V^T P^T (so that a lane's output column is its own head): k-slice
  // sg covers tiles 2sg, 2sg+1; lane group g holds rows 32sg + 4g + 0..3 and
  // 32sg + 16 + 4g + 0..3 of both operands
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {
    const f16x8 pa = __builtin_bit_cast(
        f16x8, make_uint4(__builtin_bit_cast(uint32_t, p2[4 * sg]),
                          __builtin_bit_cast(uint32_t, p2[4 * sg + 1]),
                          __builtin_bit_cast(uint32_t, p2[4 * sg + 2]),
                          __builtin_bit_cast(uint32_t, p2[4 * sg + 3])));
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      // rows 32sg + 4g + 0..3 and 32sg + 16 + 4g + 0..3 (adjacent, see vt_col)
      const _Float16 *vrow = vbuf + (dt * 16 + l16) * kPitch + 32 * sg + 8 * g;
      const f16x8 vb = __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4 *>(vrow));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vb, pa, o[dt], 0, 0, 0);
    }
  }
}

// One workgroup per (query, split of the selected rows), one wave per 16
// heads.  Per sub-chunk of 64 rows the workgroup gathers the codes (two
// sub-chunks ahead, in registers), dequantizes K^ and V^ once into LDS and
// every wave runs its heads over them.  One LDS stage (43 KB per workgroup)
// and at most 168 VGPRs let three workgroups share a CU, which hides the
// dequantization and softmax phases of one behind the others'.  With a
// single split the results are final (normalized output and lse); otherwise
// partial (O, max, sum) per split go to attn_combine_kernel.
// Q fragment (B operand): head 16*wave + l16, channels 32g..32g+31, in fp16,
// negated when the softmax scale is negative.
__device__ __forceinline__ void load_q_raw(const uint16_t *__restrict__ qg, int q, int n_heads,
                                           int wave, int l16, int g, uint4 (&raw)[4]) {
  const uint16_t *qp = qg + ((int64_t)q * n_heads + wave * 16 + l16) * 128 + 32 * g;
#pragma unroll
  for (int s = 0; s < 4; ++s) raw[s] = *reinterpret_cast<const uint4 *>(qp + 8 * s);
}

__device__ __forceinline__ void convert_q(const uint4 (&raw)[4], bool q_negate, f16x8 (&qf)[4]) {
  const uint32_t flip = q_negate ? 0x80008000u : 0u;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t w[4] = {raw[s].x ^ flip, raw[s].y ^ flip, raw[s].z ^ flip, raw[s].w ^ flip};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f16x2 h = __builtin_convertvector(
          (f32x2{__uint_as_float(w[e] << 16), __uint_as_float(w[e] & 0xFFFF0000u)}), f16x2);
      qf[s][2 * e] = h[0];
      qf[s][2 * e + 1] = h[1];
    }
  }
}

__device__ __forceinline__ void load_q(const uint16_t *__restrict__ qg, int q, int n_heads,
                                       int wave, int l16, int g, bool q_negate, f16x8 (&qf)[4]) {
  uint4 raw[4];
  load_q_raw(qg, q, n_heads, wave, l16, g, raw);
  convert_q(raw, q_negate, qf);
}

// Window rows [first, first + count) of a query at position p, whose window
// holds nall = min(window, p + 1) rows (row r = position p - nall + 1 + r):
// rows[i] = the slot of row first + i when the slot holds that position,
// else -1; padded with -1 to whole sub-chunks.  Returns the sub-chunk count.
__device__ __forceinline__ int fill_window_rows(const int32_t *__restrict__ lpos, int64_t sbase,
                                                int window, int32_t p, int nall, int first,
                                                int count, int32_t *rows, int tid, int nthreads) {
  const int nsub = (count + kSub - 1) / kSub;
  // eight slot positions per thread per batch of loads, branch-free (a row
  // past `count` reads slot 0 of the window and is dropped)
  for (int r0 = 0; r0 < nsub * kSub; r0 += 8 * nthreads) {
    int32_t have[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = r0 + u * nthreads + tid;
      const int32_t pr = p - nall + 1 + first + r;
      have[u] = lpos[sbase + (r < count ? pr % window : 0)];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = r0 + u * nthreads + tid;
      const int32_t pr = p - nall + 1 + first + r;
      if (r < nsub * kSub) rows[r] = (r < count && have[u] == pr) ? pr % window : -1;
    }
  }
  return nsub;
}

// One sub-chunk of window rows (slots rows[base..base+63], -1 read as slot 0
// and masked later) into the LDS layouts of the FP4 path: E4M3 codes convert
// exactly to fp16.  K^ fragment (tile t, k-step s, lane l) = row 16t + l%16,
// channels 32(l/16) + 8s .. +7; V^ transposed as (row 2pr, row 2pr+1) fp16
// pairs per channel.
template <int kThreads>
__device__ __forceinline__ void stage_local(const uint8_t *__restrict__ lk,
                                            const uint8_t *__restrict__ lv, int64_t sbase,
                                            const int32_t *rows, int base, uint4 *kq,
                                            _Float16 *vt, int tid) {
  for (int item = tid; item < 4 * 4 * 64; item += kThreads) {
    const int t = item >> 8, s = (item >> 6) & 3, l = item & 63;
    const int slot = max(rows[base + 16 * t + (l & 15)], 0);
    const uint2 w = *reinterpret_cast<const uint2 *>(lk + (sbase + slot) * 128 + 32 * (l >> 4) + 8 * s);
    kq[(t * 4 + s) * 64 + l] = make_uint4(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, true)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, true)));
  }
  for (int item = tid; item < 32 * 8; item += kThreads) {
    const int pr = item & 31, b = item >> 5;
    const int sa = max(rows[base + 2 * pr], 0), sb = max(rows[base + 2 * pr + 1], 0);
    const uint4 wa = *reinterpret_cast<const uint4 *>(lv + (sbase + sa) * 128 + 16 * b);
    const uint4 wb = *reinterpret_cast<const uint4 *>(lv + (sbase + sb) * 128 + 16 * b);
    const uint32_t xa[4] = {wa.x, wa.y, wa.z, wa.w}, xb[4] = {wb.x, wb.y, wb.z, wb.w};
    uint32_t *dst = reinterpret_cast<uint32_t *>(vt + (16 * b) * kVtPitch + vt_col(2 * pr));
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a[2] = {
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(xa[w], 1.0f, false)),
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(xa[w], 1.0f, true))};
      const uint32_t bb[2] = {
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(xb[w], 1.0f, false)),
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(xb[w], 1.0f, true))};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // channels 4w + 2h, 4w + 2h + 1 of the block
        const int e = 2 * w + h;
        dst[((2 * e) * kVtPitch) / 2] = __builtin_amdgcn_perm(bb[h], a[h], 0x05040100u);
        dst[((2 * e + 1) * kVtPitch) / 2] = __builtin_amdgcn_perm(bb[h], a[h], 0x07060302u);
      }
    }
  }
}

// A split's unnormalized output and (max, sum) statistics, for the combine.
__device__ __forceinline__ void store_partial(float *__restrict__ part_acc,
                                              float2 *__restrict__ part_ml, int q, int splits,
                                              int split, int n_heads, int head, int g,
                                              const f32x4 (&o)[8], float m_run, float l_run) {
  const int64_t pbase = ((int64_t)q * splits + split) * n_heads;
  float *pq = part_acc + (pbase + head) * 128 + 4 * g;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4 *>(pq + dt * 16) = o[dt];
  if (g == 0) part_ml[pbase + head] = make_float2(m_run, l_run);
}

// kWithLocal: the launch also holds the window splits (csa2_sparse_local_attn); the
// sparse-only instantiation carries none of their code.
// kDense (64 heads, grids of thousands of workgroups, sparse rows only): four
// workgroups per CU instead of three -- the split's row list passes through a
// ring of four sub-chunks in LDS (each sub-chunk's indices loaded two
// iterations ahead, through a register) instead of staying whole, and the
// codes are gathered one sub-chunk ahead, so that the stage and the registers
// fit four.
template <int kWaves, bool kWithLocal, bool kDense = false>
__global__ void __launch_bounds__(kWaves * 64, kDense ? 4 : (kWaves >= 4 ? 3 : 1)) attn_partial_kernel(
    const uint8_t *__restrict__ kv_codes, const uint8_t *__restrict__ kv_scales,
    int64_t capacity, const uint16_t *__restrict__ qg, int32_t n_heads,
    const int32_t *__restrict__ q_seq, const int32_t *__restrict__ topk, int32_t top_k,
    int32_t rows_per_split, float scale_log2, bool q_negate, float *__restrict__ part_acc,
    float2 *__restrict__ part_ml, int32_t splits, float *__restrict__ out,
    float *__restrict__ lse, int32_t sparse_splits, const uint8_t *__restrict__ lk,
    const uint8_t *__restrict__ lv, const int32_t *__restrict__ lpos, int32_t window,
    const int32_t *__restrict__ q_pos) {
  constexpr int kThreads = kWaves * 64;
  static_assert(!kDense || (kWaves == 4 && !kWithLocal), "the dense form: 64 heads, sparse rows");
  // V^T row pitch: 80 in the dense form, where the LDS bank-conflict counter
  // then reads zero (with 72 the PV fragment reads conflict, ~13% of the
  // launch's cycles); 72 measured faster in the three-per-CU form
  constexpr int kPitch = kDense ? kSub + 16 : kVtPitch;
  __shared__ int32_t rows[kDense ? 4 * kSub : kMaxRowsPerSplit + 2 * kSub];
  __shared__ uint4 kq[4 * 4 * 64];
  __shared__ __attribute__((aligned(16))) _Float16 vt[128 * kPitch];

  const int split = blockIdx.x;
  const int q = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int l16 = lane & 15;

  if (kWithLocal && split >= sparse_splits) {
    // a split of the layer's FP8 window rows (kLocalRowsPerSplit of them),
    // attended like the sparse rows and merged by the same combine
    const int32_t p = q_pos[q];
    const int nall = min(window, p + 1);
    const int first = (split - sparse_splits) * kLocalRowsPerSplit;
    const int count = max(0, min(kLocalRowsPerSplit, nall - first));
    const int64_t sbase = (int64_t)q_seq[q] * window;
    const int nsub = fill_window_rows(lpos, sbase, window, p, nall, first, count, rows, tid, kThreads);
    f16x8 qf[4];
    load_q(qg, q, n_heads, wave, l16, g, q_negate, qf);
    __syncthreads();
    f32x4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = {0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;
    for (int c = 0; c < nsub; ++c) {
      stage_local<kThreads>(lk, lv, sbase, rows, c * kSub, kq, vt, tid);
      __syncthreads();
      attend_sub<kPitch>(kq, vt, rows, c * kSub, qf, scale_log2, g, l16, lane, m_run, l_run, o);
      __syncthreads();
    }
    store_partial(part_acc, part_ml, q, splits, split, n_heads, wave * 16 + l16, g, o, m_run, l_run);
    return;
  }
  const int64_t seq_base = (int64_t)q_seq[q] * capacity;
  const uint8_t *codes = kv_codes + seq_base * 128;
  const uint8_t *scales = kv_scales + seq_base * 16;
  const int row0 = split * rows_per_split;
  const int nrows = min(rows_per_split, top_k - row0);
  const int nsub = (nrows + kSub - 1) / kSub;

  // the query's rows of Q first (their loads overlap the row list's)
  uint4 qraw[4];
  load_q_raw(qg, q, n_heads, wave, l16, g, qraw);
  const int32_t *srow = topk + (int64_t)q * top_k + row0;
  // (kDense) entry r of the split's row list, -1 past its end
  auto row_at = [&](int r) -> int32_t { return r < nrows ? srow[r] : -1; };
  int32_t pend = -1;   // (kDense) thread tid < kSub: its entry of the next sub-chunk for the ring
  if constexpr (kDense) {
    // sub-chunks 0 and 1 into ring slots 0 and 1; sub-chunk 2's entry pending
    if (tid < 2 * kSub) rows[tid] = row_at(tid);
    if (tid < kSub) pend = row_at(2 * kSub + tid);
  } else {
    // the split's row list (and -1 for two sub-chunks past its end, which the
    // look-ahead gathers read), eight entries per thread per batch of loads:
    // branch-free (an index clamped into the split), so that a batch is in
    // flight together
    const int nslots = (nsub + 2) * kSub;
    for (int r0 = 0; r0 < nslots; r0 += 8 * kThreads) {
      int32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = srow[min(r0 + u * kThreads + tid, nrows - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = r0 + u * kThreads + tid;
        if (r < nslots) rows[r] = r < nrows ? v[u] : -1;
      }
    }
  }
  f16x8 qf[4];
  convert_q(qraw, q_negate, qf);
  __syncthreads();

  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = {0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY;   // for head 16*wave + l16 (same in all four lane groups)
  float l_run = 0.0f;

  if constexpr (kDense) {
    // ring slot s & 3 holds sub-chunk s; at iteration c slot (c + 2) & 3 (last
    // read for sub-chunk c - 2) takes sub-chunk c + 2, read first by the
    // gather of iteration c + 1
    Gathered<kThreads> ga;
    gather(ga, rows, 0, codes, scales, tid);
    for (int c = 0; c < nsub; ++c) {
      __syncthreads();   // the previous sub-chunk's readers are done with the stage
      if (tid < kSub) {
        rows[((c + 2) & 3) * kSub + tid] = pend;
        pend = row_at((c + 3) * kSub + tid);
      }
      dequant<kThreads, kPitch>(ga, kq, vt, tid);
      gather(ga, rows + ((c + 1) & 3) * kSub, 0, codes, scales, tid);
      __syncthreads();
      attend_sub<kPitch>(kq, vt, rows + (c & 3) * kSub, 0, qf, scale_log2, g, l16, lane, m_run, l_run, o);
    }
  } else {
    // The codes of sub-chunk c are gathered two sub-chunks ahead, into register
    // set c & 1 (the loop is unrolled by two so that each set is a fixed
    // register array): no branch around a gather and no copy between sets, so
    // the compiler waits only for the set being dequantized.
    Gathered<kThreads> ga, gb;
    gather(ga, rows, 0, codes, scales, tid);
    gather(gb, rows, kSub, codes, scales, tid);
    for (int c = 0; c < nsub; c += 2) {
      __syncthreads();   // the previous sub-chunk's readers are done with the stage
      dequant<kThreads, kPitch>(ga, kq, vt, tid);
      gather(ga, rows, (c + 2) * kSub, codes, scales, tid);
      __syncthreads();
      attend_sub<kPitch>(kq, vt, rows, c * kSub, qf, scale_log2, g, l16, lane, m_run, l_run, o);
      if (c + 1 >= nsub) break;
      __syncthreads();
      dequant<kThreads, kPitch>(gb, kq, vt, tid);
      gather(gb, rows, (c + 3) * kSub, codes, scales, tid);
      __syncthreads();
      attend_sub<kPitch>(kq, vt, rows, (c + 1) * kSub, qf, scale_log2, g, l16, lane, m_run, l_run, o);
    }
  }

  // O^T tile dt: this lane's head 16*wave + l16, channels 16 dt + 4g + 0..3
  const int head = wave * 16 + l16;
  if (splits == 1) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float *oq = out + ((int64_t)q * n_heads + head) * 128 + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4 *>(oq + dt * 16) = o[dt] * inv;
    if (lse != nullptr && g == 0)
      lse[(int64_t)q * n_heads + head] = l_run > 0.0f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    return;
  }
  store_partial(part_acc, part_ml, q, splits, split, n_heads, head, g, o, m_run, l_run);
}

// One workgroup per (query, 4 heads): thread (head, d) merges every split.
// Every load is issued before its value is needed: the outputs of the
// thread's channel in batches of kCombineBatch splits (the first batch before
// the statistics), the split statistics one per lane of the head's first
// wave, so that the usual split counts take a single round of loads.
__global__ void __launch_bounds__(512) attn_combine_kernel(
    const float *__restrict__ part_acc, const float2 *__restrict__ part_ml, int32_t n_heads,
    int32_t splits, float *__restrict__ out, float *__restrict__ lse) {
  constexpr int kHeadsPer = 4;
  constexpr int kStatPerLane = kMaxSplits / 64;
  __shared__ float w_sh[kHeadsPer][kMaxSplits];   // exp2(m_s - max) per split
  __shared__ float inv_sh[kHeadsPer];
  __shared__ float lse_sh[kHeadsPer];
  const int q = blockIdx.y;
  const int hl = threadIdx.x >> 7;
  const int h = blockIdx.x * kHeadsPer + hl;
  const int d = threadIdx.x & 127;
  const float2 *ml = part_ml + (int64_t)q * splits * n_heads + h;
  const float *pa = part_acc + ((int64_t)q * splits * n_heads + h) * 128 + d;
  const int64_t sstride = (int64_t)n_heads * 128;
  float a[kCombineBatch];
#pragma unroll
  for (int u = 0; u < kCombineBatch; ++u) a[u] = u < splits ? pa[u * sstride] : 0.0f;
  if (d < 64) {
    // the split statistics of head h: overall max, weights and normalizer
    float2 v[kStatPerLane];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kStatPerLane; ++u) {
      const int sp = d + 64 * u;
      v[u] = sp < splits ? ml[(int64_t)sp * n_heads] : make_float2(-INFINITY, 0.0f);
      mx = fmaxf(mx, v[u].x);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float tot = 0.0f;
#pragma unroll
    for (int u = 0; u < kStatPerLane; ++u) {
      const int sp = d + 64 * u;
      const float w = v[u].x == -INFINITY ? 0.0f : exp2f(v[u].x - mx);
      if (sp < splits) w_sh[hl][sp] = w;
      tot += w * v[u].y;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o, 64);
    if (d == 0) {
      inv_sh[hl] = tot > 0.0f ? 1.0f / tot : 0.0f;
      lse_sh[hl] = tot > 0.0f ? (mx + log2f(tot)) * kLn2 : -INFINITY;
    }
  }
  __syncthreads();
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < kCombineBatch; ++u)
    if (u < splits) acc += w_sh[hl][u] * a[u];
  for (int s0 = kCombineBatch; s0 < splits; s0 += kCombineBatch) {
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)
      a[u] = s0 + u < splits ? pa[(int64_t)(s0 + u) * sstride] : 0.0f;
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)
      if (s0 + u < splits) acc += w_sh[hl][s0 + u] * a[u];
  }
  const int64_t oi = (int64_t)q * n_heads + h;
  out[oi * 128 + d] = acc * inv_sh[hl];
  if (lse != nullptr && d == 0) lse[oi] = lse_sh[hl];
}

// The local window branch (aiwiki "DeepSeek V4.1-Flash", "Compressed Sparse
// Attention 2": every layer's own sliding-window K and V; "KV-cache formats
// and bounded replay": kept in FP8).  One workgroup per query, one wave per 16
// heads; the window's rows (ascending positions, -1 where the slot holds
// another position) in sub-chunks of 64: the E4M3 codes convert exactly to
// fp16 into the LDS layouts of the FP4 path and attend_sub runs over them.
// The result is merged into the sparse branch's (out, lse) in place:
//   lse = ln(e^lse_s + e^lse_l),
//   out = out_s e^(lse_s - lse) + out_l e^(lse_l - lse).
template <int kWaves>
__global__ void __launch_bounds__(kWaves * 64) local_attn_kernel(
    const uint8_t *__restrict__ lk, const uint8_t *__restrict__ lv,
    const int32_t *__restrict__ lpos, int32_t window, const uint16_t *__restrict__ qg,
    int32_t n_heads, const int32_t *__restrict__ q_seq, const int32_t *__restrict__ q_pos,
    float scale_log2, bool q_negate, float *__restrict__ out, float *__restrict__ lse) {
  constexpr int kThreads = kWaves * 64;
  __shared__ int32_t rows[kMaxLocalWindow + kSub];   // slot of each row, -1: no row
  __shared__ uint4 kq[4 * 4 * 64];
  constexpr int kPitch = kVtPitch;
  __shared__ __attribute__((aligned(16))) _Float16 vt[128 * kPitch];

  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int32_t p = q_pos[q];
  const int nall = min(window, p + 1);   // positions p - nall + 1 .. p
  const int64_t sbase = (int64_t)q_seq[q] * window;
  const int nsub = fill_window_rows(lpos, sbase, window, p, nall, 0, nall, rows, tid, kThreads);
  f16x8 qf[4];
  load_q(qg, q, n_heads, wave, l16, g, q_negate, qf);
  __syncthreads();

  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = {0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY;
  float l_run = 0.0f;
  for (int c = 0; c < nsub; ++c) {
    stage_local<kThreads>(lk, lv, sbase, rows, c * kSub, kq, vt, tid);
    __syncthreads();
    attend_sub<kPitch>(kq, vt, rows, c * kSub, qf, scale_log2, g, l16, lane, m_run, l_run, o);
    __syncthreads();   // the stage is rewritten next
  }

  // merge into the sparse branch's result (natural-log lse)
  const int head = wave * 16 + l16;
  const int64_t hi = (int64_t)q * n_heads + head;
  const float lse_l = l_run > 0.0f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  const float lse_s = lse[hi];
  const float mx = fmaxf(lse_s, lse_l);
  if (mx == -INFINITY) return;   // no row in either set: out stays 0, lse -inf
  const float ws = lse_s == -INFINITY ? 0.0f : expf(lse_s - mx);
  const float wl = lse_l == -INFINITY ? 0.0f : expf(lse_l - mx);
  const float den = ws + wl;
  const float cs = ws / den;
  const float cl = l_run > 0.0f ? (wl / den) / l_run : 0.0f;
  float *oq = out + hi * 128 + 4 * g;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    f32x4 *po = reinterpret_cast<f32x4 *>(oq + dt * 16);
    *po = *po * cs + o[dt] * cl;
  }
  if (g == 0) lse[hi] = mx + logf(den);
}

// Rows per split: as many as possible (one split needs no combine) while the
// grid still has kTargetGroups workgroups, at most kMaxRowsPerSplit, a
// multiple of the sub-chunk.  Splits of one sub-chunk become two (whose
// gathers overlap) when that still leaves kTwoSubMinGroups workgroups.
int32_t rows_per_split(int32_t nq, int32_t top_k, int32_t max_splits) {
  const int32_t subs = (top_k + kSub - 1) / kSub;
  const int32_t nq1 = std::max(nq, 1);   // a size query may ask for no queries
  int32_t splits = std::min((kTargetGroups + nq1 - 1) / nq1, max_splits);
  splits = std::max(1, std::min(splits, subs));
  if (subs / splits < 2 && (int64_t)nq * (subs / 2) >= kTwoSubMinGroups)
    splits = std::max(1, subs / 2);
  int32_t per = (subs + splits - 1) / splits;
  per = std::min(per, kMaxRowsPerSplit / kSub);
  return per * kSub;
}

// Scratch of csa2_sparse_attn_noalloc (callers that cannot allocate): the
// split partials live in this file-scope array instead of a caller workspace.
// Every device the library runs on holds its own copy until the process ends;
// host code reaches a device's copy only through the address that
// hipGetSymbolAddress returns on that device (the array's name is a host-side
// stand-in, not a device address).
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
uint8_t *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(uint8_t **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // once per device, with that device current (this thread's current device)
  std::call_once(g_scratch_once[dev], [dev] {
    void *p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = static_cast<uint8_t *>(p);
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

AttnWorkspace attn_workspace_layout(const csa2_cache &c, int32_t nq, int32_t n_heads,
                                    int32_t top_k, int32_t window) {
  AttnWorkspace w;
  w.local_splits = window > 0 ? (window + kLocalRowsPerSplit - 1) / kLocalRowsPerSplit : 0;
  const int32_t rps = rows_per_split(nq, top_k, kMaxSplits - w.local_splits);
  w.splits = (top_k + rps - 1) / rps;
  // sparse splits <= max(kMaxSplits - local splits, top_k / kMaxRowsPerSplit), and
  // top_k / kMaxRowsPerSplit <= 32 for top_k <= 65536: the total stays <= kMaxSplits.
  // A single split writes the final results directly (no partials).
  const int32_t total = w.splits + w.local_splits;
  const size_t units = total > 1 ? (size_t)nq * total * n_heads : 0;
  w.part_acc = 0;
  w.part_ml = align256(units * c.dv * sizeof(float));
  w.total = std::max<size_t>(256, align256(w.part_ml + units * sizeof(float2)));
  return w;
}

hipError_t launch_sparse_attn(const csa2_cache &c, const uint16_t *q, int32_t n_heads,
                              const int32_t *q_seq, int32_t nq, const int32_t *topk,
                              int32_t top_k, float softmax_scale, float *out, float *lse,
                              uint8_t *ws, const AttnWorkspace &L, hipStream_t s,
                              const csa2_local_cache *lc, const int32_t *q_pos) {
  float *acc = reinterpret_cast<float *>(ws + L.part_acc);
  float2 *ml = reinterpret_cast<float2 *>(ws + L.part_ml);
  const float scale_log2 = fabsf(softmax_scale) * kLog2e;
  const bool q_negate = softmax_scale < 0.0f;
  const int32_t rps = rows_per_split(nq, top_k, kMaxSplits - L.local_splits);
  const int32_t total = L.splits + L.local_splits;
  if (total > kMaxSplits || (L.local_splits > 0 && (lc == nullptr || q_pos == nullptr)))
    return hipErrorInvalidValue;
  const uint8_t *lk = lc ? lc->k : nullptr, *lv = lc ? lc->v : nullptr;
  const int32_t *lpos = lc ? lc->pos : nullptr;
  const int32_t window = lc ? lc->window : 0;
  dim3 grid((unsigned)total, (unsigned)nq);
  const int waves = n_heads / 16;
  if (waves == 4 && L.local_splits == 0 && (int64_t)nq * total >= kDenseMinGroups) {
    hipLaunchKernelGGL((attn_partial_kernel<4, false, true>), grid, dim3(4 * 64), 0, s,
                       c.kv_codes, c.kv_scales, (int64_t)c.capacity, q, n_heads, q_seq, topk,
                       top_k, rps, scale_log2, q_negate, acc, ml, total, out, lse, L.splits, lk,
                       lv, lpos, window, q_pos);
    if (total == 1) return hipGetLastError();
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(n_heads / 4), (unsigned)nq), dim3(512),
                       0, s, acc, ml, n_heads, total, out, lse);
    return hipGetLastError();
  }
#define CSA2_ATTN_CASE(W)                                                                        \
  case W:                                                                                        \
    if (L.local_splits > 0)                                                                      \
      hipLaunchKernelGGL((attn_partial_kernel<W, true>), grid, dim3(W * 64), 0, s, c.kv_codes,   \
                         c.kv_scales, (int64_t)c.capacity, q, n_heads, q_seq, topk, top_k, rps,  \
                         scale_log2, q_negate, acc, ml, total, out, lse, L.splits, lk, lv, lpos, \
                         window, q_pos);                                                         \
    else                                                                                         \
      hipLaunchKernelGGL((attn_partial_kernel<W, false>), grid, dim3(W * 64), 0, s, c.kv_codes,  \
                         c.kv_scales, (int64_t)c.capacity, q, n_heads, q_seq, topk, top_k, rps,  \
                         scale_log2, q_negate, acc, ml, total, out, lse, L.splits, lk, lv, lpos, \
                         window, q_pos);                                                         \
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
  if (total == 1) return hipGetLastError();
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(n_heads / 4), (unsigned)nq), dim3(512),
                     0, s, acc, ml, n_heads, total, out, lse);
  return hipGetLastError();
}

hipError_t launch_local_attn(const csa2_local_cache &c, const uint16_t *q, int32_t n_heads,
                             const int32_t *q_seq, const int32_t *q_pos, int32_t nq,
                             float softmax_scale, float *out, float *lse, hipStream_t s) {
  const float scale_log2 = fabsf(softmax_scale) * kLog2e;
  const bool q_negate = softmax_scale < 0.0f;
#define CSA2_LOCAL_CASE(W)                                                                       \
  case W:                                                                                        \
    hipLaunchKernelGGL(local_attn_kernel<W>, dim3((unsigned)nq), dim3(W * 64), 0, s, c.k, c.v,   \
                       c.pos, c.window, q, n_heads, q_seq, q_pos, scale_log2, q_negate, out, lse); \
    break;
  switch (n_heads / 16) {
    CSA2_LOCAL_CASE(1)
    CSA2_LOCAL_CASE(2)
    CSA2_LOCAL_CASE(3)
    CSA2_LOCAL_CASE(4)
    CSA2_LOCAL_CASE(5)
    CSA2_LOCAL_CASE(6)
    CSA2_LOCAL_CASE(7)
    CSA2_LOCAL_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef CSA2_LOCAL_CASE
  return hipGetLastError();
}

}  // namespace csa2
