// Index scoring, Top-K and the candidate pool, in Full / Reindex / Reuse mode.
//
// aiwiki "DeepSeek V4.1-Flash", section "Compressed Sparse Attention 2": a Full
// layer scores every causally visible position with its index query and makes
// a fresh Top-K; a Reindex layer scores an earlier layer's index keys with its
// own query; a Reuse layer recycles the latest compatible Top-K.  The decoder's
// first Full layer also ranks blocks of eight positions by their maximum index
// score and keeps the best as a shared candidate pool that later Reindex
// layers search.  Model card, Introduction, CSA2 paragraph: the hierarchical
// indexer bounds the deeper indexers' cost by the pool size.
//
// Kernels, in launch order for one call:
//   zero2_u32_kernel clear the per-query histograms
//   score_kernel     (Full, or Reindex without a pool; gather_score_kernel for
//                    a Reindex pool) stream the (tiled) index keys, compute the canonical fp32
//                    score of each candidate, keep its order-preserving key
//                    (written out per workgroup in one burst), histogram the
//                    top 12 key bits, and for a pool-building Full layer the
//                    8-position block maxima and their histogram.
//   filter_kernel    per wave and 512 or 1024 keys: keep every key whose top 12 bits
//                    reach b1 -- the bin of the 12-bit histogram holding the
//                    K-th largest key, which each workgroup reads off the
//                    histogram itself -- with its index, in index order
//                    (ballot compaction)
//   resolve_kernel   per query: the candidates (typically K plus one bin) in
//                    LDS; radix passes on bits 19..8 and 7..0 within bin b1 give
//                    the K-th largest key tau; an ordered compaction emits every
//                    key > tau and the first ties == tau, ascending, -1 padded.
//                    With more candidates than LDS holds (heavy ties) it
//                    streams the full key array with the same logic.
//                    A pool-building Full layer selects its pool blocks in the
//                    same filter and resolve launches (a second grid slice).
//                    Key arrays of at most kDirectMax entries (a Reindex pool)
//                    skip the filter: the resolve reads them, builds their
//                    histogram in LDS and compacts them (such a pool's scorer
//                    builds no global histogram, and nothing is cleared).
// Small score chunks (one wave) count keys straight into the global histogram.
//   copy_i32_kernel  Reuse mode: topk_out = reuse_src.
// The selection helpers (select_bin, select_core, gather_regions) live in
// csa2_select.h; E4M3 index queries against E4M3 keys over every visible
// position go to the matrix-core scorer in csa2_index_gemm.hip instead.
#include <algorithm>

#include "csa2_select.h"

namespace csa2 {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFilterThreads = 1024;      // few, wide workgroups: each derives the threshold bin
// Keys per filter wave (one candidate slot region): 512, or 1024 for key
// arrays past kFilterSmallMax keys, so that the resolve's one round of early
// slot reads covers every region (at most one region per resolve thread).
constexpr int kFilterSubMin = 512;
constexpr int kFilterSubMax = 1024;
constexpr int64_t kFilterSmallMax = (int64_t)kFilterSubMin * 1024;
constexpr int64_t kDirectMax = 32768;      // up to this many keys the resolve filters them itself
constexpr int kEarlySlots = 8;             // candidate slots per resolve thread read before the counts
// Keys in the threshold bin beyond which the filter leaves the bits 19..8 pass
// to the resolve (heavy ties would serialize the global atomics).
constexpr uint32_t kH2MaxKeys = 8192;

#ifndef CSA2_SCORE_UNROLL
#define CSA2_SCORE_UNROLL 4            // 16-B loads per lane per prefetch batch
#endif
#ifndef CSA2_SCORE_WAVES
#define CSA2_SCORE_WAVES 4             // waves per SIMD the register budget allows
#endif

// Score launch shapes: (threads, candidates per workgroup).
constexpr int64_t kBigChunkMinGroups = 512;   // use 4096-candidate chunks when >= this many groups
constexpr int64_t kSmallGridGroups = 256;     // below this, one-wave groups of 64 candidates

// ---------------------------------------------------------------------------
// cross-lane sums inside quads / half rows (commutative, so both lanes of a
// butterfly pair compute the same bits)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}
// lane i <-> 7 - i within each group of 8: pairs quad 0 with quad 1
__device__ __forceinline__ float dpp_half_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
}

__global__ void zero2_u32_kernel(uint32_t *__restrict__ p, uint32_t *__restrict__ p2, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += step) {
    p[i] = 0u;
    if (p2 != nullptr) p2[i] = 0u;
  }
}

__global__ void copy_i32_kernel(int32_t *__restrict__ dst, const int32_t *__restrict__ src,
                                int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += step) dst[i] = src[i];
}


// ---------------------------------------------------------------------------
// score_kernel
//
// Lane layout: lane l owns head h = l % H of token l / H, i.e. 64 channels =
// 64 B (E4M3) or 128 B (bf16) of the token's index keys; a wave covers
// TPI = 64 / H tokens per step = one tile of the tiled index-key layout, so
// each of its 16-B loads is one contiguous 1 KB span across the wave.  Each
// lane runs the canonical fp32 chains -- per 16-channel block, fused
// multiply-adds in channel order -- as four independent chains, adds the
// block sums as (b0+b1)+(b2+b3), and the head sums meet in a balanced tree
// over lanes: xor-1, xor-2 (quad permutes) and xor-4 (half-row mirror; the
// quads are uniform by then) DPP adds.  Every lane of a token ends with the
// same bits.
// ---------------------------------------------------------------------------
template <int H, bool kFp8Keys, bool kPool, int kThreads, int kChunk>
struct ScoreCtx {
  // Small chunks count their keys straight into the query's global histogram
  // (one atomic per key) instead of clearing and flushing 4096 LDS bins.
  static constexpr bool kDirectHist = kChunk <= kWave && !kPool;
  static constexpr int kEsz = kFp8Keys ? 1 : 2;
  static constexpr int TPI = kWave / H;
  static constexpr int kLoads = 4 * kEsz;
  static constexpr int kNumWaves = kThreads / kWave;
  const uint8_t *seq_base;
  int32_t qp;
  int64_t t_begin, t_end;
  int wave, h, tl, lane;
  uint32_t *ghist;         // the query's global histogram (kDirectHist)

  // Step s of this wave covers tile s * kNumWaves + wave of the chunk, so at
  // any step the workgroup's waves read adjacent tiles (one moving window).
  __device__ __forceinline__ int64_t tile_start(int s) const {
    return t_begin + ((int64_t)s * kNumWaves + wave) * TPI;
  }
  __device__ __forceinline__ int64_t token(int s) const { return tile_start(s) + tl; }

  // loads of steps s0 .. s0+U-1; lanes past the end (or on an empty pool
  // slot) read an in-bounds row and are masked
  template <int U>
  __device__ __forceinline__ void issue(int s0, uint4 (&buf)[U][kLoads], bool (&val)[U]) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = token(s0 + u);
      const bool valid = t < t_end;
      const int64_t row = valid ? t : t_begin;
      val[u] = valid;
      // Full mode: row % TPI == tl, so a wave's loads cover one tile contiguously.
      // Every key is read once: non-temporal loads keep the stream from
      // churning the L2 (measured +14-17% bandwidth).
      const uint8_t *src = seq_base + idx_chunk_offset<H, kEsz>(row, h, 0);
#pragma unroll
      for (int v = 0; v < kLoads; ++v) {
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + v * 1024));
        buf[u][v] = make_uint4(t.x, t.y, t.z, t.w);
      }
    }
  }

  // canonical score of steps s0 .. s0+U-1; closes a group after its last step
  template <int U>
  __device__ __forceinline__ void score(int s0, const uint4 (&buf)[U][kLoads], const bool (&val)[U],
                                        const float (&qf)[64], uint32_t &mykey, uint32_t *skeys,
                                        uint32_t *hist, uint32_t *sblk, uint32_t *histb) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float blk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float acc = 0.0f;
        if (kFp8Keys) {
          const uint4 a = buf[u][j];
          const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[k], false);
            auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[k], true);
            acc = __builtin_fmaf(qf[16 * j + 4 * k + 0], lo[0], acc);
            acc = __builtin_fmaf(qf[16 * j + 4 * k + 1], lo[1], acc);
            acc = __builtin_fmaf(qf[16 * j + 4 * k + 2], hi[0], acc);
            acc = __builtin_fmaf(qf[16 * j + 4 * k + 3], hi[1], acc);
          }
        } else {
#pragma unroll
          for (int hv = 0; hv < 2; ++hv) {
            const uint4 a = buf[u][2 * j + hv];
            const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              acc = __builtin_fmaf(qf[16 * j + 8 * hv + 2 * k], __uint_as_float(w[k] << 16), acc);
              acc = __builtin_fmaf(qf[16 * j + 8 * hv + 2 * k + 1],
                                   __uint_as_float(w[k] & 0xFFFF0000u), acc);
            }
          }
        }
        blk[j] = acc;
      }
      float acc = (blk[0] + blk[1]) + (blk[2] + blk[3]);
      acc = acc + dpp_xor1(acc);
      acc = acc + dpp_xor2(acc);
      if (H == 8) acc = acc + dpp_half_mirror(acc);
      const uint32_t key = val[u] ? score_key(acc) : 0u;
      const int s = s0 + u;
      mykey = (h == s % H) ? key : mykey;
      if (s % H == H - 1) close_group(s / H, mykey, skeys, hist, sblk, histb);
    }
  }

  // lane (tl, h) holds the key of step grp*H + h, token tl; permute so that
  // lane l holds step grp*H + l/TPI, token l%TPI, then stage its key in LDS,
  // count it, and take the 8-position block maxima (8 consecutive lanes = 8
  // positions).  Histogram bins are 16-bit halves of LDS words.
  __device__ __forceinline__ void close_group(int grp, uint32_t mykey, uint32_t *skeys,
                                              uint32_t *hist, uint32_t *sblk, uint32_t *histb) const {
    const uint32_t key = (uint32_t)__shfl((int)mykey, (lane % TPI) * H + lane / TPI, kWave);
    const int64_t t = tile_start(grp * H + lane / TPI) + lane % TPI;
    if (t < t_end) {
      skeys[t - t_begin] = key;
      if (kDirectHist)
        atomicAdd(&ghist[key >> 20], 1u);
      else
        atomicAdd(&hist[key >> 21], 1u << ((key >> 16) & 16u));
    }
    if (kPool) {
      // block maximum over lanes 8b..8b+7 (keys of tokens past the end count as 0)
      uint32_t m = t < t_end ? key : 0u;
      m = max(m, shfl_xor_u(m, 1));
      m = max(m, shfl_xor_u(m, 2));
      m = max(m, shfl_xor_u(m, 4));
      if ((lane & (kPoolBlock - 1)) == 0 && t < t_end) {
        sblk[(t - t_begin) / kPoolBlock] = m;
        atomicAdd(&histb[m >> 21], 1u << ((m >> 16) & 16u));
      }
    }
  }
};

template <int H, bool kFp8Keys, bool kPool, int kThreads, int kChunk>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kThreads == 64 ? 2 : (kFp8Keys ? CSA2_SCORE_WAVES : CSA2_SCORE_WAVES - 1))))
score_kernel(
    const uint8_t *__restrict__ idx_k, int64_t capacity, const uint16_t *__restrict__ q_idx,
    int32_t q_fp8, const int32_t *__restrict__ q_seq, const int32_t *__restrict__ q_pos,
    uint32_t *__restrict__ keys_tok, int64_t tok_stride, uint32_t *__restrict__ hist_tok,
    uint32_t *__restrict__ keys_blk, int64_t blk_stride, uint32_t *__restrict__ hist_blk,
    int64_t hstride, int32_t hcopies) {
  constexpr int kEsz = kFp8Keys ? 1 : 2;
  constexpr int TPI = kWave / H;
  constexpr int kBpt = H * 64 * kEsz;     // bytes per token
  constexpr int kLoads = 4 * kEsz;        // 16-B loads per lane per token (64 channels)
  constexpr int kNumWaves = kThreads / kWave;
  constexpr int kUnroll = CSA2_SCORE_UNROLL / kLoads > 0 ? CSA2_SCORE_UNROLL / kLoads : 1;
  static_assert(kChunk % (kWave * kNumWaves) == 0, "chunk shape");
  constexpr int kMainWords = kHistBins / 2 + kChunk;

  // LDS: 16-bit histogram bins packed in pairs, the chunk's keys (written out
  // in one burst at the end: small stores interleaved with the read stream
  // cost HBM efficiency), block maxima, the index query.
  __shared__ uint32_t lds_main[kMainWords];
  __shared__ uint32_t histb[kPool ? kHistBins / 2 : 1];
  __shared__ uint32_t sblk[kPool ? kChunk / kPoolBlock : 1];
  __shared__ float qlds[H * 64];
  uint32_t *hist = lds_main;
  uint32_t *skeys = lds_main + kHistBins / 2;

  const int q = blockIdx.y;
  const int32_t qp = q_pos[q];
  const int64_t n = (int64_t)qp + 1;
  const int64_t t_begin = (int64_t)blockIdx.x * kChunk;
  if (t_begin >= n) return;
  const int64_t t_end = min(n, t_begin + kChunk);

  using Ctx = ScoreCtx<H, kFp8Keys, kPool, kThreads, kChunk>;
  // this workgroup's copy of the query's histogram(s)
  const int64_t hoff = (int64_t)q * hstride + (int64_t)(blockIdx.x % hcopies) * kHistBins;
  uint32_t *hq = hist_tok + hoff;
  if (!Ctx::kDirectHist) {
    for (int i = threadIdx.x; i < kHistBins / 2; i += kThreads) {
      hist[i] = 0u;
      if (kPool) histb[i] = 0u;
    }
  }
  // the index query as scored (bf16, or cast to E4M3), staged once through LDS
  for (int i = threadIdx.x; i < H * 64; i += kThreads) {
    float f = bf16_to_f32(q_idx[(int64_t)q * H * 64 + i]);
    if (q_fp8) f = e4m3_to_f32(e4m3_from_f32_nonneg(fabsf(f)) | ((__float_as_uint(f) >> 24) & 0x80u));
    qlds[i] = f;
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int h = lane % H;
  const int tl = lane / H;
  float qf[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) qf[i] = qlds[h * 64 + i];

  // tiled index keys: the lane slot of (position-in-tile tl, head h) is `lane`
  const uint8_t *seq_base = idx_k + (int64_t)q_seq[q] * capacity * kBpt;

  // The wave walks its steps (one tile each; H steps make a group of 64
  // tokens) with a ping-pong prefetch: the loads of the next kUnroll steps are
  // in flight while the current ones are scored.  Every issue is
  // unconditional (steps past the end read a masked in-bounds tile): with no
  // branch around a prefetch the compiler waits only for the batch being
  // scored.
  const int64_t ntiles = (t_end - t_begin + TPI - 1) / TPI;
  const int64_t wave_steps = (ntiles + kNumWaves - 1) / kNumWaves;
  const int nsteps = (int)((wave_steps + H - 1) / H * H);
  Ctx cx{seq_base, qp, t_begin, t_end, wave, h, tl, lane, hq};
  uint4 bufA[kUnroll][kLoads], bufB[kUnroll][kLoads];
  bool valA[kUnroll], valB[kUnroll];
  uint32_t mykey = 0u;
  static_assert(H % (2 * kUnroll) == 0, "steps per group must be a multiple of the ping-pong");
  if (nsteps > 0) {
    cx.template issue<kUnroll>(0, bufA, valA);
    for (int s0 = 0; s0 < nsteps; s0 += 2 * kUnroll) {
      cx.template issue<kUnroll>(s0 + kUnroll, bufB, valB);
      cx.template score<kUnroll>(s0, bufA, valA, qf, mykey, skeys, hist, sblk, histb);
      cx.template issue<kUnroll>(s0 + 2 * kUnroll, bufA, valA);
      cx.template score<kUnroll>(s0 + kUnroll, bufB, valB, qf, mykey, skeys, hist, sblk, histb);
    }
  }
  __syncthreads();

  // the chunk's keys and block maxima in one burst of coalesced stores
  const int64_t cnt = t_end - t_begin;
  {
    uint32_t *dst = keys_tok + (int64_t)q * tok_stride + t_begin;
    for (int64_t i = threadIdx.x; i < cnt; i += kThreads) dst[i] = skeys[i];
    if (kPool) {
      const int64_t nb = (cnt + kPoolBlock - 1) / kPoolBlock;
      uint32_t *db = keys_blk + (int64_t)q * blk_stride + t_begin / kPoolBlock;
      for (int64_t i = threadIdx.x; i < nb; i += kThreads) db[i] = sblk[i];
    }
  }
  if (Ctx::kDirectHist) return;
  uint32_t *hbq = kPool ? hist_blk + hoff : nullptr;
  for (int i = threadIdx.x; i < kHistBins / 2; i += kThreads) {
    const uint32_t w = hist[i];
    if (w & 0xFFFFu) atomicAdd(&hq[2 * i], w & 0xFFFFu);
    if (w >> 16) atomicAdd(&hq[2 * i + 1], w >> 16);
    if (kPool) {
      const uint32_t b = histb[i];
      if (b & 0xFFFFu) atomicAdd(&hbq[2 * i], b & 0xFFFFu);
      if (b >> 16) atomicAdd(&hbq[2 * i + 1], b >> 16);
    }
  }

}

// ---------------------------------------------------------------------------
// gather_score_kernel: Reindex over a pool.  Each pool entry takes H lanes,
// one per index head: lane h gathers the entry's head-h keys (all its 16-B
// pieces in flight at once; the pool's positions are scattered, so there is
// nothing to coalesce across entries) and runs the canonical fp32 order of
// that head -- per 16-channel block an FMA chain in channel order, blocks
// (b0+b1)+(b2+b3).  The heads' balanced pairwise tree then runs across the H
// lanes with DPP moves (each level adds a lane's value to its partner's, so
// both partners hold the same bits): the same bits as score_kernel.  The
// group's first lane stores the key; the 12-bit histogram is aggregated in
// LDS, where only the bins in use are cleared and flushed.
// ---------------------------------------------------------------------------
constexpr int kGatherThreads = 256;
constexpr int kQPitch = 68;   // floats per head row of the staged query (spreads LDS banks)

template <int H, bool kFp8Keys>
__global__ void __launch_bounds__(kGatherThreads) gather_score_kernel(
    const uint8_t *__restrict__ idx_k, int64_t capacity, const uint16_t *__restrict__ q_idx,
    int32_t q_fp8, const int32_t *__restrict__ q_seq, const int32_t *__restrict__ q_pos,
    const int32_t *__restrict__ pool_in, int32_t pool_len, uint32_t *__restrict__ keys_tok,
    int64_t tok_stride, uint32_t *__restrict__ hist_tok, int64_t hstride, int32_t hcopies) {
  // hist_tok == nullptr: no global histogram (the resolve builds its own for a
  // pool it reads whole)
  constexpr int kEsz = kFp8Keys ? 1 : 2;
  constexpr int kLoads = 4 * kEsz;                   // 16-B pieces per head (64 channels)
  constexpr int kEntries = kGatherThreads / H;       // pool entries per workgroup
  __shared__ __attribute__((aligned(16))) float qlds[H * kQPitch];
  __shared__ __attribute__((aligned(16))) uint32_t lh[kHistBins];
  const int q = blockIdx.y;
  const int tid = threadIdx.x;
  const int h = tid % H;                             // this lane's head
  const int32_t qp = q_pos[q];
  const int64_t t = (int64_t)blockIdx.x * kEntries + tid / H;
  const bool in = t < pool_len;
  const int32_t p = in ? pool_in[(int64_t)q * pool_len + t] : -1;
  const bool valid = p >= 0 && p <= qp;
  const int64_t row = valid ? p : 0;
  const uint8_t *base = idx_k + (int64_t)q_seq[q] * capacity * (H * 64 * kEsz);
  for (int i = tid; i < H * 64; i += kGatherThreads) {
    float f = bf16_to_f32(q_idx[(int64_t)q * H * 64 + i]);
    if (q_fp8) f = e4m3_to_f32(e4m3_from_f32_nonneg(fabsf(f)) | ((__float_as_uint(f) >> 24) & 0x80u));
    qlds[(i / 64) * kQPitch + i % 64] = f;
  }

  uint4 buf[kLoads];
  {
    const uint8_t *src = base + idx_chunk_offset<H, kEsz>(row, h, 0);
#pragma unroll
    for (int v = 0; v < kLoads; ++v) buf[v] = *reinterpret_cast<const uint4 *>(src + v * 1024);
  }
  __syncthreads();
  const float *qh = qlds + h * kQPitch;
  float blk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float qv[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 f = *reinterpret_cast<const float4 *>(qh + 16 * j + 4 * k);
      qv[4 * k] = f.x;
      qv[4 * k + 1] = f.y;
      qv[4 * k + 2] = f.z;
      qv[4 * k + 3] = f.w;
    }
    float acc = 0.0f;
    if (kFp8Keys) {
      const uint4 a = buf[j];
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[k], false);
        auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[k], true);
        acc = __builtin_fmaf(qv[4 * k + 0], lo[0], acc);
        acc = __builtin_fmaf(qv[4 * k + 1], lo[1], acc);
        acc = __builtin_fmaf(qv[4 * k + 2], hi[0], acc);
        acc = __builtin_fmaf(qv[4 * k + 3], hi[1], acc);
      }
    } else {
#pragma unroll
      for (int hv = 0; hv < 2; ++hv) {
        const uint4 a = buf[2 * j + hv];
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc = __builtin_fmaf(qv[8 * hv + 2 * k], __uint_as_float(w[k] << 16), acc);
          acc = __builtin_fmaf(qv[8 * hv + 2 * k + 1], __uint_as_float(w[k] & 0xFFFF0000u), acc);
        }
      }
    }
    blk[j] = acc;
  }
  float hs = (blk[0] + blk[1]) + (blk[2] + blk[3]);
  // balanced pairwise tree over the heads, across the entry's lanes
  hs = hs + dpp_xor1(hs);
  hs = hs + dpp_xor2(hs);
  if (H == 8) hs = hs + dpp_half_mirror(hs);
  const uint32_t key = valid ? score_key(hs) : 0u;
  const bool lead = in && h == 0;
  if (lead) keys_tok[(int64_t)q * tok_stride + t] = key;
  if (hist_tok == nullptr) return;   // uniform

  const uint32_t bin = key >> 20;
  if (lead) lh[bin] = 0u;
  __syncthreads();
  if (lead) atomicAdd(&lh[bin], 1u);
  __syncthreads();
  if (lead) {
    const uint32_t c = atomicExch(&lh[bin], 0u);
    if (c)
      atomicAdd(&hist_tok[(int64_t)q * hstride + (int64_t)(blockIdx.x % hcopies) * kHistBins + bin], c);
  }
}

// One selection problem of a call: per query, the kk largest keys of an array
// (the scored candidates, or the pool blocks of a pool-building Full layer).
struct SelProblem {
  const uint32_t *keys;   // [nq][n_stride] order-preserving keys
  int64_t n_stride;
  uint32_t *hist;         // [nq][hstride]: histogram copies, state, second histogram
  int64_t hstride;
  int32_t hcopies;
  uint32_t *cand_key;     // [nq][cand_stride] filter output, one region per `region` keys
  int32_t *cand_id;
  int64_t cand_stride;
  uint32_t *cnt;          // [nq][nsub] candidates per region
  int64_t nsub;
  int32_t *out;           // [nq][out_stride]
  int64_t out_stride;
  int32_t kk;
  int32_t mode;           // OutMode
  int32_t direct;         // short arrays: no filter pass, the resolve reads the keys
  int32_t region;         // keys per filter wave: kFilterSubMin or kFilterSubMax
};

struct SelProblems {
  SelProblem p[2];
};

// grid (filter groups, nq, problems).  Each wave takes A.region keys and
// keeps every key whose top 12 bits reach bin b1, with its index, in index
// order, in its own slot region.  Every workgroup derives b1 from the query's
// histogram itself (16 KB from L2), so no separate pass is needed.  The keys
// of bin b1 itself also go into the query's second histogram (bits 19..8),
// unless the bin holds more than kH2MaxKeys of them; the first workgroup
// records (keff, b1, above, second histogram valid) in the query's state.
template <int kIters>   // largest region / 256 among the launch's problems
__global__ void __launch_bounds__(kFilterThreads) filter_kernel(
    const SelProblems P, const int32_t *__restrict__ q_pos, int32_t pool_len) {
  __shared__ __attribute__((aligned(16))) uint32_t lh[kHistBins];
  __shared__ uint32_t scratch[kFilterThreads / kWave + 1];
  __shared__ uint32_t res[4];
  const SelProblem &A = P.p[blockIdx.z];
  const int q = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t n = sel_len(A.mode, q_pos[q], pool_len);
  if (A.direct || (int64_t)blockIdx.x * (kFilterThreads / kWave) * A.region >= n) return;   // uniform
  // the wave's keys first (their loads overlap the threshold's)
  const int64_t sub = (int64_t)blockIdx.x * (kFilterThreads / kWave) + threadIdx.x / kWave;
  const int64_t start = sub * A.region;
  const uint32_t *kq = A.keys + (int64_t)q * A.n_stride;
  // region / 256 x 4 keys per lane; key (k, lane, e) sits at start + k*256 + lane*4 + e
  const int iters = A.region / 256;   // uniform, <= kIters
  uint32_t kv[kIters][4];
#pragma unroll
  for (int k = 0; k < kIters; ++k) {
    const int64_t i0 = start + k * 256 + lane * 4;
    if (k >= iters) {
#pragma unroll
      for (int e = 0; e < 4; ++e) kv[k][e] = 0u;
    } else if (i0 + 3 < n) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kq + i0));
      kv[k][0] = v.x;
      kv[k][1] = v.y;
      kv[k][2] = v.z;
      kv[k][3] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) kv[k][e] = i0 + e < n ? kq[i0 + e] : 0u;
    }
  }
  uint32_t *hs = A.hist + (int64_t)q * A.hstride;
  const Threshold th = hist_threshold(hs, A.hcopies, n, A.kk, lh, scratch, res);
  const bool use_h2 = th.keff > 0u && lh[th.b1] <= kH2MaxKeys;   // lh still holds the histogram
  if (blockIdx.x == 0 && threadIdx.x == 0)
    *reinterpret_cast<uint4 *>(hs + state_off(A.hcopies)) =
        make_uint4(th.keff, th.b1, th.above, use_h2 ? 1u : 0u);
  if (start >= n) return;
  const bool none = th.keff == 0u;
  const uint32_t thr = th.b1 << 20;
  uint32_t *h2 = hs + h2_off(A.hcopies);
  uint32_t *ck = A.cand_key + (int64_t)q * A.cand_stride + start;
  int32_t *ci = A.cand_id + (int64_t)q * A.cand_stride + start;
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t written = 0;
#pragma unroll
  for (int k = 0; k < kIters; ++k) {
    bool f[4];
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = start + k * 256 + lane * 4 + e;
      f[e] = !none && k < iters && i < n && kv[k][e] >= thr;
      const uint64_t b = __ballot(f[e]);
      before += __popcll(b & lt);
      total += __popcll(b);
    }
    uint32_t o = written + before;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (f[e]) {
        ck[o] = kv[k][e];
        ci[o] = (int32_t)(start + k * 256 + lane * 4 + e);
        ++o;
        if (use_h2 && (kv[k][e] >> 20) == th.b1) atomicAdd(&h2[(kv[k][e] >> 8) & 0xFFFu], 1u);
      }
    }
    written += total;
  }
  if (lane == 0) A.cnt[(int64_t)q * A.nsub + sub] = written;
}

// grid (nq, problems).  Per query: b1 from the histogram, the candidates of
// the filter's regions in index order into LDS, the radix passes and the
// ordered compaction; with more candidates than LDS holds (heavy ties) it
// streams the full key array instead.  Then the -1 padding.  The first slots
// of every region are read together with the histogram and the region counts,
// before the counts say how many of them hold candidates.
__global__ void __launch_bounds__(kSelectThreads) resolve_kernel(
    const SelProblems P, const int32_t *__restrict__ q_pos, const int32_t *__restrict__ pool_in,
    int32_t pool_len) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kHistBins];
  __shared__ uint32_t scratch[kSelectThreads / kWave + 1];
  __shared__ uint32_t res[4];
  __shared__ uint32_t lkey[kResolveCap];
  __shared__ int32_t lid[kResolveCap];
  __shared__ uint32_t goff[kSelectThreads];

  const SelProblem &A = P.p[blockIdx.y];
  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t qp = q_pos[q];
  const int64_t n = sel_len(A.mode, qp, pool_len);
  // A short key array is read here, in one batch of loads issued before the
  // histogram's (keys 4*tid + 4096*it .. +3 of iteration it).
  constexpr int kDirectIters = (int)(kDirectMax / (4 * kSelectThreads));
  const uint32_t *kq = A.keys + (int64_t)q * A.n_stride;
  uint4 kr[kDirectIters];
  if (A.direct) {
#pragma unroll
    for (int it = 0; it < kDirectIters; ++it) {
      const int64_t i0 = (int64_t)it * 4 * kSelectThreads + 4 * tid;
      kr[it] = i0 + 3 < n ? *reinterpret_cast<const uint4 *>(kq + i0) : make_uint4(0u, 0u, 0u, 0u);
      if (i0 < n && i0 + 3 >= n) {
        kr[it].x = kq[i0];
        if (i0 + 1 < n) kr[it].y = kq[i0 + 1];
        if (i0 + 2 < n) kr[it].z = kq[i0 + 2];
      }
    }
  }
  const int64_t nsub = (n + A.region - 1) / A.region;
  const uint32_t *cq = A.cnt + (int64_t)q * A.nsub;
  const uint32_t first_count = A.direct ? 0u : first_region_count(cq, nsub);
  const SplitSlots slots{A.cand_key + (int64_t)q * A.cand_stride,
                         A.cand_id + (int64_t)q * A.cand_stride};
  const EarlySlots<kEarlySlots> early =
      early_slots<kEarlySlots, kSelectThreads>(!A.direct, slots, nsub, A.region);
  const uint32_t *hs = A.hist + (int64_t)q * A.hstride;
  Threshold th;
  Pass19 p19{false, 0u, 0u};
  if (A.direct) {
    // the 12-bit histogram of the short key array, built here in LDS (the
    // keys past n are not counted)
    for (int i = tid; i < kHistBins; i += kSelectThreads) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kDirectIters; ++it) {
      const int64_t i0 = (int64_t)it * 4 * kSelectThreads + 4 * tid;
      if ((int64_t)it * 4 * kSelectThreads >= n) break;   // uniform
      const uint32_t k4[4] = {kr[it].x, kr[it].y, kr[it].z, kr[it].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i0 + e < n) atomicAdd(&hist[k4[e] >> 20], 1u);
    }
    __syncthreads();
    th = lds_threshold(n, A.kk, hist, scratch, res);
  } else {
    // the filter's threshold, and its second histogram (read before knowing
    // whether it is valid, in the same round of loads)
    const uint4 st = *reinterpret_cast<const uint4 *>(hs + state_off(A.hcopies));
    for (int i = tid; i < kHistBins / 4; i += kSelectThreads)
      reinterpret_cast<uint4 *>(hist)[i] = reinterpret_cast<const uint4 *>(hs + h2_off(A.hcopies))[i];
    th.keff = st.x;
    th.b1 = st.y;
    th.above = st.z;
    __syncthreads();
    if (st.w != 0u) {
      select_bin(hist, kHistBins, th.keff - th.above, scratch, res);
      p19 = Pass19{true, (th.b1 << 12) | res[0], th.above + res[1]};
      __syncthreads();   // res and hist free again
    }
  }
  const EmitAny emit{A.mode, A.out + (int64_t)q * A.out_stride,
                     pool_in ? pool_in + (int64_t)q * pool_len : nullptr, qp, (uint32_t)A.kk};

  // the candidates (keys whose top 12 bits reach b1), in index order, into LDS:
  // straight from a short key array, or from the filter's slot regions
  uint32_t carry = 0;
  if (A.direct) {
    // ordered compaction with two barriers: per iteration a wave-local scan,
    // then one wave scans the (iteration, wave) totals in key order
    const uint32_t thr = th.b1 << 20;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    constexpr int kWaves = kSelectThreads / kWave;
    constexpr int kEnt = kDirectIters * kWaves;
    constexpr int kPerLane = (kEnt + kWave - 1) / kWave;   // totals per lane in the one-wave scan
    static_assert(kEnt + 1 <= kSelectThreads, "totals and the sum fit goff");
    // only the iterations that hold keys (uniform); the totals of the others count as 0
    const int nd = (int)n;   // <= kDirectMax
    const int nit = (nd + 4 * kSelectThreads - 1) / (4 * kSelectThreads);
    uint32_t wexcl[kDirectIters];
#pragma unroll
    for (int it = 0; it < kDirectIters; ++it) {
      if (it >= nit) break;
      const int i0 = it * 4 * kSelectThreads + 4 * tid;
      const uint32_t k4[4] = {kr[it].x, kr[it].y, kr[it].z, kr[it].w};
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) c += (th.keff > 0 && i0 + e < nd && k4[e] >= thr) ? 1u : 0u;
      const uint32_t inc = wave_inclusive_scan(c);
      wexcl[it] = inc - c;
      if (lane == kWave - 1) goff[it * kWaves + wave] = inc;
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t v[kPerLane], sum = 0u;
#pragma unroll
      for (int u = 0; u < kPerLane; ++u) {
        const int e = kPerLane * lane + u;
        v[u] = (e < kEnt && e / kWaves < nit) ? goff[e] : 0u;
        sum += v[u];
      }
      uint32_t ex = wave_inclusive_scan(sum) - sum;
#pragma unroll
      for (int u = 0; u < kPerLane; ++u) {
        const int e = kPerLane * lane + u;
        if (e < kEnt) goff[e] = ex;
        ex += v[u];
      }
      if (lane == kWave - 1) goff[kEnt] = ex;
    }
    __syncthreads();
    carry = goff[kEnt];
#pragma unroll
    for (int it = 0; it < kDirectIters; ++it) {
      if (it >= nit) break;
      const int i0 = it * 4 * kSelectThreads + 4 * tid;
      const uint32_t k4[4] = {kr[it].x, kr[it].y, kr[it].z, kr[it].w};
      uint32_t o = goff[it * kWaves + wave] + wexcl[it];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (th.keff > 0 && i0 + e < nd && k4[e] >= thr) {
          if (o < kResolveCap) {
            lkey[o] = k4[e];
            lid[o] = (int32_t)(i0 + e);
          }
          ++o;
        }
      }
    }
    __syncthreads();
  } else if (early.on) {
    carry = gather_regions_early<kResolveCap, kSelectThreads>(nsub, A.region, slots, early, lkey,
                                                              lid, goff, scratch, first_count);
  } else {
    carry = gather_regions(cq, nsub, A.region, slots, lkey, lid, goff, scratch, first_count);
  }
  if (carry <= kResolveCap) {
    select_core(LdsCands{lkey, lid}, (int64_t)carry, th.keff, th.b1, th.above, hist, scratch,
                res, emit, p19);
  } else {
    select_core(GlobalKeys{A.keys + (int64_t)q * A.n_stride}, n, th.keff, th.b1, th.above, hist,
                scratch, res, emit, p19);
  }
  // padding
  const bool blocks = A.mode == kOutPoolBlocks;
  const int64_t pad_from = blocks ? (int64_t)th.keff * kPoolBlock : th.keff;
  const int64_t pad_to = blocks ? (int64_t)A.kk * kPoolBlock : A.kk;
  int32_t *oq = A.out + (int64_t)q * A.out_stride;
  for (int64_t i = pad_from + tid; i < pad_to; i += kSelectThreads) oq[i] = -1;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int H, bool kFp8, bool kPool, int kThreads, int kChunk>
void launch_score_shape(const IndexArgs &a, int64_t n_cand_max, hipStream_t s) {
  const csa2_cache &c = *a.cache;
  const TopkWorkspace &L = a.layout;
  dim3 grid((unsigned)((n_cand_max + kChunk - 1) / kChunk), (unsigned)a.nq);
  hipLaunchKernelGGL((score_kernel<H, kFp8, kPool, kThreads, kChunk>), grid, dim3(kThreads), 0, s,
                     static_cast<const uint8_t *>(c.idx_k), (int64_t)c.capacity, a.q_idx, a.q_fp8,
                     a.q_seq, a.q_pos, reinterpret_cast<uint32_t *>(a.ws + L.tok.keys), L.tok.n,
                     reinterpret_cast<uint32_t *>(a.ws + L.tok.hist),
                     kPool ? reinterpret_cast<uint32_t *>(a.ws + L.blk.keys) : nullptr, L.blk.n,
                     kPool ? reinterpret_cast<uint32_t *>(a.ws + L.blk.hist) : nullptr,
                     L.tok.hstride, L.tok.hcopies);
}

// Workgroup shape from the amount of work: long streams when there are enough
// groups, one-wave groups for small searches so that they spread over the chip.
template <int H, bool kFp8, bool kPool>
void launch_score(const IndexArgs &a, int64_t n_cand_max, hipStream_t s) {
  const int64_t big = (int64_t)a.nq * ((n_cand_max + 4095) / 4096);
  const int64_t mid = (int64_t)a.nq * ((n_cand_max + 2047) / 2048);
  if (big >= kBigChunkMinGroups)
    launch_score_shape<H, kFp8, kPool, 256, 4096>(a, n_cand_max, s);
  else if (mid >= kSmallGridGroups || kPool)
    launch_score_shape<H, kFp8, kPool, 256, 2048>(a, n_cand_max, s);
  else
    launch_score_shape<H, kFp8, false, 64, 64>(a, n_cand_max, s);
}

template <int H, bool kFp8>
void launch_score_mode(const IndexArgs &a, int64_t n, bool pool, bool reindex_pool, hipStream_t s) {
  if (reindex_pool) {
    const TopkWorkspace &L = a.layout;
    constexpr int kEntries = kGatherThreads / H;
    hipLaunchKernelGGL((gather_score_kernel<H, kFp8>),
                       dim3((unsigned)((a.pool_len + kEntries - 1) / kEntries), (unsigned)a.nq),
                       dim3(kGatherThreads), 0, s, static_cast<const uint8_t *>(a.cache->idx_k),
                       (int64_t)a.cache->capacity, a.q_idx, a.q_fp8, a.q_seq, a.q_pos, a.pool_in,
                       a.pool_len, reinterpret_cast<uint32_t *>(a.ws + L.tok.keys), L.tok.n,
                       a.pool_len <= kDirectMax ? nullptr
                                                : reinterpret_cast<uint32_t *>(a.ws + L.tok.hist),
                       L.tok.hstride, L.tok.hcopies);
  } else if (pool) {
    launch_score<H, kFp8, true>(a, n, s);
  } else {
    launch_score<H, kFp8, false>(a, n, s);
  }
}

SelProblem sel_problem(const IndexArgs &a, const SelectArrays &A, int32_t kk, int mode,
                       int32_t *out, int64_t out_stride) {
  uint8_t *w = a.ws;
  SelProblem p;
  p.keys = reinterpret_cast<const uint32_t *>(w + A.keys);
  p.n_stride = A.n;
  p.hist = reinterpret_cast<uint32_t *>(w + A.hist);
  p.hstride = A.hstride;
  p.hcopies = A.hcopies;
  p.cand_key = reinterpret_cast<uint32_t *>(w + A.cand_key);
  p.cand_id = reinterpret_cast<int32_t *>(w + A.cand_id);
  p.cand_stride = A.cand_stride;
  p.cnt = reinterpret_cast<uint32_t *>(w + A.cnt);
  p.nsub = A.nsub;
  p.out = out;
  p.out_stride = out_stride;
  p.kk = kk;
  p.mode = mode;
  p.direct = A.n <= kDirectMax;
  p.region = A.region;
  return p;
}

// Filter + resolve of one or two selection problems (tokens, pool blocks),
// both problems in the same two launches.
void launch_select(const IndexArgs &a, const SelProblems &P, int nprob, int64_t max_nsub,
                   hipStream_t s) {
  const int64_t waves = kFilterThreads / kWave;
  bool all_direct = true;
  for (int i = 0; i < nprob; ++i) all_direct = all_direct && P.p[i].direct;
  int32_t region = 0;
  for (int i = 0; i < nprob; ++i) region = std::max(region, P.p[i].direct ? 0 : P.p[i].region);
  const dim3 grid((unsigned)((max_nsub + waves - 1) / waves), (unsigned)a.nq, (unsigned)nprob);
  if (region > kFilterSubMin)
    hipLaunchKernelGGL(filter_kernel<kFilterSubMax / 256>, grid, dim3(kFilterThreads), 0, s, P,
                       a.q_pos, a.pool_len);
  else if (!all_direct)
    hipLaunchKernelGGL(filter_kernel<kFilterSubMin / 256>, grid, dim3(kFilterThreads), 0, s, P,
                       a.q_pos, a.pool_len);
  hipLaunchKernelGGL(resolve_kernel, dim3((unsigned)a.nq, (unsigned)nprob), dim3(kSelectThreads),
                     0, s, P, a.q_pos, a.pool_in, a.pool_len);
}

thread_local hipEvent_t g_scan_before = nullptr;
thread_local hipEvent_t g_scan_after = nullptr;

// Histogram copies for a key array of n_slots: one per 128K keys, at most 4
// (a single query's hundreds of scorer workgroups would otherwise queue their
// atomics on the same few hot bins; readers add the copies up).
int32_t hist_copies(int64_t n_slots) {
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>(4, n_slots / 131072));
}

size_t carve(SelectArrays &A, int64_t n_slots, int32_t nq, size_t off, int32_t hcopies) {
  A.n = (n_slots + 63) / 64 * 64;
  A.hcopies = hcopies;
  A.hstride = hist_stride(hcopies);
  A.region = A.n > kFilterSmallMax ? kFilterSubMax : kFilterSubMin;
  A.nsub = (A.n + A.region - 1) / A.region;
  A.cand_stride = A.nsub * A.region;
  A.keys = off;
  off = align256(off + (size_t)nq * A.n * 4);
  A.hist = off;
  off = align256(off + (size_t)nq * A.hstride * 4);
  A.cand_key = off;
  off = align256(off + (size_t)nq * A.cand_stride * 4);
  A.cand_id = off;
  off = align256(off + (size_t)nq * A.cand_stride * 4);
  A.cnt = off;
  off = align256(off + (size_t)nq * A.nsub * 4);
  return off;
}

}  // namespace

void set_index_scan_events(hipEvent_t before, hipEvent_t after) {
  g_scan_before = before;
  g_scan_after = after;
}

TopkWorkspace topk_workspace_layout(const csa2_cache &c, csa2_mode mode, int32_t nq,
                                    int32_t pool_len, int32_t pool_blocks) {
  TopkWorkspace w;
  if (mode == CSA2_REUSE) return w;
  const bool reindex_pool = mode == CSA2_REINDEX && pool_len > 0;
  const bool pool = mode == CSA2_FULL && pool_blocks > 0;
  // the token and block histograms are filled by the same scorer launch and
  // cleared by one launch: the same number of copies
  const int64_t n_tok = reindex_pool ? (int64_t)pool_len : (int64_t)c.capacity;
  const int32_t hc = hist_copies(n_tok);
  size_t off = carve(w.tok, n_tok, nq, 0, hc);
  if (pool) off = carve(w.blk, ((int64_t)c.capacity + kPoolBlock - 1) / kPoolBlock, nq, off, hc);
  w.total = off;
  if (gemm_eligible(c, mode, pool_len, pool_blocks)) {
    w.gemm = gemm_workspace_layout(c, nq);
    w.total = std::max(w.total, w.gemm.total);
  }
  return w;
}

hipError_t launch_index_topk(const IndexArgs &a, hipStream_t s) {
  const csa2_cache &c = *a.cache;
  if (a.mode == CSA2_REUSE) {
    const int64_t n = (int64_t)a.nq * a.top_k;
    const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(copy_i32_kernel, dim3(blocks), dim3(256), 0, s, a.topk_out, a.reuse_src, n);
    return hipGetLastError();
  }
  if (a.q_fp8 && gemm_eligible(c, a.mode, a.pool_len, a.pool_blocks))
    return launch_index_topk_gemm(a, g_scan_before, g_scan_after, s);
  const TopkWorkspace &L = a.layout;
  const bool pool = a.mode == CSA2_FULL && a.pool_blocks > 0;
  const bool reindex_pool = a.mode == CSA2_REINDEX && a.pool_in != nullptr;
  // 1. clear the histograms (the token and block histograms are cleared by one
  //    launch when both exist: the block one follows the token arrays).  A
  //    pool short enough for the resolve to read whole needs none.
  if (!(reindex_pool && a.pool_len <= kDirectMax)) {
    const int64_t n_tok = (int64_t)a.nq * L.tok.hstride;
    const unsigned blocks = (unsigned)std::min<int64_t>((n_tok + 255) / 256, 2048);
    hipLaunchKernelGGL(zero2_u32_kernel, dim3(blocks), dim3(256), 0, s,
                       reinterpret_cast<uint32_t *>(a.ws + L.tok.hist),
                       pool ? reinterpret_cast<uint32_t *>(a.ws + L.blk.hist) : nullptr, n_tok);
  }
  // 2. scores, first-pass histograms and bins
  if (g_scan_before != nullptr) (void)hipEventRecord(g_scan_before, s);
  const int64_t n_cand = reindex_pool ? (int64_t)a.pool_len : (int64_t)c.capacity;
  const bool fp8 = c.idx_k_dtype == CSA2_FP8_E4M3;
  if (c.idx_heads == 8) {
    if (fp8) launch_score_mode<8, true>(a, n_cand, pool, reindex_pool, s);
    else launch_score_mode<8, false>(a, n_cand, pool, reindex_pool, s);
  } else {
    if (fp8) launch_score_mode<4, true>(a, n_cand, pool, reindex_pool, s);
    else launch_score_mode<4, false>(a, n_cand, pool, reindex_pool, s);
  }
  if (g_scan_after != nullptr) (void)hipEventRecord(g_scan_after, s);
  // 3. selection: the Top-K, and the pool blocks in the same launches
  SelProblems P;
  P.p[0] = sel_problem(a, L.tok, a.top_k, reindex_pool ? kOutPoolIds : kOutPositions, a.topk_out,
                       a.top_k);
  int64_t max_nsub = L.tok.nsub;
  if (pool) {
    P.p[1] = sel_problem(a, L.blk, a.pool_blocks, kOutPoolBlocks, a.pool_out,
                         (int64_t)a.pool_blocks * kPoolBlock);
    max_nsub = std::max(max_nsub, L.blk.nsub);
  }
  launch_select(a, P, pool ? 2 : 1, max_nsub, s);
  return hipGetLastError();
}

}  // namespace csa2
