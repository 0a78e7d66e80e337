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
//   score_kernel     stream the (tiled) index keys, compute the canonical fp32
//                    score of each candidate, keep its order-preserving key
//                    (written out per workgroup in one burst), histogram the
//                    top 12 key bits, and for a pool-building Full layer the
//                    8-position block maxima and their histogram.
//   bins_kernel      per query: the bin b1 of the 12-bit histogram holding the
//                    K-th largest key.
//   filter_kernel    per wave and 1024 keys: keep every key whose top 12 bits
//                    reach b1, with its index, in index order (ballot compaction)
//   resolve_kernel   per query: the candidates (typically K plus one bin) in
//                    LDS; radix passes on bits 19..8 and 7..0 within bin b1 give
//                    the K-th largest key tau; an ordered compaction emits every
//                    key > tau and the first ties == tau, ascending, -1 padded.
//                    With more candidates than LDS holds (heavy ties) it
//                    streams the full key array with the same logic.
//   copy_i32_kernel  Reuse mode: topk_out = reuse_src.
// The selection helpers (select_bin, select_core, gather_regions) live in
// csa2_select.h; E4M3 index queries against E4M3 keys over every visible
// position go to the matrix-core scorer in csa2_index_gemm.hip instead.
#include <algorithm>

#include "csa2_select.h"

namespace csa2 {
namespace {

constexpr int kFilterThreads = 256;
constexpr int kFilterSub = 1024;           // keys per filter wave (one candidate slot region)

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
template <int H, bool kFp8Keys, bool kPool, bool kReindexPool, int kThreads, int kChunk>
struct ScoreCtx {
  static constexpr int kEsz = kFp8Keys ? 1 : 2;
  static constexpr int TPI = kWave / H;
  static constexpr int kLoads = 4 * kEsz;
  static constexpr int kNumWaves = kThreads / kWave;
  const uint8_t *seq_base;
  const int32_t *spool;    // this chunk's pool entries, staged in LDS (Reindex)
  int32_t qp;
  int64_t t_begin, t_end;
  int wave, h, tl, lane;

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
      bool valid = t < t_end;
      int64_t row = valid ? t : t_begin;
      if (kReindexPool) {
        const int32_t p = valid ? spool[t - t_begin] : -1;
        valid = valid && p >= 0 && p <= qp;
        row = valid ? (int64_t)p : 0;
      }
      val[u] = valid;
      // Full mode: row % TPI == tl, so a wave's loads cover one tile contiguously
      const uint8_t *src = seq_base + idx_chunk_offset<H, kEsz>(row, h, 0);
#pragma unroll
      for (int v = 0; v < kLoads; ++v) buf[u][v] = *reinterpret_cast<const uint4 *>(src + v * 1024);
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

template <int H, bool kFp8Keys, bool kPool, bool kReindexPool, int kThreads, int kChunk>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kThreads == 64 ? 2 : (kFp8Keys ? CSA2_SCORE_WAVES : CSA2_SCORE_WAVES - 1))))
score_kernel(
    const uint8_t *__restrict__ idx_k, int64_t capacity, const uint16_t *__restrict__ q_idx,
    int32_t q_fp8, const int32_t *__restrict__ q_seq, const int32_t *__restrict__ q_pos,
    const int32_t *__restrict__ pool_in, int32_t pool_len,
    uint32_t *__restrict__ keys_tok, int64_t tok_stride, uint32_t *__restrict__ hist_tok,
    uint32_t *__restrict__ keys_blk, int64_t blk_stride, uint32_t *__restrict__ hist_blk) {
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
  __shared__ int32_t spool[kReindexPool ? kChunk : 1];
  uint32_t *hist = lds_main;
  uint32_t *skeys = lds_main + kHistBins / 2;

  const int q = blockIdx.y;
  const int32_t qp = q_pos[q];
  const int64_t n = kReindexPool ? (int64_t)pool_len : (int64_t)qp + 1;
  const int64_t t_begin = (int64_t)blockIdx.x * kChunk;
  if (t_begin >= n) return;
  const int64_t t_end = min(n, t_begin + kChunk);

  for (int i = threadIdx.x; i < kHistBins / 2; i += kThreads) {
    hist[i] = 0u;
    if (kPool) histb[i] = 0u;
  }
  // Reindex: the chunk's pool entries, staged once (no dependent load per gather)
  if (kReindexPool)
    for (int64_t i = threadIdx.x; i < t_end - t_begin; i += kThreads)
      spool[i] = pool_in[(int64_t)q * pool_len + t_begin + i];
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
  ScoreCtx<H, kFp8Keys, kPool, kReindexPool, kThreads, kChunk> cx{
      seq_base, spool, qp, t_begin, t_end, wave, h, tl, lane};
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
  uint32_t *hq = hist_tok + (int64_t)q * (kHistBins + kStateWords);
  uint32_t *hbq = kPool ? hist_blk + (int64_t)q * (kHistBins + kStateWords) : nullptr;
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

// One workgroup per (query, key array): bin b1 of the K-th largest key from the
// query's 12-bit histogram, written to the state words after the histogram.
__global__ void __launch_bounds__(kSelectThreads) bins_kernel(
    uint32_t *__restrict__ hist_tok, uint32_t *__restrict__ hist_blk, const int32_t *__restrict__ q_pos,
    int32_t pool_len, int32_t reindex_pool, int32_t top_k, int32_t pool_blocks) {
  __shared__ uint32_t lds[kHistBins];
  __shared__ uint32_t scratch[kSelectThreads / kWave + 1];
  __shared__ uint32_t res[2];
  const int q = blockIdx.x;
  const bool blocks = blockIdx.y == 1;
  const int32_t qp = q_pos[q];
  int64_t n = reindex_pool ? (int64_t)pool_len : (int64_t)qp + 1;
  if (blocks) n = (n + kPoolBlock - 1) / kPoolBlock;
  uint32_t *hq = (blocks ? hist_blk : hist_tok) + (int64_t)q * (kHistBins + kStateWords);
  for (int i = threadIdx.x; i < kHistBins; i += kSelectThreads) lds[i] = hq[i];
  __syncthreads();
  const int64_t n_valid = n - (int64_t)lds[0];   // key 0 marks an empty pool slot
  const uint32_t keff = (uint32_t)min((int64_t)(blocks ? pool_blocks : top_k), n_valid);
  if (keff > 0) {
    select_bin(lds, kHistBins, keff, scratch, res);
  } else if (threadIdx.x == 0) {
    res[0] = 0u;
    res[1] = 0u;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    hq[kHistBins + kBin] = res[0];
    hq[kHistBins + kAbove] = res[1];
    hq[kHistBins + kKeff] = keff;
  }
}

// One wave per kFilterSub keys: keep every key whose top 12 bits reach bin b1,
// with its index, in index order, into the wave's own slot region.
template <int kMode>
__global__ void __launch_bounds__(kFilterThreads) filter_kernel(
    const uint32_t *__restrict__ keys, int64_t stride, const uint32_t *__restrict__ hist_g,
    const int32_t *__restrict__ q_pos, int32_t pool_len, uint32_t *__restrict__ cand_key,
    int32_t *__restrict__ cand_id, int64_t cand_stride, uint32_t *__restrict__ cnt,
    int64_t cnt_stride) {
  const int q = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t sub = (int64_t)blockIdx.x * (kFilterThreads / kWave) + threadIdx.x / kWave;
  const int64_t n = array_len<kMode>(q_pos[q], pool_len);
  const int64_t start = sub * kFilterSub;
  if (start >= n) return;
  const uint32_t *st = hist_g + (int64_t)q * (kHistBins + kStateWords) + kHistBins;
  const bool none = st[kKeff] == 0u;
  const uint32_t thr = st[kBin] << 20;
  const uint32_t *kq = keys + (int64_t)q * stride;
  uint32_t *ck = cand_key + (int64_t)q * cand_stride + start;
  int32_t *ci = cand_id + (int64_t)q * cand_stride + start;
  // 4 x 4 keys per lane; key (k, lane, e) sits at start + k*256 + lane*4 + e
  uint32_t kv[4][4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t i0 = start + k * 256 + lane * 4;
    if (i0 + 3 < n) {
      const uint4 v = *reinterpret_cast<const uint4 *>(kq + i0);
      kv[k][0] = v.x;
      kv[k][1] = v.y;
      kv[k][2] = v.z;
      kv[k][3] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) kv[k][e] = i0 + e < n ? kq[i0 + e] : 0u;
    }
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t written = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    bool f[4];
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = start + k * 256 + lane * 4 + e;
      f[e] = !none && i < n && kv[k][e] >= thr;
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
      }
    }
    written += total;
  }
  if (lane == 0) cnt[(int64_t)q * cnt_stride + sub] = written;
}

template <int kMode>
__global__ void __launch_bounds__(kSelectThreads) resolve_kernel(
    const uint32_t *__restrict__ keys, int64_t stride, const uint32_t *__restrict__ hist_g,
    const int32_t *__restrict__ q_pos, const int32_t *__restrict__ pool_in, int32_t pool_len,
    int32_t kk, const uint32_t *__restrict__ cand_key, const int32_t *__restrict__ cand_id,
    int64_t cand_stride, const uint32_t *__restrict__ cnt, int64_t cnt_stride,
    int32_t *__restrict__ out, int64_t out_stride) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t scratch[kSelectThreads / kWave + 1];
  __shared__ uint32_t res[2];
  __shared__ uint32_t lkey[kResolveCap];
  __shared__ int32_t lid[kResolveCap];
  __shared__ uint32_t goff[kSelectThreads];

  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t qp = q_pos[q];
  const int64_t n = array_len<kMode>(qp, pool_len);
  const uint32_t *st = hist_g + (int64_t)q * (kHistBins + kStateWords) + kHistBins;
  const uint32_t keff = st[kKeff];
  const uint32_t b1 = st[kBin];
  const uint32_t above1 = st[kAbove];
  Emit<kMode> emit{out + (int64_t)q * out_stride,
                   pool_in ? pool_in + (int64_t)q * pool_len : nullptr, qp};

  // candidates of the filter's slot regions, in index order, into LDS
  const int64_t nsub = (n + kFilterSub - 1) / kFilterSub;
  const uint32_t carry =
      gather_regions(cnt + (int64_t)q * cnt_stride, nsub, kFilterSub,
                     SplitSlots{cand_key + (int64_t)q * cand_stride,
                                cand_id + (int64_t)q * cand_stride},
                     lkey, lid, goff, scratch);
  if (carry <= kResolveCap) {
    select_core(LdsCands{lkey, lid}, (int64_t)carry, keff, b1, above1, hist, scratch, res, emit);
  } else {
    select_core(GlobalKeys{keys + (int64_t)q * stride}, n, keff, b1, above1, hist, scratch, res,
                emit);
  }
  // padding
  const int64_t pad_from = (kMode == kOutPoolBlocks) ? (int64_t)keff * kPoolBlock : keff;
  const int64_t pad_to = (kMode == kOutPoolBlocks) ? (int64_t)kk * kPoolBlock : kk;
  int32_t *oq = out + (int64_t)q * out_stride;
  for (int64_t i = pad_from + tid; i < pad_to; i += kSelectThreads) oq[i] = -1;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int H, bool kFp8, bool kPool, bool kReindexPool, int kThreads, int kChunk>
void launch_score_shape(const IndexArgs &a, int64_t n_cand_max, hipStream_t s) {
  const csa2_cache &c = *a.cache;
  const TopkWorkspace &L = a.layout;
  dim3 grid((unsigned)((n_cand_max + kChunk - 1) / kChunk), (unsigned)a.nq);
  const int32_t *pool = kReindexPool ? a.pool_in : nullptr;
  hipLaunchKernelGGL((score_kernel<H, kFp8, kPool, kReindexPool, kThreads, kChunk>), grid,
                     dim3(kThreads), 0, s, static_cast<const uint8_t *>(c.idx_k),
                     (int64_t)c.capacity, a.q_idx, a.q_fp8, a.q_seq, a.q_pos, pool, a.pool_len,
                     reinterpret_cast<uint32_t *>(a.ws + L.tok.keys),
                     L.tok.n, reinterpret_cast<uint32_t *>(a.ws + L.tok.hist),
                     kPool ? reinterpret_cast<uint32_t *>(a.ws + L.blk.keys) : nullptr, L.blk.n,
                     kPool ? reinterpret_cast<uint32_t *>(a.ws + L.blk.hist) : nullptr);
}

// Workgroup shape from the amount of work: long streams when there are enough
// groups, one-wave groups for small searches (a Reindex pool) so that the
// gathers spread over the chip.
template <int H, bool kFp8, bool kPool, bool kReindexPool>
void launch_score(const IndexArgs &a, int64_t n_cand_max, hipStream_t s) {
  const int64_t big = (int64_t)a.nq * ((n_cand_max + 4095) / 4096);
  const int64_t mid = (int64_t)a.nq * ((n_cand_max + 2047) / 2048);
  if (big >= kBigChunkMinGroups)
    launch_score_shape<H, kFp8, kPool, kReindexPool, 256, 4096>(a, n_cand_max, s);
  else if (mid >= kSmallGridGroups || kPool)
    launch_score_shape<H, kFp8, kPool, kReindexPool, 256, 2048>(a, n_cand_max, s);
  else
    launch_score_shape<H, kFp8, false, kReindexPool, 64, 64>(a, n_cand_max, s);
}

template <int H, bool kFp8>
void launch_score_mode(const IndexArgs &a, int64_t n, bool pool, bool reindex_pool, hipStream_t s) {
  if (pool) launch_score<H, kFp8, true, false>(a, n, s);
  else if (reindex_pool) launch_score<H, kFp8, false, true>(a, n, s);
  else launch_score<H, kFp8, false, false>(a, n, s);
}

template <int kMode>
void launch_select(const IndexArgs &a, const SelectArrays &A, int32_t kk, int32_t *out,
                   int64_t out_stride, hipStream_t s) {
  uint8_t *w = a.ws;
  const int32_t pool_len = kMode == kOutPoolIds ? a.pool_len : 0;
  const int64_t waves = kFilterThreads / kWave;
  hipLaunchKernelGGL((filter_kernel<kMode>),
                     dim3((unsigned)((A.nsub + waves - 1) / waves), (unsigned)a.nq),
                     dim3(kFilterThreads), 0, s, reinterpret_cast<const uint32_t *>(w + A.keys), A.n,
                     reinterpret_cast<const uint32_t *>(w + A.hist), a.q_pos, pool_len,
                     reinterpret_cast<uint32_t *>(w + A.cand_key),
                     reinterpret_cast<int32_t *>(w + A.cand_id), A.cand_stride,
                     reinterpret_cast<uint32_t *>(w + A.cnt), A.nsub);
  hipLaunchKernelGGL((resolve_kernel<kMode>), dim3((unsigned)a.nq), dim3(kSelectThreads), 0, s,
                     reinterpret_cast<const uint32_t *>(w + A.keys), A.n,
                     reinterpret_cast<const uint32_t *>(w + A.hist), a.q_pos,
                     kMode == kOutPoolIds ? a.pool_in : nullptr, pool_len, kk,
                     reinterpret_cast<const uint32_t *>(w + A.cand_key),
                     reinterpret_cast<const int32_t *>(w + A.cand_id), A.cand_stride,
                     reinterpret_cast<const uint32_t *>(w + A.cnt), A.nsub, out, out_stride);
}

thread_local hipEvent_t g_scan_before = nullptr;
thread_local hipEvent_t g_scan_after = nullptr;

size_t carve(SelectArrays &A, int64_t n_slots, int32_t nq, size_t off) {
  A.n = (n_slots + 63) / 64 * 64;
  A.nsub = (A.n + kFilterSub - 1) / kFilterSub;
  A.cand_stride = A.nsub * kFilterSub;
  A.keys = off;
  off = align256(off + (size_t)nq * A.n * 4);
  A.hist = off;
  off = align256(off + (size_t)nq * (kHistBins + kStateWords) * 4);
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
  size_t off = carve(w.tok, reindex_pool ? (int64_t)pool_len : (int64_t)c.capacity, nq, 0);
  if (pool) off = carve(w.blk, ((int64_t)c.capacity + kPoolBlock - 1) / kPoolBlock, nq, off);
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
  //    launch when both exist: the block one follows the token arrays)
  {
    const int64_t n_tok = (int64_t)a.nq * (kHistBins + kStateWords);
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
  // 3. first-pass bins, then selection
  hipLaunchKernelGGL(bins_kernel, dim3((unsigned)a.nq, pool ? 2u : 1u), dim3(kSelectThreads), 0, s,
                     reinterpret_cast<uint32_t *>(a.ws + L.tok.hist),
                     pool ? reinterpret_cast<uint32_t *>(a.ws + L.blk.hist) : nullptr, a.q_pos,
                     a.pool_len, (int32_t)reindex_pool, a.top_k, a.pool_blocks);
  if (reindex_pool)
    launch_select<kOutPoolIds>(a, L.tok, a.top_k, a.topk_out, a.top_k, s);
  else
    launch_select<kOutPositions>(a, L.tok, a.top_k, a.topk_out, a.top_k, s);
  if (pool)
    launch_select<kOutPoolBlocks>(a, L.blk, a.pool_blocks, a.pool_out,
                                  (int64_t)a.pool_blocks * kPoolBlock, s);
  return hipGetLastError();
}

}  // namespace csa2
