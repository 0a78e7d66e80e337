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
//   zero2_u32_kernel clear the per-query histograms (only where the scorer
//                    adds into a global histogram)
//   score_kernel     (Full, or Reindex without a pool; gather_score_kernel for
//                    a Reindex pool) stream the (tiled) index keys, compute the canonical fp32
//                    score of each candidate, keep its order-preserving key
//                    (written out per workgroup in one burst), histogram the
//                    top 12 key bits, and for a pool-building Full layer the
//                    8-position block maxima and their histogram.
// Then the selection, in one of two forms:
//   Ranked records (a Full layer without a pool, or a Reindex layer without
//   one, over at most 65536 positions in at most kMaxRankedChunks scorer
//   chunks -- decode batches up to 64K context -- and a Reindex pool of at
//   most 64 x kGatherRec entries, scored by gather_rank_kernel): each scorer
//   workgroup sorts its keys by 12-bit bin in LDS and stores them with their
//   indices and the count of keys at or above every bin, so that
//   ranked_select_kernel  one workgroup per query reads the threshold bin b1
//                    off the counts (a 64-entry coarse table, then one
//                    64-bin window), then only the keys at or above b1 (the
//                    first entries of each record), and selects in LDS:
//                    one launch instead of two, and no histogram to clear.
//   Otherwise:
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
//                    Key arrays of at most kDirectMax entries skip the
//                    filter: the resolve reads them and compacts them itself.
//                    The 12-bit histogram comes from the global histogram (a
//                    pool-building Full layer, long contexts), or is counted
//                    by the resolve (a Reindex pool).
// Small score chunks (one wave) count keys straight into the global histogram.
//   copy_i32_kernel  Reuse mode: topk_out = reuse_src.
// The selection helpers (select_bin, select_core, gather_regions) live in
// csa2_select.h; E4M3 index queries against E4M3 keys over every visible
// position go to the matrix-core scorer in csa2_index_gemm.hip instead.
#include <algorithm>

#include "csa2_kv_row.h"
#include "csa2_select.h"

namespace csa2 {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFilterThreads = 1024;      // few, wide workgroups: each derives the threshold bin
// Keys per filter wave (one candidate slot region): 512 for key arrays up to
// kFilterSmallMax keys, else 1024 -- half the filter workgroups, each of
// which reads the query's histogram copies, and at most 1024 regions for
// arrays up to 1M keys, so that the resolve's one round of early slot reads
// covers every region (one region per resolve thread).
constexpr int kFilterSubMin = 512;
constexpr int kFilterSubMax = 1024;
constexpr int64_t kFilterSmallMax = 32768;
constexpr int64_t kDirectMax = 32768;      // up to this many keys the resolve filters them itself
// Ranked records (kRanked): at most this many records per query (a
// selection wave reads four) and 65536 candidates; a Full scan's records
// are its chunks of 2048 or 4096 positions, a Reindex pool's are runs of
// kGatherRec entries.
constexpr int64_t kMaxRankedChunks = 64;
constexpr int64_t kMaxRankedKeys = 65536;
constexpr int kGatherRec = 256;
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
// The sum over the index heads, left to right.  The H lanes of a candidate
// (lanes H*t .. H*t+H-1, head h in lane H*t+h) each hold one head's dot
// product; every lane of the group ends with ((a_0 + a_1) + a_2) + ... + a_{H-1}
// in fp32, the same bits in each lane: each lane fetches the group's values
// in head order with DPP moves and adds them up itself.
// ---------------------------------------------------------------------------
template <int kLane>   // quad_perm [kLane, kLane, kLane, kLane]: lane kLane of each quad
__device__ __forceinline__ float dpp_quad_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kLane * 0x55, 0xF, 0xF, true));
}
// The value of the lane at the same position in the other quad of an 8-lane
// half row: quad_perm [3, 2, 1, 0] then row_half_mirror (lane i <- 7 - i).
// Both are uniform patterns run by every lane: a DPP move reads its source
// lane only while that lane is active, so no DPP move may sit under a
// lane-dependent branch.
__device__ __forceinline__ float dpp_other_quad(float v) {
  const int r = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x1B, 0xF, 0xF, true);
  return __int_as_float(__builtin_amdgcn_mov_dpp(r, 0x141, 0xF, 0xF, true));
}

template <int H>
__device__ __forceinline__ float head_sum_ltr(float x) {
  static_assert(H == 4 || H == 8, "four or eight index heads");
  // lo: heads 0..3 of the lane's group, hi: heads 4..7, each at the lane's
  // position in its own quad (an 8-lane group is two quads of one row); the
  // choice is a bitwise select, so the compiler keeps it branch-free
  float lo = x, hi = 0.0f;
  if (H == 8) {
    const uint32_t m = 0u - ((threadIdx.x >> 2) & 1u);   // all ones in the upper quad
    const uint32_t xb = __float_as_uint(x);
    const uint32_t ob = __float_as_uint(dpp_other_quad(x));
    lo = __uint_as_float((xb & ~m) | (ob & m));
    hi = __uint_as_float((ob & ~m) | (xb & m));
  }
  float s = dpp_quad_bcast<0>(lo);
  s = s + dpp_quad_bcast<1>(lo);
  s = s + dpp_quad_bcast<2>(lo);
  s = s + dpp_quad_bcast<3>(lo);
  if (H == 8) {
    s = s + dpp_quad_bcast<0>(hi);
    s = s + dpp_quad_bcast<1>(hi);
    s = s + dpp_quad_bcast<2>(hi);
    s = s + dpp_quad_bcast<3>(hi);
  }
  return s;
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
// lane runs its head's fp32 chain of fused multiply-adds over channels 0..63
// in order; head_sum_ltr then adds the head sums from head 0 up.  Every lane
// of a token ends with the same bits.
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
      float acc = 0.0f;   // one chain over the head's 64 channels
#pragma unroll
      for (int j = 0; j < 4; ++j) {
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
      }
      acc = head_sum_ltr<H>(acc);
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

// A ranked record from a workgroup's staged keys: skeys[i] for the slots i
// with valid(i), counted in the packed 16-bit LDS histogram `hist`.  Thread
// t owns bins 16t .. 16t+15 (LDS words 8t .. 8t+7): ge of a bin = keys in
// the bins of higher threads + the thread's own bins from that one up; a
// bin's keys start at ge - count in the bin-ordered list, where LDS atomics
// on the bins' cursors place them (in no particular order inside a bin).
// Then the record (keys, slot indices), its ge table and coarse table go out
// with the global stores last (a barrier waits for a thread's stores).
// Contains barriers; uses rsk, rsp (kSlots each) and rscr.
template <int kThreads, int kSlots, class Valid>
__device__ __forceinline__ void rank_record(uint32_t *hist, const uint32_t *skeys, Valid valid,
                                            uint32_t *rsk, uint16_t *rsp, uint32_t *rscr,
                                            uint32_t *keys_out, uint16_t *pos_out,
                                            uint16_t *ge_out, uint16_t *coarse_out) {
  static_assert(kThreads * 16 == kHistBins && kSlots % kThreads == 0, "16 bins per thread");
  const int tid = threadIdx.x;
  const uint4 wa = reinterpret_cast<const uint4 *>(hist)[2 * tid];
  const uint4 wb = reinterpret_cast<const uint4 *>(hist)[2 * tid + 1];
  const uint32_t w[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
  uint32_t c[16], ge[16];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    c[2 * k] = w[k] & 0xFFFFu;
    c[2 * k + 1] = w[k] >> 16;
  }
  uint32_t s = 0;
#pragma unroll
  for (int b = 15; b >= 0; --b) {
    s += c[b];
    ge[b] = s;
  }
  uint32_t total;
  const uint32_t before = block_exclusive_scan(s, rscr, total);
  const uint32_t higher = total - before - s;   // keys in the bins of higher threads
  uint32_t g[8], cur[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t lo = ge[2 * k] + higher, hi = ge[2 * k + 1] + higher;
    g[k] = lo | (hi << 16);
    cur[k] = (lo - c[2 * k]) | ((hi - c[2 * k + 1]) << 16);
  }
  // every thread has read its words: they become the bins' insertion cursors
  reinterpret_cast<uint4 *>(hist)[2 * tid] = make_uint4(cur[0], cur[1], cur[2], cur[3]);
  reinterpret_cast<uint4 *>(hist)[2 * tid + 1] = make_uint4(cur[4], cur[5], cur[6], cur[7]);
  __syncthreads();
  // a fixed trip count with the empty slots masked (an atomic adding 0), so
  // that a thread's atomics issue back to back
#pragma unroll
  for (int u = 0; u < kSlots / kThreads; ++u) {
    const int i = tid + u * kThreads;
    const bool v = valid(i);
    const uint32_t key = skeys[i];
    const uint32_t sh = (key >> 16) & 16u;
    const uint32_t slot = (atomicAdd(&hist[key >> 21], v ? 1u << sh : 0u) >> sh) & 0xFFFFu;
    if (v) {
      rsk[slot] = key;
      rsp[slot] = (uint16_t)i;
    }
  }
  __syncthreads();
  uint4 *gq = reinterpret_cast<uint4 *>(ge_out);
  gq[2 * tid] = make_uint4(g[0], g[1], g[2], g[3]);
  gq[2 * tid + 1] = make_uint4(g[4], g[5], g[6], g[7]);
  if ((tid & 3) == 0) coarse_out[tid / 4] = (uint16_t)(g[0] & 0xFFFFu);
  const int cnt = (int)total;
  for (int i = 4 * tid; i < cnt; i += 4 * kThreads) {
    if (i + 4 <= cnt) {
      *reinterpret_cast<uint4 *>(keys_out + i) = *reinterpret_cast<const uint4 *>(rsk + i);
      *reinterpret_cast<uint2 *>(pos_out + i) = *reinterpret_cast<const uint2 *>(rsp + i);
    } else {
      for (int e = i; e < cnt; ++e) {
        keys_out[e] = rsk[e];
        pos_out[e] = rsp[e];
      }
    }
  }
}

// Ranked chunk records (kRanked), written by the scorer's workgroup of chunk
// c of query q: keys[q][c*chunk + i] (the keys array) and pos[q][c*chunk + i]
// for i < the chunk's key count, ordered by 12-bit bin from the highest (in
// no particular order inside a bin); ge[q][c][b] = the chunk's keys in bin b
// or above; coarse[q][c][j] = ge[q][c][64 j].
struct RankedOut {
  uint16_t *pos;
  uint16_t *ge;
  uint16_t *coarse;
};

template <int H, bool kFp8Keys, bool kPool, int kThreads, int kChunk, bool kRanked = false>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kThreads == 64 ? 2 : (kFp8Keys ? CSA2_SCORE_WAVES : CSA2_SCORE_WAVES - 1))))
score_kernel(
    const uint8_t *__restrict__ idx_k, int64_t capacity, const uint16_t *__restrict__ q_idx,
    int32_t q_fp8, const int32_t *__restrict__ q_seq, const int32_t *__restrict__ q_pos,
    uint32_t *__restrict__ keys_tok, int64_t tok_stride, uint32_t *__restrict__ hist_tok,
    uint32_t *__restrict__ keys_blk, int64_t blk_stride, uint32_t *__restrict__ hist_blk,
    int64_t hstride, int32_t hcopies, RankedOut rk, const AppendRows ap, int32_t nq) {
  // kRanked: the chunk's record goes to rk (and the keys array, in bin order)
  // instead of adding its histogram into the global one.
  // ap.n > 0 (a fused append, 256-thread shapes, ap.n <= kThreads): the
  // workgroups past the nq query rows store the appended rows, one wave per
  // row; a scoring workgroup whose chunk holds an appended position of its
  // query's sequence scores that position from the row's input instead of
  // the cache (which those workgroups may not have written yet).
  static_assert(!kRanked || (!kPool && kThreads * 16 == kHistBins), "ranked chunks: 16 bins per thread");
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
  __shared__ __attribute__((aligned(16))) uint32_t lds_main[kMainWords];
  __shared__ uint32_t histb[kPool ? kHistBins / 2 : 1];
  __shared__ uint32_t sblk[kPool ? kChunk / kPoolBlock : 1];
  __shared__ float qlds[H * 64];
  __shared__ __attribute__((aligned(16))) uint32_t rsk[kRanked ? kChunk : 1];   // the chunk's keys in bin order
  __shared__ __attribute__((aligned(16))) uint16_t rsp[kRanked ? kChunk : 1];   // and their chunk-local positions
  __shared__ uint32_t rscr[kThreads / kWave + 1];
  __shared__ uint32_t fix_n;                          // a fused append's rows in this chunk
  __shared__ int32_t fix_row[kThreads > 64 ? kThreads : 1];
  __shared__ int32_t fix_pos[kThreads > 64 ? kThreads : 1];
  __shared__ uint32_t fix_key[kThreads > 64 ? kThreads : 1];
  uint32_t *hist = lds_main;
  uint32_t *skeys = lds_main + kHistBins / 2;

  if ((int)blockIdx.y >= nq) {   // a fused append's rows
    const int row = (int)(((int64_t)(blockIdx.y - nq) * gridDim.x + blockIdx.x) * kNumWaves +
                          threadIdx.x / kWave);
    if (row < ap.n) append_row(ap, row, threadIdx.x & (kWave - 1));
    return;
  }
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
  const int32_t sq = q_seq[q];
  const uint8_t *seq_base = idx_k + (int64_t)sq * capacity * kBpt;
  // a fused append: thread r's row (read now, used after the stream; the
  // arrays hold at least one entry, so the clamped read is in bounds)
  const bool fuse = ap.n > 0 && ap.idx_in != nullptr && !Ctx::kDirectHist;   // uniform
  const int ar = max(0, min((int)threadIdx.x, ap.n - 1));
  const int32_t aseq = ap.seq[ar], apos = ap.pos[ar];

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
  if (fuse) {
    // appended positions in this chunk: their keys from the rows' input
    if (threadIdx.x == 0) fix_n = 0;
    __syncthreads();
    if ((int)threadIdx.x < ap.n && aseq == sq && apos >= t_begin && apos < t_end) {
      const uint32_t f = atomicAdd(&fix_n, 1u);
      fix_row[f] = threadIdx.x;
      fix_pos[f] = apos;
    }
    __syncthreads();
    const int nfix = (int)fix_n;
    for (int f = wave; f < nfix; f += kNumWaves) {   // uniform per wave
      // lane (tl, h): head h's chain over the row's channels 0..63, then the
      // heads added in order -- the canonical score (every group of H lanes
      // computes the same)
      const int r = fix_row[f];
      const uint4 *src = reinterpret_cast<const uint4 *>(ap.idx_in + (int64_t)r * ap.idx_elems + h * 64);
      const float *qh = qlds + h * 64;   // (the query from LDS and a rolled loop: few registers)
      float acc = 0.0f;
#pragma unroll 1
      for (int j = 0; j < 8; ++j) {
        const uint4 rw = src[j];
        const uint32_t w4[4] = {rw.x, rw.y, rw.z, rw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = __builtin_fmaf(qh[8 * j + 2 * e], idx_key_value(w4[e] & 0xFFFFu, kFp8Keys), acc);
          acc = __builtin_fmaf(qh[8 * j + 2 * e + 1], idx_key_value(w4[e] >> 16, kFp8Keys), acc);
        }
      }
      const uint32_t key = score_key(head_sum_ltr<H>(acc));
      if (lane == 0) fix_key[f] = key;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int f = 0; f < nfix; ++f) {
        const int64_t i = fix_pos[f] - t_begin;
        const uint32_t old = skeys[i], key = fix_key[f];
        skeys[i] = key;
        hist[old >> 21] -= 1u << ((old >> 16) & 16u);
        hist[key >> 21] += 1u << ((key >> 16) & 16u);
        if (kPool) {   // the block maximum of the position's 8-block
          const int64_t b0 = i / kPoolBlock * kPoolBlock;
          uint32_t m = 0u;
          for (int64_t j = b0; j < min(b0 + kPoolBlock, t_end - t_begin); ++j) m = max(m, skeys[j]);
          const uint32_t om = sblk[i / kPoolBlock];
          sblk[i / kPoolBlock] = m;
          histb[om >> 21] -= 1u << ((om >> 16) & 16u);
          histb[m >> 21] += 1u << ((m >> 16) & 16u);
        }
      }
    }
    __syncthreads();
  }

  const int64_t cnt = t_end - t_begin;
  if constexpr (kRanked) {
    const int64_t rec = (int64_t)q * gridDim.x + blockIdx.x;
    rank_record<kThreads, kChunk>(hist, skeys, [&](int i) { return i < (int)cnt; }, rsk, rsp, rscr,
                                  keys_tok + (int64_t)q * tok_stride + t_begin,
                                  rk.pos + (int64_t)q * tok_stride + t_begin,
                                  rk.ge + rec * kHistBins, rk.coarse + rec * (kHistBins / 64));
    return;
  }
  // the chunk's keys and block maxima in one burst of coalesced stores
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
// nothing to coalesce across entries) and runs that head's fp32 chain of
// fused multiply-adds over channels 0..63 in order; head_sum_ltr adds the
// head sums from head 0 up: the same bits as score_kernel.  The group's first
// lane stores the key; the 12-bit histogram is aggregated in LDS, where only
// the bins in use are cleared and flushed.
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
  float acc = 0.0f;   // one chain over the head's 64 channels
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
  }
  const float hs = head_sum_ltr<H>(acc);
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

// gather_rank_kernel: Reindex over a pool whose selection takes ranked
// records (kRanked).  grid (records, nq); workgroup w scores the pool
// entries [w kGatherRec, (w+1) kGatherRec) in rounds of kGatherThreads / H
// entries (H lanes per entry, as gather_score_kernel: the same bits), the
// next round's loads in flight while one is scored, and stores the record of
// its candidates (the entries in [0, q_pos]) by rank_record.
template <int H, bool kFp8Keys>
__global__ void __launch_bounds__(kGatherThreads) gather_rank_kernel(
    const uint8_t *__restrict__ idx_k, int64_t capacity, const uint16_t *__restrict__ q_idx,
    int32_t q_fp8, const int32_t *__restrict__ q_seq, const int32_t *__restrict__ q_pos,
    const int32_t *__restrict__ pool_in, int32_t pool_len, uint32_t *__restrict__ keys,
    int64_t stride, uint16_t *__restrict__ rpos, uint16_t *__restrict__ rge,
    uint16_t *__restrict__ rcoarse) {
  constexpr int kEsz = kFp8Keys ? 1 : 2;
  constexpr int kLoads = 4 * kEsz;                   // 16-B pieces per head (64 channels)
  constexpr int kEntries = kGatherThreads / H;       // entries per round
  constexpr int kRounds = kGatherRec / kEntries;
  static_assert(kGatherRec == kGatherThreads, "one pool entry per thread staged");
  __shared__ __attribute__((aligned(16))) float qlds[H * kQPitch];
  __shared__ __attribute__((aligned(16))) uint32_t hist[kHistBins / 2];   // 16-bit bins in pairs
  __shared__ uint32_t skeys[kGatherRec];
  __shared__ int32_t spos[kGatherRec];   // the entries' positions, -1: not a candidate
  __shared__ __attribute__((aligned(16))) uint32_t rsk[kGatherRec];
  __shared__ __attribute__((aligned(16))) uint16_t rsp[kGatherRec];
  __shared__ uint32_t rscr[kGatherThreads / kWave + 1];
  const int q = blockIdx.y;
  const int w = blockIdx.x;
  const int tid = threadIdx.x;
  const int h = tid % H;
  const int32_t qp = q_pos[q];
  {
    // this thread's pool entry (a clamped read: entries past the pool are dropped)
    const int64_t e = (int64_t)w * kGatherRec + tid;
    const int32_t p = pool_in[(int64_t)q * pool_len + min(e, (int64_t)pool_len - 1)];
    spos[tid] = (e < pool_len && p >= 0 && p <= qp) ? p : -1;
  }
  for (int i = tid; i < kHistBins / 2; i += kGatherThreads) hist[i] = 0u;
  for (int i = tid; i < H * 64; i += kGatherThreads) {
    float f = bf16_to_f32(q_idx[(int64_t)q * H * 64 + i]);
    if (q_fp8) f = e4m3_to_f32(e4m3_from_f32_nonneg(fabsf(f)) | ((__float_as_uint(f) >> 24) & 0x80u));
    qlds[(i / 64) * kQPitch + i % 64] = f;
  }
  __syncthreads();
  const uint8_t *base = idx_k + (int64_t)q_seq[q] * capacity * (H * 64 * kEsz);
  const float *qh = qlds + h * kQPitch;
  auto load = [&](int r, uint4 (&buf)[kLoads]) {
    const int32_t p = spos[r * kEntries + tid / H];
    const uint8_t *src = base + idx_chunk_offset<H, kEsz>(p >= 0 ? p : 0, h, 0);
#pragma unroll
    for (int v = 0; v < kLoads; ++v) buf[v] = *reinterpret_cast<const uint4 *>(src + v * 1024);
  };
  auto score = [&](int r, const uint4 (&buf)[kLoads]) {
    float acc = 0.0f;   // one chain over the head's 64 channels
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
      if (kFp8Keys) {
        const uint4 a = buf[j];
        const uint32_t wd[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(wd[k], false);
          auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(wd[k], true);
          acc = __builtin_fmaf(qv[4 * k + 0], lo[0], acc);
          acc = __builtin_fmaf(qv[4 * k + 1], lo[1], acc);
          acc = __builtin_fmaf(qv[4 * k + 2], hi[0], acc);
          acc = __builtin_fmaf(qv[4 * k + 3], hi[1], acc);
        }
      } else {
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) {
          const uint4 a = buf[2 * j + hv];
          const uint32_t wd[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            acc = __builtin_fmaf(qv[8 * hv + 2 * k], __uint_as_float(wd[k] << 16), acc);
            acc = __builtin_fmaf(qv[8 * hv + 2 * k + 1], __uint_as_float(wd[k] & 0xFFFF0000u), acc);
          }
        }
      }
    }
    const uint32_t key = score_key(head_sum_ltr<H>(acc));
    if (h == 0) skeys[r * kEntries + tid / H] = key;
  };
  uint4 bA[kLoads], bB[kLoads];
  load(0, bA);
#pragma unroll
  for (int r = 0; r < kRounds; r += 2) {
    load(r + 1, bB);
    score(r, bA);
    if (r + 2 < kRounds) load(r + 2, bA);
    score(r + 1, bB);
  }
  __syncthreads();
  const uint32_t mykey = skeys[tid];
  if (spos[tid] >= 0) atomicAdd(&hist[mykey >> 21], 1u << ((mykey >> 16) & 16u));
  __syncthreads();
  const int64_t rec = (int64_t)q * gridDim.x + w;
  rank_record<kGatherThreads, kGatherRec>(
      hist, skeys, [&](int i) { return spos[i] >= 0; }, rsk, rsp, rscr,
      keys + (int64_t)q * stride + (int64_t)w * kGatherRec,
      rpos + (int64_t)q * stride + (int64_t)w * kGatherRec, rge + rec * kHistBins,
      rcoarse + rec * (kHistBins / 64));
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
  int32_t hsrc;           // HistSource of a direct array (kHistKeys or kHistGlobal)
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
  // region / 256 x 4 keys per lane; key (k, lane, e) sits at start + k*256 + lane*4 + e.
  // Branch-free loads (all in flight together): addresses clamped into the
  // query's row; keys of steps past `iters` or at or past n are masked below.
  const int iters = A.region / 256;   // uniform, <= kIters
  const int64_t last4 = A.n_stride - 4;
  uint32_t kv[kIters][4];
#pragma unroll
  for (int k = 0; k < kIters; ++k) {
    const int64_t i0 = min(start + k * 256 + lane * 4, last4);
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kq + i0));
    kv[k][0] = v.x;
    kv[k][1] = v.y;
    kv[k][2] = v.z;
    kv[k][3] = v.w;
  }
  uint32_t *hs = A.hist + (int64_t)q * A.hstride;
  const Threshold th = hist_threshold(hs, A.hcopies, n, A.kk, lh, scratch, res);
  // the second histogram (bits 19..8 of the threshold bin's keys) is added
  // into global memory (cleared with the first)
  const bool use_h2 = th.keff > 0u && lh[th.b1] <= kH2MaxKeys;
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
  // A short key array is read by this workgroup whole, in one batch of loads
  // issued first (keys 4*tid + 4096*it .. +3 of iteration it) and held in
  // registers for the histogram, the count and the compaction.  The loads
  // are branch-free, so that all of them are in flight together (a load under
  // a lane-dependent branch is waited for before the branch closes): every
  // lane loads four whole keys, its address clamped into the query's row;
  // keys at or past n are masked wherever they are used.
  constexpr int kDirectIters = (int)(kDirectMax / (4 * kSelectThreads));
  const uint32_t *kq = A.keys + (int64_t)q * A.n_stride;
  uint4 kr[kDirectIters];
  if (A.direct) {
    const int64_t last4 = A.n_stride - 4;
#pragma unroll
    for (int it = 0; it < kDirectIters; ++it) {
      const int64_t i0 = min((int64_t)it * 4 * kSelectThreads + 4 * tid, last4);
      kr[it] = *reinterpret_cast<const uint4 *>(kq + i0);
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
  if (A.direct && A.hsrc == kHistGlobal) {
    th = hist_threshold(hs, A.hcopies, n, A.kk, hist, scratch, res);
  } else if (A.direct) {
    // the 12-bit histogram of the short key array, built here in LDS (the
    // keys past n are not counted)
    for (int i = tid; i < kHistBins; i += kSelectThreads) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kDirectIters; ++it) {
      const int64_t i0 = (int64_t)it * 4 * kSelectThreads + 4 * tid;
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
    // per iteration this lane's candidates and the wave's exclusive scan of
    // them (at most 252: two 16-bit halves per word)
    uint32_t wx[kDirectIters / 2];
#pragma unroll
    for (int i = 0; i < kDirectIters / 2; ++i) wx[i] = 0u;
#pragma unroll
    for (int it = 0; it < kDirectIters; ++it) {
      const int i0 = it * 4 * kSelectThreads + 4 * tid;
      const uint32_t k4[4] = {kr[it].x, kr[it].y, kr[it].z, kr[it].w};
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) c += (th.keff > 0 && i0 + e < nd && k4[e] >= thr) ? 1u : 0u;
      const uint32_t inc = wave_inclusive_scan(c);
      wx[it / 2] |= (inc - c) << (16 * (it & 1));
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
    // the candidates written in index order
#pragma unroll
    for (int it = 0; it < kDirectIters; ++it) {
      const int i0 = it * 4 * kSelectThreads + 4 * tid;
      const uint32_t k4[4] = {kr[it].x, kr[it].y, kr[it].z, kr[it].w};
      uint32_t o = goff[it * kWaves + wave] + ((wx[it / 2] >> (16 * (it & 1))) & 0xFFFFu);
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
// ranked_select_kernel: the Top-K of one query from its ranked records
// (kRanked): a Full scan's chunk records, or a Reindex pool's records of
// kGatherRec entries.  grid (nq), kRankThreads threads; wave w takes records
// w, w + 16, w + 32, w + 48.
//   1. the coarse tables: per 64-bin group j, the keys at or above bin 64 j
//      summed over the records (group 0: the candidate count, so keff =
//      min(K, candidates)); the keff-th largest key lies in the last group J
//      whose sum reaches keff (the sums fall with j).
//   2. ge of the 64 bins of group J in every record: likewise the bin b1.
//      Per record, its first ge(b1 + 1) keys lie above bin b1 and are all
//      taken, the next ge(b1) - ge(b1 + 1) are bin b1's.
//   3. those keys: the ones above b1 set their candidate index (record *
//      chunk + index in the record) in the selection bitmap, bin b1's go to
//      LDS.  Radix passes on bits 19..8 and 7..0 of bin b1's keys give the
//      keff-th largest key tau; keys above tau are taken, and of the keys
//      equal to tau the ones at the lowest indices (a tie bitmap, scanned in
//      index order).
// The bitmap, scanned in order, gives the indices ascending -- positions, or
// pool entries (looked up at the end; a pool lists its positions in
// ascending order); -1 padding.  The first keys of every record (4096 over
// the records) are read with the coarse tables, before anything says how
// many are needed (usually all that are); bin b1 holding more keys than LDS
// takes (heavy ties) is read from the records again in each pass.
// ---------------------------------------------------------------------------
constexpr int kRankThreads = 1024;
constexpr int kRankWaves = kRankThreads / kWave;
constexpr int kRankCap = 8192;                       // bin-b1 keys held in LDS
constexpr int kRankMaxKeys = (int)kMaxRankedKeys;
constexpr int kRankWords = kRankMaxKeys / 32;        // selection bitmap words
static_assert(4 * kRankWaves == kMaxRankedChunks && kMaxRankedChunks == kWave,
              "at most four records per wave; one per lane of a wave");
static_assert(kRankWords == 2 * kRankThreads, "two bitmap words per thread");

struct RankedSel {
  const uint32_t *keys;     // [nq][n_stride] each record's keys in bin order
  const uint16_t *pos;      // [nq][n_stride] their indices within the record
  const uint16_t *ge;       // [nq][nchunks][kHistBins]
  const uint16_t *coarse;   // [nq][nchunks][kHistBins / 64]
  int64_t n_stride;
  int32_t nchunks;          // records per query
  int32_t chunk;            // candidates per record: candidate = record * chunk + index
  int32_t *out;             // [nq][kk]
  int32_t kk;
  const int32_t *pool;      // Reindex pool [nq][pool_len] (candidates = its entries), or nullptr
  int32_t pool_len;
};

// The query's taken keys as one list: first every chunk's keys above bin b1,
// then every chunk's bin-b1 keys.  Per chunk (LDS tables): lo = its keys above
// b1, hi = lo + its bin-b1 keys, aoff / boff = where its part of each half
// starts.  Entry g of the bin-b1 half lies in the last chunk whose boff
// reaches g (chunks without such keys share the next one's offset).
struct RankedTabs {
  const uint32_t *lo, *hi, *boff;
  int chunk;
  int nrec;
  __device__ __forceinline__ int64_t bin_index(uint32_t g) const {
    int c = 0;
#pragma unroll
    for (int k = 1; k < nrec; ++k) c += boff[k] <= g ? 1 : 0;
    return (int64_t)c * chunk + lo[c] + (g - boff[c]);
  }
};

__device__ __forceinline__ void set_bit(uint32_t *bm, uint32_t p) {
  atomicOr(&bm[p >> 5], 1u << (p & 31u));
}

// The passes over bin b1's keys: the key and position of its entry g.
struct RankedBinLds {
  const uint32_t *k;
  const uint16_t *p;
  __device__ __forceinline__ uint32_t key(uint32_t g) const { return k[g]; }
  __device__ __forceinline__ uint32_t pos(uint32_t g) const { return p[g]; }
};
struct RankedBinGlobal {
  const uint32_t *k;   // the query's keys row
  const uint16_t *p;   // the query's positions row
  RankedTabs t;
  __device__ __forceinline__ uint32_t key(uint32_t g) const { return k[t.bin_index(g)]; }
  __device__ __forceinline__ uint32_t pos(uint32_t g) const {
    const int64_t r = t.bin_index(g);
    return (uint32_t)(r / t.chunk * t.chunk) + p[r];
  }
};

// tau among bin b1's T keys (need = how many of them are taken), then the
// selection bits of the ones taken.  All threads; barriers.
template <class Bin>
__device__ void ranked_refine(const Bin &bin, uint32_t T, uint32_t b1, uint32_t need,
                              uint32_t *hist, uint32_t *sel, uint32_t *tie, int nwords,
                              uint32_t *scratch, uint32_t *res) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kHistBins; i += kRankThreads) hist[i] = 0u;
  __syncthreads();
  for (uint32_t g = tid; g < T; g += kRankThreads) atomicAdd(&hist[(bin.key(g) >> 8) & 0xFFFu], 1u);
  __syncthreads();
  select_bin(hist, kHistBins, need, scratch, res);
  const uint32_t pre24 = (b1 << 12) | res[0];
  const uint32_t need2 = need - res[1];
  __syncthreads();   // res read
  for (int i = tid; i < 256; i += kRankThreads) hist[i] = 0u;
  __syncthreads();
  for (uint32_t g = tid; g < T; g += kRankThreads) {
    const uint32_t k = bin.key(g);
    if ((k >> 8) == pre24) atomicAdd(&hist[k & 0xFFu], 1u);
  }
  __syncthreads();
  select_bin(hist, 256, need2, scratch, res);
  const uint32_t tau = (pre24 << 8) | res[0];
  const uint32_t ties_wanted = need2 - res[1];
  const bool all_ties = ties_wanted == hist[res[0]];   // uniform
  for (uint32_t g = tid; g < T; g += kRankThreads) {
    const uint32_t k = bin.key(g);
    if (k > tau || (all_ties && k == tau)) set_bit(sel, bin.pos(g));
    else if (k == tau) set_bit(tie, bin.pos(g));
  }
  __syncthreads();
  if (all_ties) return;
  // the ties_wanted ties at the lowest positions: thread t holds words 2t, 2t+1
  const int w0 = 2 * tid;
  const uint32_t t0 = w0 < nwords ? tie[w0] : 0u;
  const uint32_t t1 = w0 + 1 < nwords ? tie[w0 + 1] : 0u;
  uint32_t total;
  uint32_t rank = block_exclusive_scan((uint32_t)(__popc(t0) + __popc(t1)), scratch, total);
  uint32_t m[2] = {t0, t1};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    uint32_t take = 0u;
    while (m[e] != 0u && rank < ties_wanted) {
      const uint32_t b = m[e] & (0u - m[e]);
      take |= b;
      m[e] ^= b;
      ++rank;
    }
    if (take) sel[w0 + e] |= take;
  }
  __syncthreads();
}

// One taken key (entry i of chunk c's record, a key of the query's list):
// above b1 -> its selection bit; in bin b1 -> LDS slot boff + i - lo.
__device__ __forceinline__ void ranked_take(uint32_t i, int c, int C, uint32_t key, uint32_t pos,
                                            const uint32_t *lo, const uint32_t *hi,
                                            const uint32_t *boff, bool in_lds, uint32_t *sel,
                                            uint32_t *bkey, uint16_t *bpos) {
  if (i < lo[c]) {
    set_bit(sel, (uint32_t)(c * C) + pos);
  } else if (i < hi[c] && in_lds) {
    const uint32_t g = boff[c] + i - lo[c];
    bkey[g] = key;
    bpos[g] = (uint16_t)((uint32_t)(c * C) + pos);
  }
}

// kRecPerWave: records per wave, 1 (up to 16 records) or 4 (up to 64)
template <int kRecPerWave>
__global__ void __launch_bounds__(kRankThreads) ranked_select_kernel(
    const RankedSel R, const int32_t *__restrict__ q_pos) {
  constexpr int kRecs = kRecPerWave * kRankWaves;
  __shared__ uint32_t tabc[kRecs][65];   // coarse tables (padded rows)
  __shared__ uint32_t tabf[kRecs][65];   // the 64-bin window of group J
  __shared__ uint32_t tsum[kRankWaves][65];         // per wave: its records' sums
  __shared__ __attribute__((aligned(16))) uint32_t hist[kHistBins];
  __shared__ uint32_t sel[kRankWords];
  __shared__ uint32_t tie[kRankWords];
  __shared__ uint32_t bkey[kRankCap];
  __shared__ uint16_t bpos[kRankCap];
  __shared__ uint32_t tlo[kMaxRankedChunks], thi[kMaxRankedChunks], tboff[kMaxRankedChunks];
  __shared__ uint32_t txoff[kMaxRankedChunks];
  __shared__ uint32_t scratch[kRankWaves + 1];
  __shared__ uint32_t res[5];
  static_assert(kRecs <= kMaxRankedChunks, "records");

  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int C = R.chunk;
  const int64_t rec = (int64_t)q * R.nchunks;
  const uint32_t *kq = R.keys + (int64_t)q * R.n_stride;
  const uint16_t *pq = R.pos + (int64_t)q * R.n_stride;
  // round 1, all independent of q_pos: the coarse tables (records a query
  // does not reach are masked below) and the first `early` keys of every
  // record (thread t: entry t % early of records t / early + 1024 u / early),
  // addresses clamped into the query's rows
  uint32_t cv[kRecPerWave];
#pragma unroll
  for (int k = 0; k < kRecPerWave; ++k)
    cv[k] = R.coarse[(rec + min(wave + kRankWaves * k, R.nchunks - 1)) * (kHistBins / 64) + lane];
  // early keys per record: 4096 / (a power of two >= the record count)
  const int esh = R.nchunks <= 16 ? 8 : (R.nchunks <= 32 ? 7 : 6);
  const uint32_t early = 1u << esh;
  const uint32_t ei = (uint32_t)tid & (early - 1u);
  uint32_t ek[4], ep[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = (tid + kRankThreads * u) >> esh;
    const int64_t r = min((int64_t)c * C + ei, R.n_stride - 1);
    ek[u] = kq[r];
    ep[u] = pq[r];
  }
  const int32_t qp = q_pos[q];
  sel[2 * tid] = 0u;
  sel[2 * tid + 1] = 0u;
  tie[2 * tid] = 0u;
  tie[2 * tid + 1] = 0u;
  // the bitmap's range (candidate indices) and the records this call wrote:
  // a Full scan writes the chunks that hold visible positions (q_pos <
  // capacity; clamped to the records regardless), a pool's every record
  const bool pooled = R.pool != nullptr;   // uniform
  const int64_t n = pooled ? (int64_t)R.pool_len
                           : max((int64_t)1, min((int64_t)qp + 1, (int64_t)R.nchunks * C));
  const int nch = pooled ? R.nchunks : (int)((n + C - 1) / C);
  const int nwords = (int)((n + 31) / 32);
  int32_t *oq = R.out + (int64_t)q * R.kk;
  {
    uint32_t t = 0u;
#pragma unroll
    for (int k = 0; k < kRecPerWave; ++k) {
      const int c = wave + kRankWaves * k;
      const uint32_t v = c < nch ? cv[k] : 0u;
      tabc[c][lane] = v;
      t += v;
    }
    tsum[wave][lane] = t;
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t t = 0u;
#pragma unroll
    for (int w = 0; w < kRankWaves; ++w) t += tsum[w][lane];
    // lane 0 holds the candidate count (every candidate is at or above bin 0)
    const uint32_t ncand = (uint32_t)__builtin_amdgcn_readfirstlane(t);
    const uint32_t kf = (uint32_t)min((int64_t)R.kk, (int64_t)ncand);
    const uint64_t b = __ballot(t >= kf);
    if (lane == 0) {
      res[0] = (uint32_t)__popcll(b) - 1u;
      res[4] = kf;
    }
  }
  __syncthreads();
  const uint32_t J = res[0];
  const uint32_t keff = res[4];
  // round 2
  {
    uint32_t t = 0u;
#pragma unroll
    for (int k = 0; k < kRecPerWave; ++k) {
      const int c = wave + kRankWaves * k;
      const uint32_t v = c < nch ? R.ge[(rec + min(c, nch - 1)) * kHistBins + 64 * J + lane] : 0u;
      tabf[c][lane] = v;
      t += v;
    }
    tsum[wave][lane] = t;   // (wave 0 read the round-1 sums before the barrier above)
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t t = 0u;
#pragma unroll
    for (int w = 0; w < kRankWaves; ++w) t += tsum[w][lane];
    const uint32_t L = (uint32_t)__popcll(__ballot(t >= keff)) - 1u;
    // lane c: record c's keys in bin b1 or above (hi) and above it (lo)
    const int c = lane;
    const bool mine = c < nch;
    const int cr = min(c, kRecs - 1);   // (rows past kRecs are not read: mine is false there)
    const uint32_t hi = mine ? tabf[cr][L] : 0u;
    const uint32_t lo = !mine ? 0u : (L < 63u ? tabf[cr][L + 1] : (J < 63u ? tabc[cr][J + 1] : 0u));
    const uint32_t a = lo, bb = hi - lo;
    const uint32_t ia = wave_inclusive_scan(a);
    const uint32_t ib = wave_inclusive_scan(bb);
    tlo[c] = lo;
    thi[c] = hi;
    tboff[c] = ib - bb;
    // the keys a record needs past its early ones, as one list (record by record)
    const uint32_t ex = hi > early ? hi - early : 0u;
    const uint32_t ix = wave_inclusive_scan(ex);
    txoff[c] = ix - ex;
    if (lane == kWave - 1) {
      res[0] = 64u * J + L;
      res[1] = ia;   // keys above bin b1
      res[2] = ib;   // keys in bin b1
      res[3] = ix;   // keys past the early ones
    }
  }
  __syncthreads();
  const uint32_t b1 = res[0], above = res[1], T = res[2];
  const uint32_t nextra = res[3];   // keys some records need past their early ones
  const bool in_lds = T <= (uint32_t)kRankCap;   // uniform
  // round 3: the early keys, then any a record needs beyond them
  if (keff > 0u) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = (tid + kRankThreads * u) >> esh;
      if (c < nch) ranked_take(ei, c, C, ek[u], ep[u], tlo, thi, tboff, in_lds, sel, bkey, bpos);
    }
    // entry f of the list: the last record whose offset reaches f (records
    // needing none share the next one's offset), by a binary search over the
    // offsets; all of a thread's loads issue together
    for (uint32_t f0 = 0; f0 < nextra; f0 += 4 * kRankThreads) {   // uniform
      uint32_t xk[4], xp[4];
      int xc[4];
      uint32_t xi[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t f = min(f0 + tid + u * kRankThreads, nextra - 1u);
        int lo = 0, hi = nch - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (txoff[mid] <= f) lo = mid; else hi = mid - 1;
        }
        xc[u] = lo;
        xi[u] = early + (f - txoff[lo]);
        const int64_t r = (int64_t)lo * C + xi[u];
        xk[u] = kq[r];
        xp[u] = pq[r];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (f0 + tid + u * kRankThreads < nextra)
          ranked_take(xi[u], xc[u], C, xk[u], xp[u], tlo, thi, tboff, in_lds, sel, bkey, bpos);
    }
    __syncthreads();
    const uint32_t need = keff - above;   // >= 1: the keff-th key lies in bin b1
    if (in_lds)
      ranked_refine(RankedBinLds{bkey, bpos}, T, b1, need, hist, sel, tie, nwords, scratch, res);
    else
      ranked_refine(RankedBinGlobal{kq, pq, RankedTabs{tlo, thi, tboff, C, nch}}, T, b1, need,
                    hist, sel, tie, nwords, scratch, res);
  }
  // the selection in index order: thread t emits indices 64t .. 64t+63 (a
  // pool's entries are in ascending position order); pool entries are looked
  // up after the indices are placed (through LDS, all loads at once)
  const int w0 = 2 * tid;
  uint32_t m[2] = {w0 < nwords ? sel[w0] : 0u, w0 + 1 < nwords ? sel[w0 + 1] : 0u};
  uint32_t total;
  uint32_t o = block_exclusive_scan((uint32_t)(__popc(m[0]) + __popc(m[1])), scratch, total);
  const bool via_lds = pooled && keff <= (uint32_t)kRankCap;   // uniform
  const int32_t *prow = pooled ? R.pool + (int64_t)q * R.pool_len : nullptr;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    while (m[e] != 0u) {
      const int b = __ffs(m[e]) - 1;
      m[e] &= m[e] - 1u;
      const int32_t id = 32 * (w0 + e) + b;
      if (o < keff) {
        if (via_lds) bkey[o] = (uint32_t)id;
        else oq[o] = pooled ? prow[id] : id;
      }
      ++o;
    }
  }
  if (via_lds) {
    __syncthreads();
    for (uint32_t i = tid; i < keff; i += kRankThreads) oq[i] = prow[bkey[i]];
  }
  for (int64_t i = (int64_t)keff + tid; i < R.kk; i += kRankThreads) oq[i] = -1;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int H, bool kFp8, bool kPool, int kThreads, int kChunk>
void launch_score_shape(const IndexArgs &a, int64_t n_cand_max, hipStream_t s) {
  const csa2_cache &c = *a.cache;
  const TopkWorkspace &L = a.layout;
  dim3 grid((unsigned)((n_cand_max + kChunk - 1) / kChunk), (unsigned)a.nq);
  uint32_t *keys = reinterpret_cast<uint32_t *>(a.ws + L.tok.keys);
  // a fused append (only the 256-thread shapes take one): its rows in extra
  // workgroup rows past the queries, kThreads / 64 rows per workgroup; the
  // append arrays always point at valid memory (the kernel reads entry 0)
  AppendRows ap = a.ap;
  if (kThreads != 256 || ap.n <= 0) {
    ap.n = 0;
    ap.seq = a.q_seq;
    ap.pos = a.q_pos;
  } else {
    const int64_t per = (int64_t)grid.x * (kThreads / kWave);
    grid.y += (unsigned)((ap.n + per - 1) / per);
  }
  if (L.tok.hsrc == kRanked) {
    // the layout chose ranked chunks by the same shape rule (score_chunk)
    if constexpr (!kPool && kThreads == 256) {
      if (L.tok.chunk != kChunk || (int64_t)L.tok.nchunks != (int64_t)grid.x) return;   // never
      const RankedOut rk{reinterpret_cast<uint16_t *>(a.ws + L.tok.rk_pos),
                         reinterpret_cast<uint16_t *>(a.ws + L.tok.rk_ge),
                         reinterpret_cast<uint16_t *>(a.ws + L.tok.rk_coarse)};
      hipLaunchKernelGGL((score_kernel<H, kFp8, false, kThreads, kChunk, true>), grid, dim3(kThreads),
                         0, s, static_cast<const uint8_t *>(c.idx_k), (int64_t)c.capacity, a.q_idx,
                         a.q_fp8, a.q_seq, a.q_pos, keys, L.tok.n, nullptr, nullptr, (int64_t)0,
                         nullptr, (int64_t)0, 1, rk, ap, a.nq);
    }
    return;
  }
  hipLaunchKernelGGL((score_kernel<H, kFp8, kPool, kThreads, kChunk>), grid, dim3(kThreads), 0, s,
                     static_cast<const uint8_t *>(c.idx_k), (int64_t)c.capacity, a.q_idx, a.q_fp8,
                     a.q_seq, a.q_pos, keys, L.tok.n,
                     reinterpret_cast<uint32_t *>(a.ws + L.tok.hist),
                     kPool ? reinterpret_cast<uint32_t *>(a.ws + L.blk.keys) : nullptr, L.blk.n,
                     kPool ? reinterpret_cast<uint32_t *>(a.ws + L.blk.hist) : nullptr,
                     L.tok.hstride, L.tok.hcopies, RankedOut{nullptr, nullptr, nullptr}, ap, a.nq);
}

// Workgroup shape from the amount of work: long streams when there are enough
// groups, one-wave groups for small searches so that they spread over the chip.
// Returns the candidates per workgroup (4096, 2048 or 64).
int32_t score_chunk(int32_t nq, int64_t n_cand_max, bool pool) {
  const int64_t big = (int64_t)nq * ((n_cand_max + 4095) / 4096);
  const int64_t mid = (int64_t)nq * ((n_cand_max + 2047) / 2048);
  if (big >= kBigChunkMinGroups) return 4096;
  if (mid >= kSmallGridGroups || pool) return 2048;
  return 64;
}

template <int H, bool kFp8, bool kPool>
void launch_score(const IndexArgs &a, int64_t n_cand_max, hipStream_t s) {
  switch (score_chunk(a.nq, n_cand_max, kPool)) {
    case 4096: launch_score_shape<H, kFp8, kPool, 256, 4096>(a, n_cand_max, s); break;
    case 2048: launch_score_shape<H, kFp8, kPool, 256, 2048>(a, n_cand_max, s); break;
    default: launch_score_shape<H, kFp8, false, 64, 64>(a, n_cand_max, s); break;
  }
}

template <int H, bool kFp8>
void launch_score_mode(const IndexArgs &a, int64_t n, bool pool, bool reindex_pool, hipStream_t s) {
  if (reindex_pool && a.layout.tok.hsrc == kRanked) {
    const TopkWorkspace &L = a.layout;
    hipLaunchKernelGGL((gather_rank_kernel<H, kFp8>), dim3((unsigned)L.tok.nchunks, (unsigned)a.nq),
                       dim3(kGatherThreads), 0, s, static_cast<const uint8_t *>(a.cache->idx_k),
                       (int64_t)a.cache->capacity, a.q_idx, a.q_fp8, a.q_seq, a.q_pos, a.pool_in,
                       a.pool_len, reinterpret_cast<uint32_t *>(a.ws + L.tok.keys), L.tok.n,
                       reinterpret_cast<uint16_t *>(a.ws + L.tok.rk_pos),
                       reinterpret_cast<uint16_t *>(a.ws + L.tok.rk_ge),
                       reinterpret_cast<uint16_t *>(a.ws + L.tok.rk_coarse));
  } else if (reindex_pool) {
    const TopkWorkspace &L = a.layout;
    constexpr int kEntries = kGatherThreads / H;
    hipLaunchKernelGGL((gather_score_kernel<H, kFp8>),
                       dim3((unsigned)((a.pool_len + kEntries - 1) / kEntries), (unsigned)a.nq),
                       dim3(kGatherThreads), 0, s, static_cast<const uint8_t *>(a.cache->idx_k),
                       (int64_t)a.cache->capacity, a.q_idx, a.q_fp8, a.q_seq, a.q_pos, a.pool_in,
                       a.pool_len, reinterpret_cast<uint32_t *>(a.ws + L.tok.keys), L.tok.n,
                       L.tok.hsrc == kHistKeys ? nullptr
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
  p.hsrc = A.hsrc;
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

// Ranked chunks: the keys (in bin order per chunk), their positions, the
// per-bin counts and their coarse tables; no histogram or filter arrays.
size_t carve_ranked(SelectArrays &A, int64_t n_slots, int32_t nq, int32_t chunk) {
  A.n = (n_slots + 63) / 64 * 64;
  A.hsrc = kRanked;
  A.chunk = chunk;
  A.nchunks = (int32_t)((n_slots + chunk - 1) / chunk);
  size_t off = 0;
  A.keys = off;
  off = align256(off + (size_t)nq * A.n * 4);
  A.rk_pos = off;
  off = align256(off + (size_t)nq * A.n * 2);
  A.rk_ge = off;
  off = align256(off + (size_t)nq * A.nchunks * kHistBins * 2);
  A.rk_coarse = off;
  off = align256(off + (size_t)nq * A.nchunks * (kHistBins / 64) * 2);
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
  const int64_t n_tok = reindex_pool ? (int64_t)pool_len : (int64_t)c.capacity;
  size_t off;
  const int32_t chunk = score_chunk(nq, n_tok, false);
  if (!reindex_pool && !pool && chunk >= 2048 && n_tok <= kMaxRankedKeys &&
      (n_tok + chunk - 1) / chunk <= kMaxRankedChunks) {
    // a handful of scorer chunks per query: ranked chunk records
    off = carve_ranked(w.tok, n_tok, nq, chunk);
  } else if (reindex_pool && (int64_t)pool_len <= kMaxRankedChunks * kGatherRec) {
    // a pool of up to 64 runs of kGatherRec entries: ranked records
    off = carve_ranked(w.tok, pool_len, nq, kGatherRec);
  } else {
    // the token and block histograms are filled by the same scorer launch and
    // cleared by one launch: the same number of copies
    const int32_t hc = hist_copies(n_tok);
    off = carve(w.tok, n_tok, nq, 0, hc);
    if (pool) off = carve(w.blk, ((int64_t)c.capacity + kPoolBlock - 1) / kPoolBlock, nq, off, hc);
    // where each selection finds its histogram (see HistSource)
    w.tok.hsrc = reindex_pool ? (pool_len <= kDirectMax ? kHistKeys : kHistGlobal) : kHistGlobal;
    w.blk.hsrc = kHistGlobal;
  }
  w.total = off;
  if (gemm_eligible(c, mode, pool_len, pool_blocks)) {
    w.gemm = gemm_workspace_layout(c, nq);
    w.total = std::max(w.total, w.gemm.total);
  }
  return w;
}

bool append_fusable(const IndexArgs &a) {
  if (a.ap.n <= 0 || a.ap.n > kFuseMaxRows || a.mode == CSA2_REUSE) return false;
  // the rows take up to kFuseMaxRows / 4 extra grid rows past the queries'
  if (a.nq + kFuseMaxRows / 4 > 65535) return false;
  if (a.q_fp8 && gemm_eligible(*a.cache, a.mode, a.pool_len, a.pool_blocks)) return false;
  const bool pool = a.mode == CSA2_FULL && a.pool_blocks > 0;
  const bool reindex_pool = a.mode == CSA2_REINDEX && a.pool_in != nullptr;
  return !reindex_pool && score_chunk(a.nq, a.cache->capacity, pool) >= 2048;
}

hipError_t launch_index_topk(const IndexArgs &a_in, hipStream_t s) {
  // an append the scorer cannot take runs first, on its own
  IndexArgs a = a_in;
  if (a.ap.n > 0 && !append_fusable(a)) {
    const AppendRows &p = a.ap;
    const hipError_t e = launch_kv_append(*a.cache, p.k, p.v, p.idx_in, p.seq, p.pos, p.n, s);
    if (e != hipSuccess) return e;
    a.ap.n = 0;
  }
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
  // 1. clear the global histograms (the token and block histograms are
  //    cleared by one launch when both exist: the block one follows the token
  //    arrays).  Slot histograms and a pool short enough for the resolve to
  //    count need none.
  if (L.tok.hsrc == kHistGlobal) {
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
  if (L.tok.hsrc == kRanked) {
    const RankedSel R{reinterpret_cast<const uint32_t *>(a.ws + L.tok.keys),
                      reinterpret_cast<const uint16_t *>(a.ws + L.tok.rk_pos),
                      reinterpret_cast<const uint16_t *>(a.ws + L.tok.rk_ge),
                      reinterpret_cast<const uint16_t *>(a.ws + L.tok.rk_coarse),
                      L.tok.n, L.tok.nchunks, L.tok.chunk, a.topk_out, a.top_k,
                      reindex_pool ? a.pool_in : nullptr, a.pool_len};
    if (L.tok.nchunks <= kRankWaves)
      hipLaunchKernelGGL(ranked_select_kernel<1>, dim3((unsigned)a.nq), dim3(kRankThreads), 0, s, R,
                         a.q_pos);
    else
      hipLaunchKernelGGL(ranked_select_kernel<4>, dim3((unsigned)a.nq), dim3(kRankThreads), 0, s, R,
                         a.q_pos);
    return hipGetLastError();
  }
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
