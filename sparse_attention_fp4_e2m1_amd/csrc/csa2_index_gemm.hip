// Index scoring on matrix cores (E4M3 index queries against E4M3 index keys)
// and the exact Top-K of those scores.
//
// aiwiki "DeepSeek V4.1-Flash", section "Compressed Sparse Attention 2": a Full
// layer, or a Reindex layer without a pool, scores every causally visible
// position of its sequence.  When many queries of one sequence score together
// (a prefill chunk), the scores are a dense product -- queries x positions,
// contracted over idx_heads x 64 channels -- and run here as fp8 MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales).  Each product of two
// E4M3 values is exact; their fp32 sum follows the matrix core, not the fixed
// order of the streaming scorer.
//
// The Top-K is found without storing the queries x positions score matrix:
//   gemm_prep_kernel    E4M3 copy of the index queries; the length of the
//                       position ranges the product is split into.
//   gemm_score_kernel<1> per query and block of 16 positions, the block's
//                       largest score key (its top 16 bits), in one row per
//                       query.
//   gemm_kth_kernel     per query, t = the K-th largest of those block maxima.
//                       At least K blocks reach t and each holds a score >= t,
//                       so the K-th largest score is >= t: the whole Top-K
//                       scores at least t.  (Fewer than K blocks: t = 0.)
//   gemm_score_kernel<2> the same product again (same instructions, same
//                       operand order, so the same bits) keeping every
//                       (key >= t, position) in position order, in one slot
//                       region per (query, position range).
//   gemm_resolve_kernel per query, the exact selection among the candidates
//                       (ties to the lower position, ascending output), with
//                       the radix passes of the streaming path.
// With continuous scores about K plus a few percent candidates survive.
//
// Long rows take a cheaper first pass.  gemm_score_kernel<3> computes the
// block maxima of the first eighth of every position range's groups of 16
// blocks only (a sample stratified over the ranges, about an eighth of the
// product, run like pass 1 over shorter ranges), and gemm_kth_wave_kernel<true>
// sets t' to the m-th largest sampled maximum, m chosen five standard
// deviations above the expected number of sampled blocks that hold one of
// the K largest scores, so that t' lies below the K-th largest score for
// every query but rare ones.  Pass 2 then emits every position scoring at least t'.  Whatever t'
// is, the result stays exact: when a query gets at least min(K, visible)
// candidates, its K-th largest score is at least t' and every position of
// the Top-K (ties included) is among them.  The launch after pass 2 checks
// exactly that: gemm_score_kernel<2> in its checking form reads every
// query's candidate total and, for the query groups holding a query short of
// them, emits every visible position of those queries (t = 0: the resolve
// then streams them, exact); for the other groups it returns at once.
#include <algorithm>

#include "csa2_select.h"

namespace csa2 {
namespace {

typedef int v8i __attribute__((__vector_size__(8 * sizeof(int))));
typedef float v4f __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kGemmThreads = 512;       // 8 waves, two per SIMD
constexpr int kGemmWaves = kGemmThreads / kWave;
constexpr int kGemmQ = 512;             // queries per workgroup: 64 per wave, 4 column tiles of 16
// Positions per LDS stage (16-row tiles): the lighter block-maximum pass takes
// longer stages (fewer barriers); the emitting pass needs the registers.
#ifndef CSA2_GEMM_STAGE1
#define CSA2_GEMM_STAGE1 128
#endif
#ifndef CSA2_GEMM_STAGE2
#define CSA2_GEMM_STAGE2 64
#endif
constexpr int kGemmTargetGroups = 256;  // workgroups aimed for (one per CU)
constexpr int kBlk = 16;                // positions per block maximum (one row tile)
constexpr int kBlkGroup = 16;           // block maxima a lane collects before one 32-B store
constexpr int kRangeAlign = kBlk * kBlkGroup;   // positions per range: a multiple of this

// The block maxima are stored group-major: the kBlkGroup values of block
// group g of query q at [g][q][0 .. kBlkGroup), so that the 64 lanes of a
// wave (64 consecutive queries) store one contiguous 2 KB run per group.
// Block i of query q:
__device__ __forceinline__ const uint16_t *bmax_at(const uint16_t *bmax, int32_t nq, int q,
                                                   int64_t i) {
  return bmax + ((i / kBlkGroup) * nq + q) * kBlkGroup + i % kBlkGroup;
}
constexpr int kDmaPerTile = 2;          // next-stage pieces a thread loads per row tile
constexpr int kKthThreads = 256;
// Candidates a gemm_resolve_kernel keeps in LDS: ~K(1 + 10 %) with continuous
// scores for K = 2048 and the exact threshold (blocks holding two candidates,
// the threshold's 16-bit granularity), ~1.35 K with the sampled one; at 47 KB
// of LDS per workgroup three share a CU (thousands of queries per call).
// More candidates take the streamed path.
constexpr int kGemmResolveCap = 3584;
constexpr int kGemmResolveThreads = 512;
constexpr int kGemmEarlySlots = 8;      // candidate slots per resolve thread read before the counts
constexpr int kKthRegMax = 32768;       // block maxima a gemm_kth_kernel keeps in registers
constexpr int kSampleEvery = 8;         // the sampled first pass: one block group in kSampleEvery

// Block groups a range of `sub` positions samples (its first ones).
__host__ __device__ constexpr int sampled_groups(int64_t sub) {
  return (int)(sub / kRangeAlign / kSampleEvery > 1 ? sub / kRangeAlign / kSampleEvery : 1);
}
constexpr float kSampleSigma = 5.0f;    // its margin, in standard deviations of the sample count

__device__ __forceinline__ uint32_t e4m3_code(float f) {
  return e4m3_from_f32_nonneg(fabsf(f)) | ((__float_as_uint(f) >> 24) & 0x80u);
}

// E4M3 copy of q_idx (n_elems bf16 values), and plan[0] = the position-range
// length: ceil(L / nranges) rounded up to a multiple of kRangeAlign, with
// L = 1 + max q_pos.
// Also clears tot, the per-query candidate totals pass 2 adds up.
__global__ void __launch_bounds__(256) gemm_prep_kernel(
    const uint16_t *__restrict__ q_idx, int64_t n_elems, uint8_t *__restrict__ q8,
    const int32_t *__restrict__ q_pos, int32_t nq, int32_t nranges, uint32_t *__restrict__ plan,
    uint32_t *__restrict__ tot) {
  if (blockIdx.x == 0) {
    __shared__ int32_t red[256 / kWave];
    int32_t m = -1;
    // sixteen loads in flight per thread per round (4096 queries in one round)
    for (int i0 = 0; i0 < nq; i0 += 16 * 256) {
      int32_t v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = i0 + u * 256 + (int)threadIdx.x;
        v[u] = i < nq ? q_pos[i] : -1;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) m = max(m, v[u]);
    }
    for (int d = 32; d >= 1; d >>= 1) m = max(m, __shfl_xor(m, d, kWave));
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < 256 / kWave; ++w) m = max(m, red[w]);
      const int64_t len = (int64_t)m + 1;
      int64_t sub = (len + nranges - 1) / nranges;
      sub = (sub + kRangeAlign - 1) / kRangeAlign * kRangeAlign;
      plan[0] = (uint32_t)max(sub, (int64_t)kRangeAlign);
    }
  }
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < nq) tot[t] = 0u;   // (the grid has n_elems / 8 >= nq threads)
  const int64_t i0 = t * 8;
  if (i0 >= n_elems) return;
  // eight bf16 values: one 16-byte load where the array allows it
  uint32_t v[4];
  if ((reinterpret_cast<uintptr_t>(q_idx) & 15u) == 0u) {
    const uint4 w = *reinterpret_cast<const uint4 *>(q_idx + i0);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (uint32_t)q_idx[i0 + 2 * e] | ((uint32_t)q_idx[i0 + 2 * e + 1] << 16);
  }
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t h = (uint32_t)(v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    lo |= e4m3_code(bf16_to_f32(h)) << (8 * e);
    const uint32_t h2 = (uint32_t)(v[2 + (e >> 1)] >> (16 * (e & 1))) & 0xFFFFu;
    hi |= e4m3_code(bf16_to_f32(h2)) << (8 * e);
  }
  *reinterpret_cast<uint2 *>(q8 + i0) = make_uint2(lo, hi);
}

// The lowest remaining candidate row of mask m (rows of a, m != 0) into slot
// off of c, then off + 1 and m without that row.  c is the column tile's base
// (the same in every lane) and off a slot index from it whose byte offset fits
// 32 bits, so the store takes its address from scalar registers plus one
// 32-bit offset.
__device__ __forceinline__ void emit_lowest(uint2 *c, uint32_t &off, uint32_t &m, const v4f &a,
                                            int prow) {
  const uint32_t i = (uint32_t)__builtin_ctz(m);
  float v = a[3];   // selects, not a branch per row
  v = (m & 4u) ? a[2] : v;
  v = (m & 2u) ? a[1] : v;
  v = (m & 1u) ? a[0] : v;
  *reinterpret_cast<uint2 *>(reinterpret_cast<char *>(c) + (off << 3)) =
      make_uint2(score_key(v), (uint32_t)prow + i);
  ++off;
  m &= m - 1u;
}

// ---------------------------------------------------------------------------
// gemm_score_kernel
//
// Grid (nranges, ceil(nq / kGemmQ)); workgroup (r, g) takes queries
// [g*512, g*512 + 512) and positions [r*sub, (r+1)*sub) clipped to 1 + the
// largest q_pos among them.  Each wave keeps its 64 queries' E4M3 index
// queries in registers as MFMA B operands (4 column tiles x kSteps k-steps of
// 32 bytes per lane); the 8 waves share the index keys, loaded straight into
// LDS kGemmStage positions (16-row tiles) at a time, two buffers.  With grid.x a
// multiple of 8 all query groups of one range land on one XCD and share the
// keys through its L2.
//
// MFMA operands (16x16x128, 32 bytes per lane): lane l supplies row / column
// l % 16 and the 32 k-slots of lane group l / 16.  The k-slots are mapped to
// channels identically in A (keys) and B (queries), so each output is the full
// sum over heads and channels:
//   8 heads: k-step s = channels 16s..16s+15; lane group g = heads 2g, 2g+1
//            (the two 16-B halves; adjacent in the tiled key layout).
//   4 heads: k-step s = channels 32s..32s+31; lane group g = head g.
// LDS keeps, per row tile, k-step and half, the 64 lanes' 16-byte pieces in
// lane order, so operand reads are linear (no bank conflicts).
// The output tile's lane l holds rows (positions) 4(l/16)..4(l/16)+3 of
// column (query) l % 16.
// ---------------------------------------------------------------------------
// kPass 1: block maxima of every block; 3: of the sampled block groups only,
// stored compacted (range r's sampled group j at r * sampled_groups(sub) + j);
// 2: emission, every query's candidate total added into tot[q].
// kFallback (pass 2): the checking launch after a sampled threshold.  It
// returns unless a query of the group has fewer than min(K, visible)
// candidates in tot, and emits every visible position of those queries only.
template <int H, int kPass, bool kFallback>
__global__ void __launch_bounds__(kGemmThreads) gemm_score_kernel(
    const uint8_t *__restrict__ idx_k, int64_t capacity, const uint8_t *__restrict__ q8,
    const int32_t *__restrict__ q_seq, const int32_t *__restrict__ q_pos, int32_t nq,
    const uint32_t *__restrict__ plan, uint16_t *__restrict__ bmax,
    const uint32_t *__restrict__ thr, uint2 *__restrict__ cand, int64_t cand_stride,
    uint32_t *__restrict__ cnt, int32_t nranges, uint32_t *__restrict__ tot, int32_t top_k) {
  constexpr int kGemmStage = kPass == 2 ? CSA2_GEMM_STAGE2 : CSA2_GEMM_STAGE1;
  constexpr int kPB = H * 64;                          // key bytes per position
  constexpr int kSteps = kPB / 128;                    // MFMA k-steps
  constexpr int kTileBytes = kBlk * kPB;               // one 16-row tile
  constexpr int kStageBytes = kGemmStage * kPB;
  constexpr int kPieces = kStageBytes / 16 / kGemmThreads;   // 16-B loads per thread per stage
  static_assert(kPieces >= 1 && kStageBytes % (16 * kGemmThreads) == 0, "stage shape");
  static_assert(kPass == 2 || kGemmStage * 2 == kBlk * kBlkGroup, "a block group spans two stages");
  static_assert(kPieces <= kDmaPerTile * (kGemmStage / kBlk), "the next stage's pieces fit the row tiles");

  __shared__ __attribute__((aligned(16))) uint8_t stageA[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stageB[kStageBytes];
  __shared__ int32_t s_seq[kGemmQ];
  __shared__ int32_t s_list[kGemmQ];
  __shared__ uint32_t s_scr[kGemmWaves + 1];
  __shared__ int32_t s_red[kGemmWaves];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int sub = (int)plan[0];
  const int r = blockIdx.x;
  const int qbase = blockIdx.y * kGemmQ;
  const int p_begin = r * sub;   // positions fit int32 (capacity is an int32)

  static_assert(kPass == 2 || !kFallback, "the checking form is an emission");
  static_assert(kGemmQ == kGemmThreads, "the check: one thread per query of the group");
  // a query short of candidates after the sampled threshold (the checking launch)
  auto short_of = [&](int q) -> bool {
    return (int64_t)tot[q] < min((int64_t)top_k, (int64_t)q_pos[q] + 1);
  };
  if (kFallback) {
    const int q = qbase + tid;
    if (!__syncthreads_or(q < nq && short_of(q) ? 1 : 0)) return;   // uniform
  }

  // the group's sequences and furthest visible position
  const int qt = qbase + tid;
  const int32_t my_seq = qt < nq ? q_seq[qt] : -1;
  int32_t m = qt < nq ? q_pos[qt] : -1;
  s_seq[tid] = my_seq;
  for (int d = 32; d >= 1; d >>= 1) m = max(m, __shfl_xor(m, d, kWave));
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  int32_t maxqp = s_red[0];
  for (int w = 1; w < kGemmWaves; ++w) maxqp = max(maxqp, s_red[w]);
  if (p_begin > maxqp) return;   // uniform: no query of the group sees this range
  // (pass 3: the range's first sampled_groups(sub) block groups only)
  const int p_end = min(kPass == 3 ? p_begin + sampled_groups(sub) * kRangeAlign : p_begin + sub,
                        maxqp + 1);

  bool first = qt < nq;
  for (int j = tid - 1; first && j >= 0; --j)
    if (s_seq[j] == my_seq) first = false;
  uint32_t nseq;
  const uint32_t slot = block_exclusive_scan(first ? 1u : 0u, s_scr, nseq);
  if (first) s_list[slot] = my_seq;
  __syncthreads();

  // this lane's four queries (one per column tile)
  int32_t qp[4], qs[4];
  uint32_t tq[4], run[4];
  // pass 2: each column tile's slot base (query qbase + 64 wave + 16 j, this
  // range) and the lane's slot region from it (col rows of cand_stride slots:
  // under 16 * 2^23 slots, whose byte offsets fit 32 bits)
  const uint32_t cofs = (uint32_t)(col * cand_stride);   // (a column past nq never emits)
  uint2 *tbase[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    tbase[j] = cand + (int64_t)(qbase + wave * 64 + 16 * j) * cand_stride + (int64_t)r * sub;
  v8i qb[4][kSteps];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = qbase + wave * 64 + 16 * j + col;
    const bool in = q < nq;
    const int qc = in ? q : nq - 1;
    qp[j] = in ? q_pos[q] : -1;
    // (the checking emission leaves the queries that had enough candidates
    // alone, and takes every visible position of the others)
    const bool mine = in && (!kFallback || short_of(q));
    qs[j] = mine ? q_seq[q] : -1;
    tq[j] = (kPass == 2 && in && !kFallback) ? thr[q] : 0u;
    run[j] = 0;
    const uint8_t *qrow = q8 + (int64_t)qc * kPB;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      uint4 a, b;
      if (H == 8) {
        a = *reinterpret_cast<const uint4 *>(qrow + (2 * grp) * 64 + 16 * s);
        b = *reinterpret_cast<const uint4 *>(qrow + (2 * grp + 1) * 64 + 16 * s);
      } else {
        a = *reinterpret_cast<const uint4 *>(qrow + grp * 64 + 32 * s);
        b = *reinterpret_cast<const uint4 *>(qrow + grp * 64 + 32 * s + 16);
      }
      qb[j][s] = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    }
  }

  // stage loads: piece i of a stage -> LDS offset 16 i; its key bytes are
  // (row tile rt, k-step s, half hf, lane l) of the operand layout above.
  // Piece k of thread tid is piece tid + k * kGemmThreads.
  int piece_off[kPieces];         // byte offset within the position's tile
  int piece_pos[kPieces];         // position within the stage
#pragma unroll
  for (int k = 0; k < kPieces; ++k) {
    const int i = tid + k * kGemmThreads;
    const int rt = i / (kTileBytes / 16);
    const int w = i % (kTileBytes / 16);
    const int s = w / 128, hf = (w / 64) & 1, l = w & 63;
    const int pl = rt * kBlk + (l & 15);
    const int g = l >> 4;
    const int h = H == 8 ? 2 * g + hf : g;
    const int chunk = H == 8 ? s : 2 * s + hf;
    piece_pos[k] = pl;
    piece_off[k] = chunk * 1024 + h * 16;   // plus the position's tile and slot
  }
  constexpr int T = kWave / H;   // positions per key tile
  // The keys of positions [p0, p0 + kGemmStage) (p0 a multiple of 16) are
  // contiguous bytes from p0 * kPB, and piece k of a thread sits at byte
  // k * kGemmThreads * 16 + rel0 of them: one uniform base per stage and one
  // 32-bit offset per thread.
  const uint32_t rel0 =
      (uint32_t)((piece_pos[0] / T) * 4096 + (piece_pos[0] % T) * H * 16 + piece_off[0]);
  // A piece goes from global memory straight into LDS (16 B per lane, the
  // wave's 64 pieces contiguous: lane l of wave w moves piece k*512 + 64w + l),
  // with no registers in between.  A stage running past the capacity reads
  // its last position instead.  The two stage buffers are separate LDS
  // objects so that reads of one never wait on the loads into the other; the
  // barrier that starts a stage waits for the loads into it.
  auto dma_piece = [&](const uint8_t *kb, uint8_t *dst, int p0, int k) {
    uint32_t *ldst = reinterpret_cast<uint32_t *>(dst + (k * kGemmThreads + wave * 64) * 16);
    if (p0 + kGemmStage <= capacity) {
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const uint32_t *>(kb + (int64_t)p0 * kPB + k * (kGemmThreads * 16) + rel0),
          ldst, 16, 0, 0);
    } else {
      const int p = min(p0 + piece_pos[k], (int)capacity - 1);
      const uint32_t off = (uint32_t)(p / T) * 4096u + (uint32_t)((p % T) * H * 16 + piece_off[k]);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t *>(kb + off), ldst, 16, 0, 0);
    }
  };
  for (uint32_t si = 0; si < nseq; ++si) {
    const int32_t sigma = s_list[si];
    // columns of other sequences: pass 1 never stores them, pass 2 compares
    // against +inf (no score reaches it)
    bool act[4];
    float thr_f[4];
    int32_t min_qp = INT32_MAX;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      act[j] = qs[j] == sigma;
      if (act[j]) min_qp = min(min_qp, qp[j]);
      // key >= t  <=>  score >= the float whose key is t (keys preserve order);
      // t below the key of -FLT_MAX admits everything
      const uint32_t t = tq[j];
      const float tf = t < 0x00800000u ? -INFINITY
                                       : __uint_as_float((t & 0x80000000u) ? (t & 0x7FFFFFFFu) : ~t);
      thr_f[j] = act[j] ? tf : INFINITY;
    }
    for (int d = 32; d >= 1; d >>= 1) min_qp = min(min_qp, __shfl_xor(min_qp, d, kWave));
    const bool wave_act = min_qp != INT32_MAX;
    const uint8_t *kb = idx_k + (int64_t)sigma * capacity * kPB;
    const int n_st = (p_end - p_begin + kGemmStage - 1) / kGemmStage;   // >= 1
    uint32_t sreg[kBlkGroup / 2];   // pass 1: this lane's query's block maxima, oldest lowest
    // A operand of (row tile rt, k-step s) from a staged buffer
    auto lds_a = [&](const uint8_t *cur, int rt, int s) -> v8i {
      const uint8_t *src = cur + rt * kTileBytes + (2 * s) * 1024 + lane * 16;
      const uint4 a = *reinterpret_cast<const uint4 *>(src);
      const uint4 b = *reinterpret_cast<const uint4 *>(src + 1024);
      return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    };
    // Pass 2: the rows of one tile's products that reach their column's
    // threshold, in row order, into the column's slot region.  The lane's
    // candidates of column tile j take consecutive slots, one store per
    // candidate rank (most lanes have none, a few one).
    auto emit = [&](v4f (&acc)[4], int pt) {
      const int prow = pt + 4 * grp;   // this lane's first row
      if (pt + kBlk - 1 > min_qp) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (prow + i > qp[j]) acc[j][i] = __builtin_nanf("");   // every comparison fails
      }
      uint32_t selm[4];
      uint32_t cp = 0u;   // byte j: candidates of column tile j in this lane
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        selm[j] = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) selm[j] |= (acc[j][i] >= thr_f[j] ? 1u : 0u) << i;
        cp |= (uint32_t)__popc(selm[j]) << (8 * j);
      }
      if (__ballot(cp != 0u) == 0ull) return;
      // per column tile, candidates of the lower lane groups (earlier rows)
      // and of all four, with the lane swaps described below
      const auto r16 = __builtin_amdgcn_permlane16_swap(cp, cp, false, false);
      const uint32_t pair = r16[0] + r16[1];
      const auto r32 = __builtin_amdgcn_permlane32_swap(pair, pair, false, false);
      const uint32_t tot = r32[0] + r32[1];
      const uint32_t pre = ((grp & 1) ? r16[0] : 0u) + ((grp & 2) ? r32[0] : 0u);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t off = cofs + run[j] + ((pre >> (8 * j)) & 0xFFu);
        run[j] += (tot >> (8 * j)) & 0xFFu;
        uint32_t m = selm[j];
        if (m != 0u) {
          emit_lowest(tbase[j], off, m, acc[j], prow);
          if (m != 0u) {
            emit_lowest(tbase[j], off, m, acc[j], prow);
            if (m != 0u) {
              emit_lowest(tbase[j], off, m, acc[j], prow);
              if (m != 0u) emit_lowest(tbase[j], off, m, acc[j], prow);
            }
          }
        }
      }
    };
    // The products and the pass's epilogue over one staged buffer (the
    // stage's half of a group of kBlkGroup blocks); meanwhile the next stage
    // goes into `nxt`, kDmaPerTile pieces per row tile, so that no wave stalls
    // on a burst of loads.  Pass 2 emits a tile's candidates after issuing
    // the next tile's products, so that the matrix cores work meanwhile.
    auto compute = [&](const uint8_t *cur, int p0, uint8_t *nxt, bool more, int half) {
      const int pn = p0 + kGemmStage;   // the next stage's first position
      if (!wave_act) {
        if (more) {
#pragma unroll
          for (int k = 0; k < kPieces; ++k) dma_piece(kb, nxt, pn, k);
        }
        return;
      }
      v8i an = lds_a(cur, 0, 0);   // the next k-step's A operand, read one k-step ahead
      v4f accp[4];                 // pass 2: the previous tile's products
      int ptl = p0;                // pass 2: the previous tile's first position
#pragma unroll
      for (int rt = 0; rt < kGemmStage / kBlk; ++rt) {
        const int pt = p0 + rt * kBlk;
        if (more) {
#pragma unroll
          for (int k = rt * kDmaPerTile; k < (rt + 1) * kDmaPerTile; ++k)
            if (k < kPieces) dma_piece(kb, nxt, pn, k);
        }
        if (pt >= p_end) break;
        v4f acc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
          const v8i av = an;
          if (s + 1 < kSteps) an = lds_a(cur, rt, s + 1);
          else if (rt + 1 < kGemmStage / kBlk) an = lds_a(cur, rt + 1, 0);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, qb[j][s], acc[j], 0, 0, 0,
                                                                      127, 0, 127);
        }
        if (kPass == 2) {
          if (rt > 0) emit(accp, ptl);
#pragma unroll
          for (int j = 0; j < 4; ++j) accp[j] = acc[j];
          ptl = pt;
          continue;
        }
        const int prow = pt + 4 * grp;   // this lane's first row
        // rows a column may not see hold -inf, never the block maximum of a
        // block the column sees.  Most tiles are visible to every active
        // column (and tiles never straddle a range end: ranges are multiples
        // of 16 positions).
        if (pt + kBlk - 1 > min_qp) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (prow + i > qp[j]) acc[j][i] = -INFINITY;
        }
        // block maximum in fp32 (the key order is the float order, -0 == +0);
        // E4M3 products keep every score finite, so the NaN-propagating
        // maximum (no operand canonicalization) is the maximum
        float mk[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          mk[j] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(acc[j][0], acc[j][1]),
                                                __builtin_elementwise_maximum(acc[j][2], acc[j][3]));
        // reduce over the four lane groups and scatter, lane group g ending
        // with the maximum of column tile g.  permlane32_swap(x, y) returns,
        // in lanes 0..31, (x, x of lane + 32) and in lanes 32..63 (y of
        // lane - 32, y); permlane16_swap likewise for rows of 16 lanes.
        const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mk[0]),
                                                         __float_as_uint(mk[2]), false, false);
        const auto s2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mk[1]),
                                                         __float_as_uint(mk[3]), false, false);
        const float ma = __builtin_elementwise_maximum(__uint_as_float(s1[0]), __uint_as_float(s1[1]));
        const float mb = __builtin_elementwise_maximum(__uint_as_float(s2[0]), __uint_as_float(s2[1]));
        const auto s3 = __builtin_amdgcn_permlane16_swap(__float_as_uint(ma), __float_as_uint(mb),
                                                         false, false);
        const float keep =
            __builtin_elementwise_maximum(__uint_as_float(s3[0]), __uint_as_float(s3[1]));
        const uint32_t kkey = score_key(keep);
        // kBlkGroup consecutive blocks per lane (two stages; ranges start at
        // multiples of kRangeAlign, so groups are aligned), then one 32-B
        // store; blocks past the range's end stay 0
        const int slot = half * (kGemmStage / kBlk) + rt;
        if (slot == 0) {
#pragma unroll
          for (int k = 0; k < kBlkGroup / 2; ++k) sreg[k] = 0u;
        }
        if (slot & 1) sreg[slot >> 1] |= kkey & 0xFFFF0000u;
        else sreg[slot >> 1] = kkey >> 16;
        if (slot == kBlkGroup - 1 || pt + kBlk >= p_end) {
          const int q = qbase + wave * 64 + lane;     // column tile grp, column col
          const bool own_act = grp == 0 ? act[0] : grp == 1 ? act[1] : grp == 2 ? act[2] : act[3];
          if (q < nq && own_act) {
            // the group's index (pass 3: among the sampled groups)
            const int64_t g = kPass == 3 ? (int64_t)r * sampled_groups(sub) + (pt - p_begin) / kRangeAlign
                                         : (int64_t)(pt / kBlk) / kBlkGroup;
            uint4 *dst = reinterpret_cast<uint4 *>(bmax + (g * nq + q) * kBlkGroup);
            dst[0] = make_uint4(sreg[0], sreg[1], sreg[2], sreg[3]);
            dst[1] = make_uint4(sreg[4], sreg[5], sreg[6], sreg[7]);
          }
        }
      }
      if (kPass == 2) emit(accp, ptl);   // the stage's last tile
    };
#pragma unroll
    for (int k = 0; k < kPieces; ++k) dma_piece(kb, stageA, p_begin, k);
    for (int it = 0; it < n_st; ++it) {
      const int p0 = p_begin + it * kGemmStage;
      __syncthreads();   // this stage's loads done; the other buffer no longer read
      const bool more = it + 1 < n_st;
      if ((it & 1) == 0) compute(stageA, p0, stageB, more, 0);
      else compute(stageB, p0, stageA, more, 1);
    }
    __syncthreads();   // the next sequence's first stage reuses stage A
  }
  if (kPass == 2) {
    const int q = qbase + wave * 64 + lane;
    const uint32_t own = grp == 0 ? run[0] : grp == 1 ? run[1] : grp == 2 ? run[2] : run[3];
    if (q < nq && (!kFallback || short_of(q))) cnt[(int64_t)q * nranges + r] = own;
    if (!kFallback && q < nq && own != 0u) atomicAdd(&tot[q], own);
  }
}

// thr[q] = (K-th largest 16-bit block maximum) << 16, or 0 when the query has
// fewer than K blocks.  One workgroup per query.  The K-th largest value is
// built bit by bit from the top: a bit stays set when at least K values reach
// the prefix with it set.  Each thread holds its share of the values in
// registers (kKthWords words of two values, the ones past the row's end 0,
// which no candidate prefix reaches), so a bit costs two compares per word, a
// wave sum and one barrier; rows longer than the registers hold are counted
// from global memory.
constexpr int kKthWords = 64;   // 16-bit values per thread / 2: 32768 per row
static_assert(kKthRegMax <= 2 * kKthWords * kKthThreads, "register-held rows");

__device__ __forceinline__ uint32_t kth_count_word(uint32_t w, uint32_t cand) {
  return ((w & 0xFFFFu) >= cand ? 1u : 0u) + ((w >> 16) >= cand ? 1u : 0u);
}

__device__ __forceinline__ uint32_t kth_block_sum(uint32_t c, uint32_t (*part)[kKthThreads / kWave],
                                                  int parity) {
  const int tid = threadIdx.x;
  c = __builtin_amdgcn_readlane(wave_inclusive_scan(c), kWave - 1);
  if ((tid & (kWave - 1)) == 0) part[parity][tid / kWave] = c;
  __syncthreads();   // one barrier per bit: the two part rows alternate
  uint32_t total = 0u;
#pragma unroll
  for (int w = 0; w < kKthThreads / kWave; ++w) total += part[parity][w];
  return total;
}

__global__ void __launch_bounds__(kKthThreads) gemm_kth_kernel(
    const uint16_t *__restrict__ bmax, int32_t nq, const int32_t *__restrict__ q_pos,
    int32_t top_k, uint32_t *__restrict__ thr) {
  __shared__ uint32_t part[2][kKthThreads / kWave];
  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t nblk = ((int64_t)q_pos[q] + 1 + kBlk - 1) / kBlk;
  if (nblk < top_k) {
    if (tid == 0) thr[q] = 0u;
    return;
  }
  const uint32_t k = (uint32_t)top_k;
  uint32_t prefix = 0u;
  if (nblk <= kKthRegMax) {
    // group u of thread tid: values 8 (u * kKthThreads + tid) .. +7
    const int ngroups = (int)((nblk + 8 * kKthThreads - 1) / (8 * kKthThreads));   // uniform
    uint32_t v[kKthWords];
#pragma unroll
    for (int u = 0; u < kKthWords / 4; ++u) {
      const int64_t i = 8 * ((int64_t)u * kKthThreads + tid);
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (u < ngroups && i < nblk) {
        w = *reinterpret_cast<const uint4 *>(bmax_at(bmax, nq, q, i));
        if (i + 8 > nblk) {   // the row's last group: values past its end count as 0
          uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (i + e >= nblk) ws[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
          w = make_uint4(ws[0], ws[1], ws[2], ws[3]);
        }
      }
      v[4 * u] = w.x;
      v[4 * u + 1] = w.y;
      v[4 * u + 2] = w.z;
      v[4 * u + 3] = w.w;
    }
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t cand = prefix | (1u << bit);
      uint32_t c = 0u;
#pragma unroll
      for (int u = 0; u < kKthWords / 4; ++u) {
        if (u < ngroups) {
#pragma unroll
          for (int e = 0; e < 4; ++e) c += kth_count_word(v[4 * u + e], cand);
        }
      }
      if (kth_block_sum(c, part, bit & 1) >= k) prefix = cand;
    }
  } else {
    const int64_t n8 = nblk & ~(int64_t)7;   // whole 16-byte groups; the tail is checked per value
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t cand = prefix | (1u << bit);
      uint32_t c = 0u;
      for (int64_t i = (int64_t)tid * 8; i < n8; i += kKthThreads * 8) {
        const uint4 w = *reinterpret_cast<const uint4 *>(bmax_at(bmax, nq, q, i));
        c += kth_count_word(w.x, cand) + kth_count_word(w.y, cand) + kth_count_word(w.z, cand) +
             kth_count_word(w.w, cand);
      }
      if (n8 < nblk && tid == (int)((n8 / 8) % kKthThreads)) {
        for (int64_t i = n8; i < nblk; ++i) c += *bmax_at(bmax, nq, q, i) >= cand ? 1u : 0u;
      }
      if (kth_block_sum(c, part, bit & 1) >= k) prefix = cand;
    }
  }
  if (tid == 0) thr[q] = prefix << 16;
}

// acc + [w >= cm1 + 1] per 16-bit half: a clamped packed subtract, a packed
// min with 1 and a packed add. Written out: the compiler would otherwise turn
// the pair into two compares and selects per word.
__device__ __forceinline__ uint32_t pk_count_ge(uint32_t acc, uint32_t w, uint32_t cm1,
                                                uint32_t one) {
  uint32_t t;
  asm("v_pk_sub_u16 %1, %2, %3 clamp\n\t"
      "v_pk_min_u16 %1, %1, %4\n\t"
      "v_pk_add_u16 %0, %0, %1"
      : "+v"(acc), "=&v"(t)
      : "v"(w), "v"(cm1), "v"(one));
  return acc;
}

// The same threshold with one wave per query (four queries per workgroup)
// for rows of at most kKthWaveMax block maxima: lane l holds the values
// 8 (u 64 + l) .. +7 of groups u = 0 .. kKthWaveGroups - 1 in registers (past
// the row's end: 0), and a bit costs three packed operations per word (two
// values) and a wave sum -- no barrier anywhere. Bits that the row's largest
// and smallest values share are taken from them without a pass.
// kSampled: the rows are the sampled block maxima of gemm_score_kernel<3>
// (the query's visible ones are a prefix of its row: n_s of them), and the
// threshold is their m-th largest, m the expected number of sampled blocks
// holding one of the query's K largest scores plus kSampleSigma standard
// deviations; a sample too short for that makes every visible position a
// candidate (t' = 0).  Only the groups holding the row's values are loaded.
// kGroups: register groups per lane (the row's length bound: 512 kGroups
// values); the search's work per bit grows with it.
constexpr int kKthWaveGroups = 20;
constexpr int kKthShortGroups = 4;   // sampled rows of up to 2048 values
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
constexpr int64_t kKthWaveMax = 8 * kWave * kKthWaveGroups;   // 10240 blocks: 163840 positions

template <bool kSampled, int kGroups = kKthWaveGroups>
__global__ void __launch_bounds__(256) gemm_kth_wave_kernel(
    const uint16_t *__restrict__ bmax, const int32_t *__restrict__ q_pos, int32_t nq,
    int32_t top_k, uint32_t *__restrict__ thr, const uint32_t *__restrict__ plan) {
  const int lane = threadIdx.x & (kWave - 1);
  const int q = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (q >= nq) return;   // uniform per wave
  // the host launches this kernel only for rows of at most kKthWaveMax values
  const int vis = (q_pos[q] + kBlk) / kBlk;   // visible blocks
  if (vis < top_k) {
    if (lane == 0) thr[q] = 0u;
    return;
  }
  int nblk = vis;   // values in the row
  uint32_t kk = (uint32_t)top_k;   // the rank looked for
  if (kSampled) {
    // the visible sampled blocks: every range before the query's whole, then
    // the start of its own (a prefix of the compacted row)
    const int sub = (int)plan[0];
    const int len = sampled_groups(sub) * kRangeAlign;   // sampled positions per range
    const int nvis = q_pos[q] + 1;
    const int a = nvis / sub;
    nblk = a * (len / kBlk) + (min(nvis - a * sub, len) + kBlk - 1) / kBlk;
    // a block holds one of the K largest of n scores with probability
    // 1 - (1 - K/n)^16 when they lie anywhere alike; the sample's count of such
    // blocks is about binomial
    const float p = (float)top_k / (float)(q_pos[q] + 1);
    float r = 1.0f - p;
    r *= r;
    r *= r;
    r *= r;
    r *= r;
    const float fb = 1.0f - r;
    const float mu = (float)nblk * fb;
    const float sd = sqrtf(mu * r);
    const int m = (int)ceilf(mu + kSampleSigma * sd) + 1;
    if (m > nblk) {   // every visible position a candidate (exact; the sample cannot help)
      if (lane == 0) thr[q] = 0u;
      return;
    }
    kk = (uint32_t)m;
  }
  const int ngroups = (nblk + 8 * kWave - 1) / (8 * kWave);   // uniform
  const int last8 = (nblk - 1) / 8 * 8;                       // the row's last group of 8
  uint32_t v[4 * kGroups];
  u16x2 vmax = {0, 0}, vmin = {0xFFFF, 0xFFFF};   // over the row's values only
#pragma unroll
  for (int u = 0; u < kGroups; ++u) {
    // branch-free: groups past the row read its last group and are masked
    const int i = 8 * (u * kWave + lane);
    const uint4 w = (!kSampled || u < ngroups)
                        ? *reinterpret_cast<const uint4 *>(bmax_at(bmax, nq, q, min(i, last8)))
                        : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = i + 2 * k < nblk ? 0x0000FFFFu : 0u;
      const uint32_t hi = i + 2 * k + 1 < nblk ? 0xFFFF0000u : 0u;
      v[4 * u + k] = ws[k] & (lo | hi);
      vmax = __builtin_elementwise_max(vmax, __builtin_bit_cast(u16x2, v[4 * u + k]));
      vmin = __builtin_elementwise_min(vmin, __builtin_bit_cast(u16x2, ws[k] | ~(lo | hi)));
    }
  }
  int hi_v = max((int)vmax.x, (int)vmax.y), lo_v = min((int)vmin.x, (int)vmin.y);
  for (int d = 32; d >= 1; d >>= 1) {
    hi_v = max(hi_v, __shfl_xor(hi_v, d, kWave));
    lo_v = min(lo_v, __shfl_xor(lo_v, d, kWave));
  }
  // Every value lies in [lo_v, hi_v], so the K-th largest shares the bits
  // above the highest one where the two differ: the search starts there, with
  // at least K values (all nblk of them) at or above the starting prefix.
  const uint32_t diff = (uint32_t)(hi_v ^ lo_v);
  const int top = diff ? 31 - __builtin_clz(diff) : -1;
  uint32_t prefix = (uint32_t)hi_v & ~(diff ? (2u << top) - 1u : 0u);
  const uint32_t k = kk;
  const uint32_t one = 0x00010001u;
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    // both halves at once: max(w - (cand - 1), 0) is nonzero exactly when
    // w >= cand; clamped to 1 and summed per half (at most 80 per half)
    const uint32_t cm1 = (cand - 1u) * 0x00010001u;
    uint32_t acc = 0u;
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
      if (u < ngroups) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = pk_count_ge(acc, v[4 * u + e], cm1, one);
        }
      }
    }
    const uint32_t c = (acc & 0xFFFFu) + (acc >> 16);
    const uint32_t total = __builtin_amdgcn_readlane(wave_inclusive_scan(c), kWave - 1);
    if (total >= k) prefix = cand;
  }
  if (lane == 0) thr[q] = prefix << 16;
}

// Per query: the exact Top-K among the candidates of its slot regions.  The
// first radix bin comes from the candidates themselves: every key above the
// K-th largest is a candidate, so the candidates' histogram above that bin is
// the full one.  Beyond kGemmResolveCap candidates (ties, or few blocks) the
// regions are compacted in place in global memory and streamed.
__global__ void __launch_bounds__(kGemmResolveThreads) gemm_resolve_kernel(
    const int32_t *__restrict__ q_pos, int32_t top_k, const uint32_t *__restrict__ plan,
    uint2 *__restrict__ cand, int64_t cand_stride, const uint32_t *__restrict__ cnt,
    int32_t nranges, int32_t *__restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kHistBins];
  __shared__ uint32_t scratch[kGemmResolveThreads / kWave + 1];
  __shared__ uint32_t res[4];
  __shared__ uint32_t lkey[kGemmResolveCap];
  __shared__ int32_t lid[kGemmResolveCap];
  __shared__ uint32_t goff[kGemmResolveThreads];

  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t qp = q_pos[q];
  const int64_t n_vis = (int64_t)qp + 1;
  const uint32_t keff = (uint32_t)max((int64_t)0, min((int64_t)top_k, n_vis));
  const int64_t sub = plan[0];
  const int64_t nreg = min((int64_t)nranges, (n_vis + sub - 1) / sub);
  uint2 *cq2 = cand + (int64_t)q * cand_stride;
  const uint32_t *cq = cnt + (int64_t)q * nranges;
  Emit<kOutPositions> emit{out + (int64_t)q * top_k, nullptr, qp, (uint32_t)top_k};

  // the first slots of every range are read with the counts (one round of
  // reads for the usual candidate counts)
  const uint32_t first_count = first_region_count(cq, nreg);
  const EarlySlots<kGemmEarlySlots> early =
      early_slots<kGemmEarlySlots, kGemmResolveThreads>(true, PairSlots{cq2}, nreg, sub);
  const uint32_t total =
      early.on ? gather_regions_early<kGemmResolveCap, kGemmResolveThreads>(
                     nreg, sub, PairSlots{cq2}, early, lkey, lid, goff, scratch, first_count)
               : gather_regions<kGemmResolveCap, kGemmResolveThreads>(
                     cq, nreg, sub, PairSlots{cq2}, lkey, lid, goff, scratch, first_count);
  const bool in_lds = total <= kGemmResolveCap;
  if (!in_lds) {
    // regions -> one run from slot 0 (a region's destination never passes its source)
    uint32_t dst = 0;
    for (int64_t r = 0; r < nreg; ++r) {
      const uint32_t c = (uint32_t)min((int64_t)cq[r], sub);
      for (uint32_t b = 0; b < c; b += kGemmResolveThreads) {
        const uint32_t i = b + tid;
        uint2 kv = make_uint2(0u, 0u);
        if (i < c) kv = cq2[r * sub + i];
        __syncthreads();
        if (i < c) cq2[dst + i] = kv;
        __syncthreads();
      }
      dst += c;
    }
  }
  for (int i = tid; i < kHistBins; i += kGemmResolveThreads) hist[i] = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < total; i += kGemmResolveThreads)
    atomicAdd(&hist[(in_lds ? lkey[i] : cq2[i].x) >> 20], 1u);
  __syncthreads();
  uint32_t b1 = 0, above1 = 0;
  if (keff > 0) {
    select_bin(hist, kHistBins, keff, scratch, res);
    b1 = res[0];
    above1 = res[1];
  }
  if (in_lds)
    select_core(LdsCands{lkey, lid}, (int64_t)total, keff, b1, above1, hist, scratch, res, emit);
  else
    select_core(PairSlots{cq2}, (int64_t)total, keff, b1, above1, hist, scratch, res, emit);
  int32_t *oq = out + (int64_t)q * top_k;
  for (int64_t i = (int64_t)keff + tid; i < top_k; i += kGemmResolveThreads) oq[i] = -1;
}

// Position ranges per query group: enough workgroups for the chip, a multiple
// of 8 (one XCD per range), and no more ranges than the capacity fills.
int32_t gemm_ranges(int32_t nq, int32_t capacity) {
  const int32_t groups = std::max((nq + kGemmQ - 1) / kGemmQ, 1);   // nq may be 0 in a size query
  int32_t r = (kGemmTargetGroups + groups - 1) / groups;
  r = std::max((r + 7) / 8 * 8, 8);
  return std::min(r, (capacity + kRangeAlign - 1) / kRangeAlign);
}

// pass 1, 2 or 3 (the sampled block maxima, into L.bmax_s); fallback: the
// checking form of pass 2
template <int H>
void launch_gemm_scores(const IndexArgs &a, const GemmWorkspace &L, int pass, bool fallback,
                        hipStream_t s) {
  const csa2_cache &c = *a.cache;
  uint8_t *w = a.ws;
  const dim3 grid((unsigned)L.nranges, (unsigned)((a.nq + kGemmQ - 1) / kGemmQ));
  auto args = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kGemmThreads), 0, s,
                       static_cast<const uint8_t *>(c.idx_k), (int64_t)c.capacity,
                       reinterpret_cast<const uint8_t *>(w + L.q8), a.q_seq, a.q_pos, a.nq,
                       reinterpret_cast<const uint32_t *>(w + L.plan),
                       reinterpret_cast<uint16_t *>(w + (pass == 3 ? L.bmax_s : L.bmax)),
                       reinterpret_cast<const uint32_t *>(w + L.thr),
                       reinterpret_cast<uint2 *>(w + L.cand), L.cand_stride,
                       reinterpret_cast<uint32_t *>(w + L.cnt), L.nranges,
                       reinterpret_cast<uint32_t *>(w + L.tot), a.top_k);
  };
  if (pass == 1) args(gemm_score_kernel<H, 1, false>);
  else if (pass == 2 && fallback) args(gemm_score_kernel<H, 2, true>);
  else if (pass == 2) args(gemm_score_kernel<H, 2, false>);
  else args(gemm_score_kernel<H, 3, false>);
}


}  // namespace

// The sampled first pass: rows long enough for the sample to pay (at least
// twice K blocks, ranges of at least kSampleEvery block groups), and sampled
// rows that fit one wave's threshold registers.
static bool gemm_sampled(const csa2_cache &c, int32_t top_k, const GemmWorkspace &L) {
  const int64_t blocks = ((int64_t)c.capacity + kBlk - 1) / kBlk;
  const int64_t sub_max = L.cand_stride / L.nranges;
  return blocks >= 2 * (int64_t)top_k && sub_max >= (int64_t)kSampleEvery * kRangeAlign &&
         L.bmax_s_row <= kKthWaveMax;
}

bool gemm_eligible(const csa2_cache &c, csa2_mode mode, int32_t pool_len, int32_t pool_blocks) {
  if (c.idx_k_dtype != CSA2_FP8_E4M3) return false;
  return (mode == CSA2_FULL && pool_blocks == 0) || (mode == CSA2_REINDEX && pool_len == 0);
}

GemmWorkspace gemm_workspace_layout(const csa2_cache &c, int32_t nq) {
  GemmWorkspace w;
  w.nranges = gemm_ranges(nq, c.capacity);
  const int64_t sub_max =
      (((int64_t)c.capacity + w.nranges - 1) / w.nranges + kRangeAlign - 1) / kRangeAlign * kRangeAlign;
  // one row of block maxima per query, whole 16-block groups
  w.bmax_row = ((int64_t)c.capacity + kRangeAlign - 1) / kRangeAlign * kBlkGroup;
  // the sampled block groups of every range (a range of sub <= sub_max positions)
  w.bmax_s_row = (int64_t)w.nranges * sampled_groups(sub_max) * kBlkGroup;
  w.cand_stride = sub_max * w.nranges;
  size_t off = 0;
  w.q8 = off;
  off = align256(off + (size_t)nq * c.idx_heads * 64);
  w.plan = off;
  off = align256(off + 16);
  w.thr = off;
  off = align256(off + (size_t)nq * 4);
  w.bmax = off;
  off = align256(off + (size_t)w.bmax_row * nq * 2);
  w.bmax_s = off;
  off = align256(off + (size_t)w.bmax_s_row * nq * 2);
  w.tot = off;
  off = align256(off + (size_t)nq * 4);
  w.cnt = off;
  off = align256(off + (size_t)nq * w.nranges * 4);
  w.cand = off;
  off = align256(off + (size_t)nq * w.cand_stride * 8);
  w.total = off;
  return w;
}

hipError_t launch_index_topk_gemm(const IndexArgs &a, hipEvent_t before, hipEvent_t after,
                                  hipStream_t s) {
  const csa2_cache &c = *a.cache;
  const GemmWorkspace &L = a.layout.gemm;
  uint8_t *w = a.ws;
  const int64_t n_elems = (int64_t)a.nq * c.idx_heads * 64;
  hipLaunchKernelGGL(gemm_prep_kernel, dim3((unsigned)std::max<int64_t>(1, (n_elems / 8 + 255) / 256)),
                     dim3(256), 0, s, a.q_idx, n_elems, w + L.q8, a.q_pos, a.nq, L.nranges,
                     reinterpret_cast<uint32_t *>(w + L.plan), reinterpret_cast<uint32_t *>(w + L.tot));
  if (before != nullptr) (void)hipEventRecord(before, s);
  auto pass = [&](int p, bool fallback) {
    if (c.idx_heads == 8) launch_gemm_scores<8>(a, L, p, fallback, s);
    else launch_gemm_scores<4>(a, L, p, fallback, s);
  };
  if (gemm_sampled(c, a.top_k, L)) {
    pass(3, false);
    if (L.bmax_s_row <= 8 * kWave * kKthShortGroups)   // short sampled rows: fewer registers
      hipLaunchKernelGGL((gemm_kth_wave_kernel<true, kKthShortGroups>),
                         dim3((unsigned)((a.nq + 3) / 4)), dim3(256), 0, s,
                         reinterpret_cast<const uint16_t *>(w + L.bmax_s), a.q_pos, a.nq, a.top_k,
                         reinterpret_cast<uint32_t *>(w + L.thr),
                         reinterpret_cast<const uint32_t *>(w + L.plan));
    else
      hipLaunchKernelGGL(gemm_kth_wave_kernel<true>, dim3((unsigned)((a.nq + 3) / 4)), dim3(256),
                         0, s, reinterpret_cast<const uint16_t *>(w + L.bmax_s), a.q_pos, a.nq,
                         a.top_k, reinterpret_cast<uint32_t *>(w + L.thr),
                         reinterpret_cast<const uint32_t *>(w + L.plan));
    pass(2, false);
    pass(2, true);   // the check, and the emission again for queries short of candidates
  } else {
    pass(1, false);
    if ((c.capacity + kBlk - 1) / kBlk <= kKthWaveMax)   // every row fits one wave's registers
      hipLaunchKernelGGL(gemm_kth_wave_kernel<false>, dim3((unsigned)((a.nq + 3) / 4)), dim3(256),
                         0, s, reinterpret_cast<const uint16_t *>(w + L.bmax), a.q_pos, a.nq,
                         a.top_k, reinterpret_cast<uint32_t *>(w + L.thr),
                         reinterpret_cast<const uint32_t *>(w + L.plan));
    else
      hipLaunchKernelGGL(gemm_kth_kernel, dim3((unsigned)a.nq), dim3(kKthThreads), 0, s,
                         reinterpret_cast<const uint16_t *>(w + L.bmax), a.nq, a.q_pos, a.top_k,
                         reinterpret_cast<uint32_t *>(w + L.thr));
    pass(2, false);
  }
  // the profiling events cover the product passes and the thresholds between them
  if (after != nullptr) (void)hipEventRecord(after, s);
  hipLaunchKernelGGL(gemm_resolve_kernel, dim3((unsigned)a.nq), dim3(kGemmResolveThreads), 0, s,
                     a.q_pos, a.top_k, reinterpret_cast<const uint32_t *>(w + L.plan),
                     reinterpret_cast<uint2 *>(w + L.cand), L.cand_stride,
                     reinterpret_cast<const uint32_t *>(w + L.cnt), L.nranges, a.topk_out);
  return hipGetLastError();
}

}  // namespace csa2
