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
//   zero_hist      clear the per-query radix histograms
//   score_kernel   stream the index keys (16-B coalesced loads), compute the
//                  canonical fp32 score of each candidate, store its
//                  order-preserving key, histogram the top 12 key bits in LDS
//                  (flushed with one global atomic per non-empty bin), and for
//                  a pool-building Full layer the 8-block maxima + their histogram
//   select_kernel  per query: radix-select the K-th largest key (passes on bits
//                  19..8 and 7..0 after the histogram above), then an ordered
//                  compaction that emits the winners in ascending position
//                  order, ties to the lower position, -1 padding; for the pool
//                  it emits the positions of the kept blocks.
//   reuse_copy     Reuse mode: topk_out = reuse_src.
#include <algorithm>

#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kScoreChunk = 2048;      // candidates per score workgroup (multiple of 64)
constexpr int kSelectThreads = 1024;

// ---------------------------------------------------------------------------
// cross-lane sums inside groups of 32 lanes (commutative, so every lane of a
// butterfly pair computes the same bits)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}
template <int kXor>
__device__ __forceinline__ float swz_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (kXor << 10)));
}

__global__ void zero_u32_kernel(uint32_t *__restrict__ p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += step) p[i] = 0u;
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
// Lane layout: a token's index keys (H heads x 64 channels) are split into
// H*4 lane-blocks of 16 channels; lane `sub` = 4*h + j owns head h, channels
// 16j..16j+15.  A wave covers TPI = 64 / (4H) tokens per load, so a load of
// consecutive tokens is one contiguous, coalesced span.  Each lane runs the
// canonical chain of 16 fused multiply-adds for its block; the block sums
// combine with xor-1/xor-2 butterflies ((b0+b1)+(b2+b3)), the head sums with
// xor-4/8/16 butterflies (a balanced tree over heads).
// ---------------------------------------------------------------------------
template <int H, bool kFp8Keys, bool kPool>
__global__ void __launch_bounds__(kScoreThreads) score_kernel(
    const uint8_t *__restrict__ idx_k, int64_t capacity, const uint16_t *__restrict__ q_idx,
    int32_t q_fp8, const int32_t *__restrict__ q_seq, const int32_t *__restrict__ q_pos,
    const int32_t *__restrict__ pool_in, int32_t pool_len, uint32_t *__restrict__ keys_tok,
    int64_t tok_stride, uint32_t *__restrict__ hist_tok, uint32_t *__restrict__ keys_blk,
    int64_t blk_stride, uint32_t *__restrict__ hist_blk) {
  constexpr int kEsz = kFp8Keys ? 1 : 2;
  constexpr int L = H * 4;                // lanes per token
  constexpr int TPI = kWave / L;          // tokens per wave load
  constexpr int kBpt = H * 64 * kEsz;     // bytes per token
  constexpr int kLaneBytes = 16 * kEsz;   // bytes per lane-block
  constexpr int kNumWaves = kScoreThreads / kWave;

  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t histb[kPool ? kHistBins : 1];

  const int q = blockIdx.y;
  const int32_t qp = q_pos[q];
  const int64_t n = pool_in ? (int64_t)pool_len : (int64_t)qp + 1;
  const int64_t t_begin = (int64_t)blockIdx.x * kScoreChunk;
  if (t_begin >= n) return;
  const int64_t t_end = min(n, t_begin + kScoreChunk);

  for (int i = threadIdx.x; i < kHistBins; i += kScoreThreads) {
    hist[i] = 0u;
    if (kPool) histb[i] = 0u;
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int sub = lane % L;
  const int tl = lane / L;
  const int h = sub >> 2;
  const int j = sub & 3;

  // this lane's 16 query channels, as scored (bf16, or cast to E4M3)
  float qf[16];
  {
    const uint16_t *qs = q_idx + ((int64_t)q * H + h) * 64 + j * 16;
    const uint4 a = *reinterpret_cast<const uint4 *>(qs);
    const uint4 b = *reinterpret_cast<const uint4 *>(qs + 8);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qf[2 * i] = __uint_as_float(w[i] << 16);
      qf[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    if (q_fp8) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t c = e4m3_from_f32_nonneg(fabsf(qf[i])) |
                           ((__float_as_uint(qf[i]) >> 24) & 0x80u);
        qf[i] = e4m3_to_f32(c);
      }
    }
  }

  const uint8_t *base = idx_k + (int64_t)q_seq[q] * capacity * kBpt + sub * kLaneBytes;
  __syncthreads();

  for (int64_t g = t_begin + (int64_t)wave * kWave; g < t_end; g += (int64_t)kNumWaves * kWave) {
    uint32_t mykey = 0u;
#pragma unroll 4
    for (int i = 0; i < L; ++i) {
      const int64_t t = g + (int64_t)i * TPI + tl;
      bool valid = t < t_end;
      int64_t row = t;
      if (pool_in) {
        row = valid ? (int64_t)pool_in[(int64_t)q * pool_len + t] : -1;
        valid = valid && row >= 0 && row <= qp;
      }
      float kf[16];
      if (kFp8Keys) {
        uint4 a = make_uint4(0, 0, 0, 0);
        if (valid) a = *reinterpret_cast<const uint4 *>(base + row * kBpt);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[k], false);
          auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[k], true);
          kf[4 * k + 0] = lo[0];
          kf[4 * k + 1] = lo[1];
          kf[4 * k + 2] = hi[0];
          kf[4 * k + 3] = hi[1];
        }
      } else {
        uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
        if (valid) {
          a = *reinterpret_cast<const uint4 *>(base + row * kBpt);
          b = *reinterpret_cast<const uint4 *>(base + row * kBpt + 16);
        }
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          kf[2 * k] = __uint_as_float(w[k] << 16);
          kf[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
      }
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < 16; ++c) acc = __builtin_fmaf(qf[c], kf[c], acc);
      acc = acc + dpp_xor1(acc);
      acc = acc + dpp_xor2(acc);
      acc = acc + swz_xor<4>(acc);
      acc = acc + swz_xor<8>(acc);
      if (H == 8) acc = acc + swz_xor<16>(acc);
      if (sub == i) mykey = valid ? score_key(acc) : 0u;
    }
    // lane owns token g + sub*TPI + tl; permute so that lane l holds token g + l
    const uint32_t key = (uint32_t)__shfl((int)mykey, (lane % TPI) * L + lane / TPI, kWave);
    const int64_t t = g + lane;
    if (t < t_end) {
      keys_tok[(int64_t)q * tok_stride + t] = key;
      atomicAdd(&hist[key >> 20], 1u);
    }
    if (kPool) {
      // block maximum over lanes 8b..8b+7 (keys of tokens past the end count as 0)
      uint32_t m = t < t_end ? key : 0u;
      m = max(m, shfl_xor_u(m, 1));
      m = max(m, shfl_xor_u(m, 2));
      m = max(m, shfl_xor_u(m, 4));
      if ((lane & (kPoolBlock - 1)) == 0 && t < t_end) {
        keys_blk[(int64_t)q * blk_stride + t / kPoolBlock] = m;
        atomicAdd(&histb[m >> 20], 1u);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kHistBins; i += kScoreThreads) {
    if (hist[i]) atomicAdd(&hist_tok[(int64_t)q * kHistBins + i], hist[i]);
    if (kPool && histb[i]) atomicAdd(&hist_blk[(int64_t)q * kHistBins + i], histb[i]);
  }
}

// ---------------------------------------------------------------------------
// select_kernel: one workgroup per query.
// ---------------------------------------------------------------------------
enum OutMode { kOutPositions = 0, kOutPoolIds = 1, kOutPoolBlocks = 2 };

// Finds the bin holding the element of rank `want` (1-based, counted from the
// largest key) among `nbins` LDS bins; returns the bin and the number of
// elements in higher bins.  All threads get the answer.  Contains barriers.
__device__ void select_bin(const uint32_t *bins, int nbins, uint32_t want, uint32_t *scratch,
                           uint32_t *result) {
  const int per = (nbins + kSelectThreads - 1) / kSelectThreads;  // 4 or 1
  const int lo = threadIdx.x * per;
  uint32_t s = 0;
  for (int b = lo; b < lo + per && b < nbins; ++b) s += bins[b];
  uint32_t total;
  const uint32_t excl = block_exclusive_scan(s, scratch, total);
  uint32_t above = total - excl - s;   // elements in bins of higher threads
  for (int b = lo + per - 1; b >= lo; --b) {
    if (b >= nbins) continue;
    const uint32_t c = bins[b];
    if (above < want && above + c >= want) {
      result[0] = (uint32_t)b;
      result[1] = above;
    }
    above += c;
  }
  __syncthreads();
}

template <int kMode>
__global__ void __launch_bounds__(kSelectThreads) select_kernel(
    const uint32_t *__restrict__ keys, int64_t stride, const uint32_t *__restrict__ hist_g,
    const int32_t *__restrict__ q_pos, const int32_t *__restrict__ pool_in, int32_t pool_len,
    int32_t kk, int32_t *__restrict__ out, int64_t out_stride) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t scratch[kSelectThreads / kWave + 1];
  __shared__ uint32_t res[2];

  const int q = blockIdx.x;
  const int32_t qp = q_pos[q];
  int64_t n;
  if (kMode == kOutPoolBlocks) n = ((int64_t)qp + 1 + kPoolBlock - 1) / kPoolBlock;
  else if (pool_in) n = pool_len;
  else n = (int64_t)qp + 1;
  const uint32_t *kq = keys + (int64_t)q * stride;
  int32_t *oq = out + (int64_t)q * out_stride;
  const int tid = threadIdx.x;

  for (int i = tid; i < kHistBins; i += kSelectThreads) hist[i] = hist_g[(int64_t)q * kHistBins + i];
  __syncthreads();
  const int64_t n_valid = n - (int64_t)hist[0];   // key 0 marks an empty pool slot
  const uint32_t keff = (uint32_t)min<int64_t>((int64_t)kk, n_valid);

  uint32_t tau = 0, c_gt = 0;
  if (keff > 0) {
    // pass 1 (histogram from score_kernel): bits 31..20
    select_bin(hist, kHistBins, keff, scratch, res);
    const uint32_t b1 = res[0];
    uint32_t above = res[1];
    // pass 2: bits 19..8 among keys in bin b1
    for (int i = tid; i < kHistBins; i += kSelectThreads) hist[i] = 0u;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kSelectThreads) {
      const uint32_t k = kq[i];
      if ((k >> 20) == b1) atomicAdd(&hist[(k >> 8) & 0xFFFu], 1u);
    }
    __syncthreads();
    select_bin(hist, kHistBins, keff - above, scratch, res);
    const uint32_t b2 = res[0];
    above += res[1];
    // pass 3: bits 7..0 among keys matching the top 24 bits
    const uint32_t pre24 = (b1 << 12) | b2;
    for (int i = tid; i < 256; i += kSelectThreads) hist[i] = 0u;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kSelectThreads) {
      const uint32_t k = kq[i];
      if ((k >> 8) == pre24) atomicAdd(&hist[k & 0xFFu], 1u);
    }
    __syncthreads();
    select_bin(hist, 256, keff - above, scratch, res);
    tau = (pre24 << 8) | res[0];
    c_gt = above + res[1];
  }
  // keys > tau are all taken; of the keys == tau, the first (keff - c_gt) in position order
  const uint32_t ties_wanted = keff - c_gt;

  uint32_t carry_eq = 0, carry_sel = 0;
  for (int64_t base = 0; base < n && carry_sel < keff; base += 4 * kSelectThreads) {
    const int64_t i0 = base + 4 * tid;
    uint32_t k4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) k4[u] = (i0 + u < n) ? kq[i0 + u] : 0u;
    uint32_t neq = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) neq += (k4[u] == tau && i0 + u < n && keff > 0);
    uint32_t tot_eq;
    uint32_t eq_rank = carry_eq + block_exclusive_scan(neq, scratch, tot_eq);
    bool sel[4];
    uint32_t nsel = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool in = i0 + u < n && keff > 0;
      const bool eq = in && k4[u] == tau;
      sel[u] = in && (k4[u] > tau || (eq && eq_rank < ties_wanted));
      eq_rank += eq;
      nsel += sel[u];
    }
    uint32_t tot_sel;
    uint32_t o = carry_sel + block_exclusive_scan(nsel, scratch, tot_sel);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (!sel[u]) continue;
      const int64_t id = i0 + u;
      if (kMode == kOutPositions) {
        oq[o] = (int32_t)id;
      } else if (kMode == kOutPoolIds) {
        oq[o] = pool_in[(int64_t)q * pool_len + id];
      } else {
        for (int m = 0; m < kPoolBlock; ++m) {
          const int64_t p = id * kPoolBlock + m;
          oq[(int64_t)o * kPoolBlock + m] = p <= qp ? (int32_t)p : -1;
        }
      }
      ++o;
    }
    carry_eq += tot_eq;
    carry_sel += tot_sel;
  }
  // padding
  const int64_t pad_from = (kMode == kOutPoolBlocks) ? (int64_t)keff * kPoolBlock : keff;
  const int64_t pad_to = (kMode == kOutPoolBlocks) ? (int64_t)kk * kPoolBlock : kk;
  for (int64_t i = pad_from + tid; i < pad_to; i += kSelectThreads) oq[i] = -1;
}

template <int H, bool kFp8, bool kPool>
void launch_score(const IndexArgs &a, int64_t n_cand_max, hipStream_t s) {
  const csa2_cache &c = *a.cache;
  const TopkWorkspace &L = a.layout;
  dim3 grid((unsigned)((n_cand_max + kScoreChunk - 1) / kScoreChunk), (unsigned)a.nq);
  const int32_t *pool = a.mode == CSA2_REINDEX ? a.pool_in : nullptr;
  hipLaunchKernelGGL((score_kernel<H, kFp8, kPool>), grid, dim3(kScoreThreads), 0, s,
                     static_cast<const uint8_t *>(c.idx_k), (int64_t)c.capacity, a.q_idx, a.q_fp8,
                     a.q_seq, a.q_pos, pool, a.pool_len,
                     reinterpret_cast<uint32_t *>(a.ws + L.keys_tok), L.n_tok,
                     reinterpret_cast<uint32_t *>(a.ws + L.hist_tok),
                     kPool ? reinterpret_cast<uint32_t *>(a.ws + L.keys_blk) : nullptr, L.n_blk,
                     kPool ? reinterpret_cast<uint32_t *>(a.ws + L.hist_blk) : nullptr);
}

template <int H, bool kFp8>
void launch_score_pool(const IndexArgs &a, int64_t n, bool pool, hipStream_t s) {
  if (pool) launch_score<H, kFp8, true>(a, n, s);
  else launch_score<H, kFp8, false>(a, n, s);
}

thread_local hipEvent_t g_scan_before = nullptr;
thread_local hipEvent_t g_scan_after = nullptr;

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
  w.n_tok = ((reindex_pool ? (int64_t)pool_len : (int64_t)c.capacity) + 63) / 64 * 64;
  const bool pool = mode == CSA2_FULL && pool_blocks > 0;
  w.n_blk = pool ? (((int64_t)c.capacity + kPoolBlock - 1) / kPoolBlock + 63) / 64 * 64 : 0;
  size_t off = 0;
  w.keys_tok = off;
  off = align256(off + (size_t)nq * w.n_tok * 4);
  w.hist_tok = off;
  off = align256(off + (size_t)nq * kHistBins * 4);
  if (pool) {
    w.keys_blk = off;
    off = align256(off + (size_t)nq * w.n_blk * 4);
    w.hist_blk = off;
    off = align256(off + (size_t)nq * kHistBins * 4);
  }
  w.total = off;
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
  const TopkWorkspace &L = a.layout;
  const bool pool = a.mode == CSA2_FULL && a.pool_blocks > 0;
  const bool reindex_pool = a.mode == CSA2_REINDEX && a.pool_in != nullptr;
  // 1. clear histograms (hist_tok and, with a pool, hist_blk which follows keys_blk)
  {
    const int64_t n = (int64_t)a.nq * kHistBins;
    const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 2048);
    hipLaunchKernelGGL(zero_u32_kernel, dim3(blocks), dim3(256), 0, s,
                       reinterpret_cast<uint32_t *>(a.ws + L.hist_tok), n);
    if (pool)
      hipLaunchKernelGGL(zero_u32_kernel, dim3(blocks), dim3(256), 0, s,
                         reinterpret_cast<uint32_t *>(a.ws + L.hist_blk), n);
  }
  // 2. scores
  if (g_scan_before != nullptr) (void)hipEventRecord(g_scan_before, s);
  const int64_t n_cand = reindex_pool ? (int64_t)a.pool_len : (int64_t)c.capacity;
  const bool fp8 = c.idx_k_dtype == CSA2_FP8_E4M3;
  if (c.idx_heads == 8) {
    if (fp8) launch_score_pool<8, true>(a, n_cand, pool, s);
    else launch_score_pool<8, false>(a, n_cand, pool, s);
  } else {
    if (fp8) launch_score_pool<4, true>(a, n_cand, pool, s);
    else launch_score_pool<4, false>(a, n_cand, pool, s);
  }
  if (g_scan_after != nullptr) (void)hipEventRecord(g_scan_after, s);
  // 3. select
  const uint32_t *keys_tok = reinterpret_cast<const uint32_t *>(a.ws + L.keys_tok);
  const uint32_t *hist_tok = reinterpret_cast<const uint32_t *>(a.ws + L.hist_tok);
  if (reindex_pool)
    hipLaunchKernelGGL((select_kernel<kOutPoolIds>), dim3(a.nq), dim3(kSelectThreads), 0, s,
                       keys_tok, L.n_tok, hist_tok, a.q_pos, a.pool_in, a.pool_len, a.top_k,
                       a.topk_out, (int64_t)a.top_k);
  else
    hipLaunchKernelGGL((select_kernel<kOutPositions>), dim3(a.nq), dim3(kSelectThreads), 0, s,
                       keys_tok, L.n_tok, hist_tok, a.q_pos, nullptr, 0, a.top_k, a.topk_out,
                       (int64_t)a.top_k);
  if (pool)
    hipLaunchKernelGGL((select_kernel<kOutPoolBlocks>), dim3(a.nq), dim3(kSelectThreads), 0, s,
                       reinterpret_cast<const uint32_t *>(a.ws + L.keys_blk), L.n_blk,
                       reinterpret_cast<const uint32_t *>(a.ws + L.hist_blk), a.q_pos, nullptr,
                       0, a.pool_blocks, a.pool_out, (int64_t)a.pool_blocks * kPoolBlock);
  return hipGetLastError();
}

}  // namespace csa2
