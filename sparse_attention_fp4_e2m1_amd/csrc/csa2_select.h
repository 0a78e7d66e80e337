// Exact Top-K selection on order-preserving score keys, shared by the
// streaming scorer and the matrix-core scorer (device code, one workgroup of
// kSelectThreads threads per query).
//
// Ordering rule (aiwiki "DeepSeek V4.1-Flash", section "Compressed Sparse
// Attention 2", per-query Top-K): the K largest scores, ties to the lower
// index, emitted in ascending index order.
#pragma once

#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kSelectThreads = 1024;
constexpr int kResolveCap = 8192;          // candidates held in LDS by a resolve
// Per query, a selection's global histogram region holds `copies` copies of
// the 12-bit histogram of the keys' top bits (the scorer's workgroups spread
// their atomics over them; readers add them up), kStateWords of state (keff,
// b1, above, second histogram valid), then the histogram of bits 19..8 of the
// keys in the threshold bin (filled by the filter when it runs).
constexpr int kStateWords = 16;
__host__ __device__ constexpr int64_t hist_stride(int copies) {
  return (int64_t)(copies + 1) * kHistBins + kStateWords;
}
__host__ __device__ constexpr int64_t state_off(int copies) { return (int64_t)copies * kHistBins; }
__host__ __device__ constexpr int64_t h2_off(int copies) {
  return (int64_t)copies * kHistBins + kStateWords;
}

// ---------------------------------------------------------------------------
// Selection helpers
// ---------------------------------------------------------------------------
enum OutMode { kOutPositions = 0, kOutPoolIds = 1, kOutPoolBlocks = 2 };

// Per wave: the bin of the 256 LDS bins `h` holding the element of rank `want`
// (1-based from the top) -> {bin, elements in higher bins}, seen by every lane.
__device__ __forceinline__ uint2 wave_select_bin256(const uint32_t *h, uint32_t want) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t c[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) c[b] = h[4 * lane + b];
  const uint32_t sum = c[0] + c[1] + c[2] + c[3];
  const uint32_t incl = wave_inclusive_scan(sum);
  const uint32_t total = (uint32_t)__shfl((int)incl, kWave - 1, kWave);
  uint32_t above = total - incl;   // elements in the bins of higher lanes
  uint32_t found = 0xFFFFFFFFu, found_above = 0u;
#pragma unroll
  for (int b = 3; b >= 0; --b) {
    if (above < want && above + c[b] >= want) {
      found = 4 * lane + b;
      found_above = above;
    }
    above += c[b];
  }
  const uint64_t who = __ballot(found != 0xFFFFFFFFu);
  const int src = who ? __ffsll((unsigned long long)who) - 1 : 0;
  return make_uint2((uint32_t)__shfl((int)found, src, kWave),
                    (uint32_t)__shfl((int)found_above, src, kWave));
}

// Finds the bin holding the element of rank `want` (1-based, counted from the
// largest key) among `nbins` LDS bins; result = {bin, elements in higher bins}.
// All threads of the block take part and see the result.  Contains barriers.
// 4096 bins (with at least 256 threads): sums of 16 bins by 256 threads, one
// wave picks the 16-bin group and then the bin in it.  256 bins: one wave.
__device__ void select_bin(const uint32_t *bins, int nbins, uint32_t want, uint32_t *scratch,
                           uint32_t *result) {
  const int nt = blockDim.x;
  const int tid = threadIdx.x;
  if (nbins == 4096 && nt >= 256) {
    __shared__ uint32_t coarse[256];
    if (tid < 256) {
      const uint4 *p = reinterpret_cast<const uint4 *>(bins + 16 * tid);
      uint32_t s = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 v = p[k];
        s += v.x + v.y + v.z + v.w;
      }
      coarse[tid] = s;
    }
    __syncthreads();
    if (tid < kWave) {
      const uint2 cb = wave_select_bin256(coarse, want);
      const uint32_t v = tid < 16 ? bins[16 * cb.x + tid] : 0u;
      const uint32_t inc = wave_inclusive_scan(v);
      const uint32_t tot16 = (uint32_t)__shfl((int)inc, 15, kWave);
      const uint32_t above = cb.y + tot16 - inc;   // elements in the group's higher bins and above
      const bool hit = tid < 16 && above < want && above + v >= want;
      const uint64_t who = __ballot(hit);
      const int f = who ? __ffsll((unsigned long long)who) - 1 : 0;
      const uint32_t fa = (uint32_t)__shfl((int)above, f, kWave);
      if (tid == 0 && who) {
        result[0] = 16 * cb.x + (uint32_t)f;
        result[1] = fa;
      }
    }
    __syncthreads();
    return;
  }
  if (nbins == 256) {
    if (tid < kWave) {
      const uint2 r = wave_select_bin256(bins, want);
      if (tid == 0) {
        result[0] = r.x;
        result[1] = r.y;
      }
    }
    __syncthreads();
    return;
  }
  const int per = (nbins + nt - 1) / nt;
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

// ---------------------------------------------------------------------------
// Selection proper
// ---------------------------------------------------------------------------
struct GlobalKeys {   // keys[i], index i
  const uint32_t *k;
  __device__ uint32_t key(int64_t i) const { return k[i]; }
  __device__ int64_t id(int64_t i) const { return i; }
};

struct LdsCands {     // candidates gathered in index order
  const uint32_t *k;
  const int32_t *ids;
  __device__ uint32_t key(int64_t i) const { return k[i]; }
  __device__ int64_t id(int64_t i) const { return ids[i]; }
};

// An emitter turns a selected candidate into output entries in two steps:
// value(id) (for pool ids the pool lookup, a global load, issued before the
// compaction's scans so that its latency overlaps them), then store(o, v).
template <int kMode>
struct Emit {
  int32_t *out;          // this query's output row
  const int32_t *pool;   // this query's pool row (kOutPoolIds)
  int32_t qp;
  uint32_t limit;        // entries in the row (a guard: o < keff <= limit by construction)
  __device__ int64_t value(int64_t id) const { return kMode == kOutPoolIds ? (int64_t)pool[id] : id; }
  __device__ void store(uint32_t o, int64_t v) const {
    if (o >= limit) return;
    if (kMode == kOutPoolBlocks) {
      for (int m = 0; m < kPoolBlock; ++m) {
        const int64_t p = v * kPoolBlock + m;
        out[(int64_t)o * kPoolBlock + m] = p <= qp ? (int32_t)p : -1;
      }
    } else {
      out[o] = (int32_t)v;
    }
  }
};

// Emitter whose output kind (OutMode) is chosen at run time.
struct EmitAny {
  int mode;
  int32_t *out;
  const int32_t *pool;
  int32_t qp;
  uint32_t limit;        // entries (blocks) in the row; o < keff <= limit by construction
  __device__ int64_t value(int64_t id) const {
    return mode == kOutPoolIds ? (int64_t)pool[id] : id;
  }
  __device__ void store(uint32_t o, int64_t v) const {
    if (o >= limit) return;
    if (mode == kOutPoolBlocks) {
      for (int m = 0; m < kPoolBlock; ++m) {
        const int64_t p = v * kPoolBlock + m;
        out[(int64_t)o * kPoolBlock + m] = p <= qp ? (int32_t)p : -1;
      }
    } else {
      out[o] = (int32_t)v;
    }
  }
};

__device__ __forceinline__ int64_t sel_len(int mode, int32_t qp, int32_t pool_len) {
  if (mode == kOutPoolBlocks) return ((int64_t)qp + 1 + kPoolBlock - 1) / kPoolBlock;
  if (mode == kOutPoolIds) return pool_len;
  return (int64_t)qp + 1;
}

// First radix pass of one query from its 12-bit histogram (global): keff =
// min(kk, keys present), b1 = the bin of the keff-th largest key, above = keys
// in higher bins.  Key 0 marks an empty pool slot (no score maps there).  The
// whole block takes part; `lh` holds kHistBins words of LDS.  Contains barriers.
struct Threshold {
  uint32_t keff, b1, above;
};

// The same from a histogram already in LDS (all threads, barriers).
__device__ Threshold lds_threshold(int64_t n, int32_t kk, uint32_t *lh, uint32_t *scratch,
                                   uint32_t *res) {
  Threshold t;
  t.keff = (uint32_t)max((int64_t)0, min((int64_t)kk, n - (int64_t)lh[0]));
  t.b1 = 0u;
  t.above = 0u;
  if (t.keff > 0) {
    select_bin(lh, kHistBins, t.keff, scratch, res);
    t.b1 = res[0];
    t.above = res[1];
  }
  __syncthreads();   // res and lh free again
  return t;
}

__device__ Threshold hist_threshold(const uint32_t *__restrict__ hq, int copies, int64_t n,
                                    int32_t kk, uint32_t *lh, uint32_t *scratch, uint32_t *res) {
  for (int i = threadIdx.x; i < kHistBins / 4; i += blockDim.x) {
    uint4 v = reinterpret_cast<const uint4 *>(hq)[i];
    for (int c = 1; c < copies; ++c) {
      const uint4 w = reinterpret_cast<const uint4 *>(hq + (int64_t)c * kHistBins)[i];
      v.x += w.x;
      v.y += w.y;
      v.z += w.z;
      v.w += w.w;
    }
    reinterpret_cast<uint4 *>(lh)[i] = v;
  }
  __syncthreads();
  return lds_threshold(n, kk, lh, scratch, res);
}

// The K-th largest key tau and the selection: keys > tau, then the first ties
// == tau in index order, emitted in index order.  One block; `hist` has
// kHistBins words of LDS, `res` 4.  tau comes from radix passes on bits 19..8
// and 7..0 among the keys of bin b1 (above1 keys lie in higher bins).  The
// ordered compaction takes 4 consecutive keys per thread per tile; when every
// tie is selected (the usual case) one block scan per tile suffices.
// Known result of the bits 19..8 pass (from a histogram built elsewhere).
struct Pass19 {
  bool known;
  uint32_t pre24, above;   // top 24 bits of tau, keys above that 24-bit bin
};

template <class Src, class E>
__device__ void select_core(const Src &src, int64_t n, uint32_t keff, uint32_t b1,
                            uint32_t above1, uint32_t *hist, uint32_t *scratch, uint32_t *res,
                            const E &emit, Pass19 p19 = Pass19{false, 0u, 0u}) {
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  uint32_t tau = 0, c_gt = 0, n_tau = 0;
  if (keff > 0) {
    uint32_t above = above1;
    uint32_t pre24;
    if (p19.known) {
      pre24 = p19.pre24;
      above = p19.above;
    } else {
      for (int i = tid; i < kHistBins; i += nt) hist[i] = 0u;
      __syncthreads();
      for (int64_t i = tid; i < n; i += nt) {                // bits 19..8 within bin b1
        const uint32_t k = src.key(i);
        if ((k >> 20) == b1) atomicAdd(&hist[(k >> 8) & 0xFFFu], 1u);
      }
      __syncthreads();
      select_bin(hist, kHistBins, keff - above, scratch, res);
      pre24 = (b1 << 12) | res[0];
      above += res[1];
    }
    for (int i = tid; i < 256; i += nt) hist[i] = 0u;
    __syncthreads();
    for (int64_t i = tid; i < n; i += nt) {                  // bits 7..0
      const uint32_t k = src.key(i);
      if ((k >> 8) == pre24) atomicAdd(&hist[k & 0xFFu], 1u);
    }
    __syncthreads();
    select_bin(hist, 256, keff - above, scratch, res);
    tau = (pre24 << 8) | res[0];
    c_gt = above + res[1];
    n_tau = hist[res[0]];   // every key equal to tau
  }
  const uint32_t ties_wanted = keff - c_gt;
  const bool all_ties = ties_wanted == n_tau;
  // ordered compaction, 4 consecutive keys per thread per tile
  uint32_t carry_eq = 0, carry_sel = 0;
  for (int64_t base = 0; base < n && carry_sel < keff; base += 4 * (int64_t)nt) {
    const int64_t i0 = base + 4 * tid;
    uint32_t k4[4];
    bool in4[4];
    int64_t v4[4];   // output values, loaded before the scans
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      in4[u] = i0 + u < n;
      k4[u] = in4[u] ? src.key(i0 + u) : 0u;
      v4[u] = in4[u] ? emit.value(src.id(i0 + u)) : 0;
    }
    bool sel[4];
    uint32_t nsel = 0;
    if (all_ties) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sel[u] = in4[u] && k4[u] >= tau;
        nsel += sel[u];
      }
    } else {
      uint32_t neq = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) neq += (in4[u] && k4[u] == tau);
      uint32_t tot_eq;
      uint32_t eq_rank = carry_eq + block_exclusive_scan(neq, scratch, tot_eq);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool eq = in4[u] && k4[u] == tau;
        sel[u] = in4[u] && (k4[u] > tau || (eq && eq_rank < ties_wanted));
        eq_rank += eq;
        nsel += sel[u];
      }
      carry_eq += tot_eq;
    }
    uint32_t tot_sel;
    uint32_t o = carry_sel + block_exclusive_scan(nsel, scratch, tot_sel);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (sel[u]) emit.store(o++, v4[u]);
    carry_sel += tot_sel;
  }
}

// Candidate slots as two arrays (key, index).
struct SplitSlots {
  const uint32_t *k;
  const int32_t *ids;
  __device__ uint32_t key(int64_t i) const { return k[i]; }
  __device__ int64_t id(int64_t i) const { return ids[i]; }
};

// Candidate slots as one array of (key, index) pairs.
struct PairSlots {
  const uint2 *kv;
  __device__ uint32_t key(int64_t i) const { return kv[i].x; }
  __device__ int64_t id(int64_t i) const { return (int32_t)kv[i].y; }
};

// Copies one query's candidates, held in `nreg` slot regions of `region`
// entries each (counts in cq, region r at slots r * region of `slots`), into
// LDS in region order when they fit (<= kCap); returns the total either
// way.  Slot offsets come from a block scan; every thread then finds the
// region of each slot it copies by binary search over the offsets.  Contains
// barriers.
// first_count: this thread's count of the first group (region tid), loaded by
// the caller early so that its latency overlaps other work.
__device__ __forceinline__ uint32_t first_region_count(const uint32_t *cq, int64_t nreg) {
  return (int64_t)threadIdx.x < nreg ? cq[threadIdx.x] : 0u;
}

template <int kCap = kResolveCap, int kThreads = kSelectThreads, class Slots>
__device__ uint32_t gather_regions(const uint32_t *cq, int64_t nreg, int64_t region,
                                   const Slots &slots, uint32_t *lkey, int32_t *lid,
                                   uint32_t *goff, uint32_t *scratch, uint32_t first_count) {
  const int tid = threadIdx.x;
  uint32_t carry = 0;
  for (int64_t c0 = 0; c0 < nreg; c0 += kThreads) {
    const int64_t c = c0 + tid;
    const uint32_t raw = c0 == 0 ? first_count : (c < nreg ? cq[c] : 0u);
    // a region never holds more than `region` slots; the clamp keeps every
    // read inside the query's slots whatever the counts say
    const uint32_t mine = c < nreg ? (uint32_t)min((int64_t)raw, region) : 0u;
    uint32_t tot;
    const uint32_t off = carry + block_exclusive_scan(mine, scratch, tot);
    goff[tid] = off;
    __syncthreads();
    if (carry + tot <= kCap) {
      const int group = (int)min((int64_t)kThreads, nreg - c0);
      for (uint32_t j = carry + tid; j < carry + tot; j += kThreads) {
        int lo = 0, hi = group - 1;           // last region with goff <= j
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (goff[mid] <= j) lo = mid; else hi = mid - 1;
        }
        const int64_t src = (c0 + lo) * region + (j - goff[lo]);
        lkey[j] = slots.key(src);
        lid[j] = (int32_t)slots.id(src);
      }
    }
    carry += tot;
    __syncthreads();
  }
  return carry;
}


// Reads of the first slots of every region issued before the region counts
// are known (with the counts and the histogram), so that for the usual
// candidate counts the copy into LDS needs no second dependent round trip.
// Entry u of a thread (e = tid + u * kThreads) reads slot e % S of region
// e / S, S = 2^shift the largest power of two with nreg * S <= kSpec * kThreads
// and S <= region.  Only for one group of regions (nreg <= kThreads) whose
// slot total fits 21 bits (the overflow flags of gather_regions_early ride
// above them in one scan).
template <int kSpec>
struct EarlySlots {
  uint32_t key[kSpec];
  int32_t id[kSpec];
  uint32_t shift;
  bool on;
};

template <int kSpec, int kThreads, class Slots>
__device__ __forceinline__ EarlySlots<kSpec> early_slots(bool enable, const Slots &slots,
                                                         int64_t nreg, int64_t region) {
  EarlySlots<kSpec> e;
  e.shift = 0;
  e.on = enable && nreg > 0 && nreg <= kThreads && nreg * region < (1 << 21);
  if (!e.on) return e;   // uniform
  while ((nreg << (e.shift + 1)) <= (int64_t)kSpec * kThreads &&
         ((int64_t)1 << (e.shift + 1)) <= region)
    ++e.shift;
  const int64_t mask = ((int64_t)1 << e.shift) - 1;
#pragma unroll
  for (int u = 0; u < kSpec; ++u) {
    const int64_t ent = (int64_t)threadIdx.x + (int64_t)u * kThreads;
    // past the last region the read is clamped into it and later ignored
    const int64_t r = min(ent >> e.shift, nreg - 1);
    const int64_t src = r * region + (ent & mask);
    e.key[u] = slots.key(src);
    e.id[u] = (int32_t)slots.id(src);
  }
  return e;
}

// gather_regions for a group of regions read early by early_slots (e.on):
// the early slots go to LDS straight from registers; only regions holding
// more than S candidates send a second round of reads.  Contains barriers.
template <int kCap, int kThreads, int kSpec, class Slots>
__device__ uint32_t gather_regions_early(int64_t nreg, int64_t region, const Slots &slots,
                                         const EarlySlots<kSpec> &e, uint32_t *lkey,
                                         int32_t *lid, uint32_t *goff, uint32_t *scratch,
                                         uint32_t first_count) {
  constexpr uint32_t kLow = (1u << 21) - 1u;
  const int tid = threadIdx.x;
  const uint32_t S = 1u << e.shift;
  const uint32_t mine = tid < nreg ? (uint32_t)min((int64_t)first_count, region) : 0u;
  uint32_t tot_packed;
  const uint32_t off =
      block_exclusive_scan(mine | ((mine > S ? 1u : 0u) << 21), scratch, tot_packed) & kLow;
  const uint32_t tot = tot_packed & kLow;
  const bool more = (tot_packed >> 21) != 0u;
  goff[tid] = off;
  __syncthreads();
  if (tot <= kCap) {
#pragma unroll
    for (int u = 0; u < kSpec; ++u) {
      const uint32_t ent = (uint32_t)tid + (uint32_t)u * kThreads;
      const uint32_t r = ent >> e.shift;
      const uint32_t j = ent & (S - 1u);
      if (r < (uint32_t)nreg) {
        const uint32_t end = r + 1 < (uint32_t)nreg ? goff[r + 1] : tot;
        if (goff[r] + j < end) {
          lkey[goff[r] + j] = e.key[u];
          lid[goff[r] + j] = e.id[u];
        }
      }
    }
    if (more) {
      for (uint32_t j = tid; j < tot; j += kThreads) {
        int lo = 0, hi = (int)nreg - 1;           // last region with goff <= j
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (goff[mid] <= j) lo = mid; else hi = mid - 1;
        }
        const uint32_t k = j - goff[lo];
        if (k >= S) {
          const int64_t src = (int64_t)lo * region + k;
          lkey[j] = slots.key(src);
          lid[j] = (int32_t)slots.id(src);
        }
      }
    }
  }
  __syncthreads();
  return tot;
}

}  // namespace
}  // namespace csa2
