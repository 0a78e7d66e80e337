// Internal launchers of the CSA2 library (host side), one translation unit each.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa2.h"
#include "csa2_device.h"

namespace csa2 {

constexpr int kHistBins = 4096;      // first radix pass: top 12 bits of the score key
// Where a selection's 12-bit histogram comes from:
//   kHistKeys    the resolve counts the keys itself (a Reindex pool: its scorer
//                builds no histogram);
//   kHistGlobal  the scorer's workgroups add theirs into the query's global
//                histogram copies (cleared by a launch before the scorer);
//   kRanked      no histogram as such: each scorer workgroup stores its
//                chunk's keys ordered by 12-bit bin, highest bin first, with
//                their positions and, per bin, the count of the chunk's keys
//                in that bin or above; ranked_select_kernel reads the
//                threshold bin off those counts and then only the keys at or
//                above it (nothing to clear: every chunk record a selection
//                reads is written by the same call).
enum HistSource { kHistKeys = 0, kHistGlobal = 1, kRanked = 2 };
constexpr int kPoolBlock = 8;        // positions per candidate-pool block

hipError_t launch_kv_append(const csa2_cache &c, const uint16_t *k, const uint16_t *v,
                            const uint16_t *idx_in, const int32_t *seq, const int32_t *pos,
                            int32_t n, hipStream_t stream);

// Workspace carve-up of csa2_index_topk (byte offsets, 256-B aligned).
struct SelectArrays {      // one selection problem per query (tokens, or pool blocks)
  size_t keys = 0;         // uint32 [nq][n]      order-preserving score keys
  size_t hist = 0;         // uint32 [nq][hstride]  histogram copies, state words, second histogram
  size_t cand_key = 0;     // uint32 [nq][cand_stride] filter output, one slot region per wave
  size_t cand_id = 0;      // int32  [nq][cand_stride]
  size_t cnt = 0;          // uint32 [nq][nsub]   candidates per slot region
  int64_t n = 0;           // key slots per query
  int64_t cand_stride = 0;
  int64_t nsub = 0;
  int32_t region = 0;      // keys per filter wave (slots per region)
  int32_t hcopies = 1;     // copies of the 12-bit histogram (scorer workgroups spread over them)
  int64_t hstride = 0;     // words per query: hcopies histograms, state words, second histogram
  int32_t hsrc = 0;        // HistSource: where the resolve finds the 12-bit histogram
  // ranked chunks (kRanked): the keys array holds each chunk's keys in bin order
  size_t rk_pos = 0;       // uint16 [nq][n]  chunk-local position of each ranked key
  size_t rk_ge = 0;        // uint16 [nq][nchunks][kHistBins]  keys in bin b or above, per chunk
  size_t rk_coarse = 0;    // uint16 [nq][nchunks][kHistBins / 64]  every 64th entry of rk_ge
  int32_t nchunks = 0;     // scorer chunks per query
  int32_t chunk = 0;       // candidates per scorer chunk
};

// Workspace carve-up of the matrix-core scorer (E4M3 index queries and keys).
struct GemmWorkspace {
  size_t q8 = 0;           // uint8  [nq][idx_heads * 64]   E4M3 index queries
  size_t plan = 0;         // uint32 [1]  positions per range
  size_t thr = 0;          // uint32 [nq] candidate threshold key
  size_t bmax = 0;         // uint16 [bmax_row / 16][nq][16]  block maxima of 16 positions (top 16 key bits), group-major
  size_t bmax_s = 0;       // uint16 [bmax_s_row / 16][nq][16]  the sampled block groups' maxima, compacted
  size_t tot = 0;          // uint32 [nq]  candidates pass 2 emitted for the query (all ranges)
  size_t cnt = 0;          // uint32 [nq][nranges]  candidates per (query, range)
  size_t cand = 0;         // uint2  [nq][cand_stride]  (score key, position)
  int64_t bmax_row = 0;
  int64_t bmax_s_row = 0;
  int64_t cand_stride = 0;
  int32_t nranges = 0;
  size_t total = 0;
};

struct TopkWorkspace {
  SelectArrays tok;        // candidate positions (or pool entries)
  SelectArrays blk;        // pool blocks (Full layer with a pool), else n = 0
  GemmWorkspace gemm;      // the matrix-core scorer's arrays, when it can run
  size_t total = 0;        // covers either scorer
};

TopkWorkspace topk_workspace_layout(const csa2_cache &c, csa2_mode mode, int32_t nq,
                                    int32_t pool_len, int32_t pool_blocks);

// The rows of one append call (csa2_kv_append's arguments).
struct AppendRows {
  uint8_t *kv_codes;
  uint8_t *kv_scales;
  void *idx_k;
  const uint16_t *k, *v, *idx_in;   // idx_in may be null: index keys untouched
  const int32_t *seq, *pos;
  int32_t n;
  int32_t capacity;
  int32_t idx_elems;                // index heads x 64
  int32_t idx_fp8;
};
AppendRows append_rows(const csa2_cache &c, const uint16_t *k, const uint16_t *v,
                       const uint16_t *idx_in, const int32_t *seq, const int32_t *pos, int32_t n);
// Appended rows the scorer takes in one launch at most (more run on their own).
constexpr int32_t kFuseMaxRows = 256;

struct IndexArgs {
  const csa2_cache *cache;
  csa2_mode mode;
  const uint16_t *q_idx;
  int32_t q_fp8;
  const int32_t *q_seq;
  const int32_t *q_pos;
  int32_t nq;
  int32_t top_k;
  const int32_t *pool_in;
  int32_t pool_len;
  int32_t pool_blocks;
  int32_t *pool_out;
  const int32_t *reuse_src;
  int32_t *topk_out;
  uint8_t *ws;
  TopkWorkspace layout;
  AppendRows ap;           // rows to append first (ap.n = 0: none)
};

hipError_t launch_index_topk(const IndexArgs &a, hipStream_t stream);

// The matrix-core scorer serves E4M3 index queries against E4M3 keys when the
// candidates are every visible position (FULL without a pool, REINDEX without one).
bool gemm_eligible(const csa2_cache &c, csa2_mode mode, int32_t pool_len, int32_t pool_blocks);
GemmWorkspace gemm_workspace_layout(const csa2_cache &c, int32_t nq);
hipError_t launch_index_topk_gemm(const IndexArgs &a, hipEvent_t before, hipEvent_t after,
                                  hipStream_t stream);

// Events recorded around the scoring kernel (csa2_profile_index_scan); per host thread.
void set_index_scan_events(hipEvent_t before, hipEvent_t after);

struct AttnWorkspace {
  size_t part_acc = 0;     // float [nq][splits][heads][dv]
  size_t part_ml = 0;      // float2 [nq][splits][heads]  (max, sum) of exp2-scaled scores
  size_t total = 0;
  int32_t splits = 0;         // splits of the selected rows
  int32_t local_splits = 0;   // splits of the window rows (fused call)
};

AttnWorkspace attn_workspace_layout(const csa2_cache &c, int32_t nq, int32_t n_heads,
                                    int32_t top_k, int32_t window = 0);

hipError_t launch_sparse_attn(const csa2_cache &c, const uint16_t *q, int32_t n_heads,
                              const int32_t *q_seq, int32_t nq, const int32_t *topk,
                              int32_t top_k, float softmax_scale, float *out, float *lse,
                              uint8_t *ws, const AttnWorkspace &layout, hipStream_t stream,
                              const csa2_local_cache *lc = nullptr,
                              const int32_t *q_pos = nullptr);

// The allocation-free attention call: its split partials in a static device
// array of this many bytes (per device), reached through noalloc_scratch,
// which returns the current device's address of the array (looked up once per
// device).
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;
hipError_t noalloc_scratch(uint8_t **ptr);

hipError_t launch_proj_append(const csa2_cache &c, const uint16_t *x, int32_t d_model,
                              const uint16_t *w, const int32_t *seq, const int32_t *pos,
                              int32_t n, hipStream_t stream);
hipError_t launch_local_clear(const csa2_local_cache &c, int32_t seq, hipStream_t stream);
hipError_t launch_local_append(const csa2_local_cache &c, const uint16_t *k, const uint16_t *v,
                               const int32_t *seq, const int32_t *pos, int32_t n,
                               hipStream_t stream);
hipError_t launch_local_attn(const csa2_local_cache &c, const uint16_t *q, int32_t n_heads,
                             const int32_t *q_seq, const int32_t *q_pos, int32_t nq,
                             float softmax_scale, float *out, float *lse, hipStream_t stream);
constexpr int32_t kMaxLocalWindow = 1024;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace csa2
