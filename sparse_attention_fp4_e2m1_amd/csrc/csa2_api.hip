// C ABI of the CSA2 library: host-side validation, workspace sizing, dispatch.
// Every check runs before anything is enqueued, so a rejected call leaves the
// device untouched.
#include <cstring>

#include "csa2_internal.h"

using namespace csa2;

namespace {

// The integer a caller passed for an enum parameter.  A C caller may pass any
// int, and reading a value outside the enumerators' range through the C++
// enum type is undefined, so the bits are copied out, unread as the enum, and
// validated as an int.
template <class E>
int32_t raw_enum(const E &e) {
  static_assert(sizeof(E) == sizeof(int32_t), "int-sized enum");
  int32_t v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

// Largest capacity: the kernels address a sequence's rows and index-key tiles
// with 32-bit byte offsets (a tile of positions p is (p / T) * 64 * 64 * E
// bytes in, which reaches 2^32 at p = 2^23).
constexpr int32_t kMaxCapacity = 1 << 23;

csa2_status check_cache(const csa2_cache *c, bool need_idx) {
  if (c == nullptr || c->kv_codes == nullptr || c->kv_scales == nullptr) return CSA2_ERR_NULL;
  if (need_idx && c->idx_k == nullptr) return CSA2_ERR_NULL;
  if (c->batch < 1 || c->capacity < 1 || c->capacity % 16 != 0) return CSA2_ERR_SHAPE;
  if (c->capacity > kMaxCapacity) return CSA2_ERR_SHAPE;
  if (c->dk != 128 || c->dv != 128 || c->idx_dim != 64) return CSA2_ERR_UNSUPPORTED;
  if (c->idx_heads != 4 && c->idx_heads != 8) return CSA2_ERR_UNSUPPORTED;
  if (c->idx_k_dtype != CSA2_BF16 && c->idx_k_dtype != CSA2_FP8_E4M3) return CSA2_ERR_UNSUPPORTED;
  return CSA2_OK;
}

constexpr int32_t kMaxTopK = 1 << 16;

csa2_status check_local(const csa2_local_cache *c) {
  if (c == nullptr || c->k == nullptr || c->v == nullptr || c->pos == nullptr) return CSA2_ERR_NULL;
  if (c->batch < 1 || c->window < 1 || c->window > kMaxLocalWindow) return CSA2_ERR_SHAPE;
  if (c->dk != 128 || c->dv != 128) return CSA2_ERR_UNSUPPORTED;
  return CSA2_OK;
}

csa2_status check_topk_args(const csa2_cache *cache, int32_t mode, int32_t nq, int32_t top_k,
                            int32_t pool_len, int32_t pool_blocks) {
  csa2_status st = check_cache(cache, mode != CSA2_REUSE);
  if (st != CSA2_OK) return st;
  if (mode != CSA2_FULL && mode != CSA2_REINDEX && mode != CSA2_REUSE) return CSA2_ERR_ARG;
  if (nq < 0 || top_k < 1 || top_k > kMaxTopK) return CSA2_ERR_SHAPE;
  if (pool_len < 0 || pool_blocks < 0 || pool_blocks > kMaxTopK) return CSA2_ERR_SHAPE;
  if (mode != CSA2_FULL && pool_blocks != 0) return CSA2_ERR_ARG;
  if (mode != CSA2_REINDEX && pool_len != 0) return CSA2_ERR_ARG;
  if (nq > 65535) return CSA2_ERR_SHAPE;   // one grid row per query
  return CSA2_OK;
}

}  // namespace

extern "C" {

const char *csa2_strerror(csa2_status status) {
  switch (raw_enum(status)) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_NULL: return "a required pointer is NULL";
    case CSA2_ERR_SHAPE: return "a size is out of range";
    case CSA2_ERR_UNSUPPORTED: return "unsupported dimension or dtype";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA2_ERR_HIP: return "HIP launch error";
    case CSA2_ERR_ARG: return "inconsistent arguments";
  }
  return "unknown status";
}

int csa2_abi_version(void) { return CSA2_ABI_VERSION; }

void csa2_profile_index_scan(void *before, void *after) {
  set_index_scan_events(static_cast<hipEvent_t>(before), static_cast<hipEvent_t>(after));
}

csa2_status csa2_kv_append(const csa2_cache *cache, const uint16_t *k, const uint16_t *v,
                           const uint16_t *idx_k_in, const int32_t *seq, const int32_t *pos,
                           int32_t n, void *stream) {
  csa2_status st = check_cache(cache, idx_k_in != nullptr);
  if (st != CSA2_OK) return st;
  if (n < 0) return CSA2_ERR_SHAPE;
  if (n == 0) return CSA2_OK;
  if (k == nullptr || v == nullptr || seq == nullptr || pos == nullptr) return CSA2_ERR_NULL;
  if (launch_kv_append(*cache, k, v, idx_k_in, seq, pos, n, (hipStream_t)stream) != hipSuccess)
    return CSA2_ERR_HIP;
  return CSA2_OK;
}

size_t csa2_index_topk_workspace(const csa2_cache *cache, csa2_mode mode_arg, int32_t nq,
                                 int32_t top_k, int32_t pool_len, int32_t pool_blocks) {
  const int32_t mode = raw_enum(mode_arg);
  if (check_topk_args(cache, mode, nq, top_k, pool_len, pool_blocks) != CSA2_OK) return 0;
  return topk_workspace_layout(*cache, static_cast<csa2_mode>(mode), nq, pool_len, pool_blocks).total;
}

}  // extern "C"

namespace {

// csa2_index_topk with rows to append first (ap.n = 0: none).
// (mode and q_dtype as the caller's raw values: an out-of-range one is an
// error, not an enum load)
csa2_status index_topk(const csa2_cache *cache, int32_t mode, const uint16_t *q_idx,
                       int32_t q_dtype, const int32_t *q_seq, const int32_t *q_pos,
                       int32_t nq, int32_t top_k, const int32_t *pool_in, int32_t pool_len,
                       int32_t pool_blocks, int32_t *pool_out, const int32_t *reuse_src,
                       int32_t *topk_out, void *workspace, size_t workspace_bytes, void *stream,
                       const AppendRows &ap) {
  csa2_status st = check_topk_args(cache, mode, nq, top_k, pool_len, pool_blocks);
  if (st != CSA2_OK) return st;
  if (nq == 0) {   // no queries: the pointers of the index call may be NULL
    if (ap.n > 0 && launch_kv_append(*cache, ap.k, ap.v, ap.idx_in, ap.seq, ap.pos, ap.n,
                                     (hipStream_t)stream) != hipSuccess)
      return CSA2_ERR_HIP;
    return CSA2_OK;
  }
  if (topk_out == nullptr) return CSA2_ERR_NULL;
  if (mode == CSA2_REUSE) {
    if (reuse_src == nullptr) return CSA2_ERR_ARG;
    if (pool_in != nullptr || pool_out != nullptr) return CSA2_ERR_ARG;
  } else {
    if (q_idx == nullptr || q_seq == nullptr || q_pos == nullptr) return CSA2_ERR_NULL;
    if (q_dtype != CSA2_BF16 && q_dtype != CSA2_FP8_E4M3) return CSA2_ERR_UNSUPPORTED;
    if (reuse_src != nullptr) return CSA2_ERR_ARG;
    if (mode == CSA2_FULL && pool_in != nullptr) return CSA2_ERR_ARG;
    if (mode == CSA2_FULL && pool_blocks > 0 && pool_out == nullptr) return CSA2_ERR_ARG;
    if (mode == CSA2_FULL && pool_blocks == 0 && pool_out != nullptr) return CSA2_ERR_ARG;
    if (mode == CSA2_REINDEX) {
      if (pool_out != nullptr) return CSA2_ERR_ARG;
      if ((pool_in == nullptr) != (pool_len == 0)) return CSA2_ERR_ARG;
    }
  }
  IndexArgs a;
  a.cache = cache;
  a.mode = static_cast<csa2_mode>(mode);
  a.q_idx = q_idx;
  a.q_fp8 = q_dtype == CSA2_FP8_E4M3;
  a.q_seq = q_seq;
  a.q_pos = q_pos;
  a.nq = nq;
  a.top_k = top_k;
  a.pool_in = pool_in;
  a.pool_len = pool_len;
  a.pool_blocks = pool_blocks;
  a.pool_out = pool_out;
  a.reuse_src = reuse_src;
  a.topk_out = topk_out;
  a.layout = topk_workspace_layout(*cache, a.mode, nq, pool_len, pool_blocks);
  if (a.layout.total > 0 && (workspace == nullptr || workspace_bytes < a.layout.total))
    return CSA2_ERR_WORKSPACE;
  a.ws = static_cast<uint8_t *>(workspace);
  a.ap = ap;
  if (launch_index_topk(a, (hipStream_t)stream) != hipSuccess) return CSA2_ERR_HIP;
  return CSA2_OK;
}

}  // namespace

extern "C" {

csa2_status csa2_index_topk(const csa2_cache *cache, csa2_mode mode, const uint16_t *q_idx,
                            csa2_dtype q_dtype, const int32_t *q_seq, const int32_t *q_pos,
                            int32_t nq, int32_t top_k, const int32_t *pool_in, int32_t pool_len,
                            int32_t pool_blocks, int32_t *pool_out, const int32_t *reuse_src,
                            int32_t *topk_out, void *workspace, size_t workspace_bytes,
                            void *stream) {
  AppendRows none{};
  none.n = 0;
  return index_topk(cache, raw_enum(mode), q_idx, raw_enum(q_dtype), q_seq, q_pos, nq, top_k,
                    pool_in, pool_len, pool_blocks, pool_out, reuse_src, topk_out, workspace,
                    workspace_bytes, stream, none);
}

csa2_status csa2_index_topk_append(const csa2_cache *cache, const uint16_t *k, const uint16_t *v,
                                   const uint16_t *idx_k_in, const int32_t *a_seq,
                                   const int32_t *a_pos, int32_t n_append, csa2_mode mode,
                                   const uint16_t *q_idx, csa2_dtype q_dtype,
                                   const int32_t *q_seq, const int32_t *q_pos, int32_t nq,
                                   int32_t top_k, const int32_t *pool_in, int32_t pool_len,
                                   int32_t pool_blocks, int32_t *pool_out,
                                   const int32_t *reuse_src, int32_t *topk_out, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  // the append's own checks first (csa2_kv_append's), then the index call's
  csa2_status st = check_cache(cache, idx_k_in != nullptr);
  if (st != CSA2_OK) return st;
  if (n_append < 0) return CSA2_ERR_SHAPE;
  if (n_append > 0 && (k == nullptr || v == nullptr || a_seq == nullptr || a_pos == nullptr))
    return CSA2_ERR_NULL;
  AppendRows ap = append_rows(*cache, k, v, idx_k_in, a_seq, a_pos, n_append);
  return index_topk(cache, raw_enum(mode), q_idx, raw_enum(q_dtype), q_seq, q_pos, nq, top_k,
                    pool_in, pool_len, pool_blocks, pool_out, reuse_src, topk_out, workspace,
                    workspace_bytes, stream, ap);
}

size_t csa2_sparse_attn_workspace(const csa2_cache *cache, int32_t nq, int32_t n_heads,
                                  int32_t top_k) {
  if (check_cache(cache, false) != CSA2_OK) return 0;
  if (nq < 0 || n_heads < 16 || n_heads > 128 || n_heads % 16 != 0) return 0;
  if (top_k < 1 || top_k > kMaxTopK) return 0;
  return attn_workspace_layout(*cache, nq, n_heads, top_k).total;
}

csa2_status csa2_sparse_attn(const csa2_cache *cache, const uint16_t *q, int32_t n_heads,
                             const int32_t *q_seq, int32_t nq, const int32_t *topk, int32_t top_k,
                             float softmax_scale, float *out, float *lse, void *workspace,
                             size_t workspace_bytes, void *stream) {
  csa2_status st = check_cache(cache, false);
  if (st != CSA2_OK) return st;
  if (n_heads < 16 || n_heads > 128 || n_heads % 16 != 0) return CSA2_ERR_UNSUPPORTED;
  if (nq < 0 || top_k < 1 || top_k > kMaxTopK || nq > 65535) return CSA2_ERR_SHAPE;
  if (nq == 0) return CSA2_OK;
  if (q == nullptr || q_seq == nullptr || topk == nullptr || out == nullptr) return CSA2_ERR_NULL;
  const AttnWorkspace L = attn_workspace_layout(*cache, nq, n_heads, top_k);
  if (workspace == nullptr || workspace_bytes < L.total) return CSA2_ERR_WORKSPACE;
  if (launch_sparse_attn(*cache, q, n_heads, q_seq, nq, topk, top_k, softmax_scale, out, lse,
                         static_cast<uint8_t *>(workspace), L, (hipStream_t)stream) != hipSuccess)
    return CSA2_ERR_HIP;
  return CSA2_OK;
}

csa2_status csa2_sparse_attn_noalloc(const csa2_cache *cache, const uint16_t *q, int32_t n_heads,
                                     const int32_t *q_seq, int32_t nq, const int32_t *topk,
                                     int32_t top_k, float softmax_scale, float *out, float *lse,
                                     void *stream) {
  csa2_status st = check_cache(cache, false);
  if (st != CSA2_OK) return st;
  if (n_heads < 16 || n_heads > 128 || n_heads % 16 != 0) return CSA2_ERR_UNSUPPORTED;
  if (nq < 0 || top_k < 1 || top_k > kMaxTopK || nq > 65535) return CSA2_ERR_SHAPE;
  if (nq == 0) return CSA2_OK;
  if (q == nullptr || q_seq == nullptr || topk == nullptr || out == nullptr) return CSA2_ERR_NULL;
  const AttnWorkspace L = attn_workspace_layout(*cache, nq, n_heads, top_k);
  if (L.total > kNoallocScratchBytes) return CSA2_ERR_WORKSPACE;
  uint8_t *ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return CSA2_ERR_HIP;
  if (launch_sparse_attn(*cache, q, n_heads, q_seq, nq, topk, top_k, softmax_scale, out, lse, ws,
                         L, (hipStream_t)stream) != hipSuccess)
    return CSA2_ERR_HIP;
  return CSA2_OK;
}

size_t csa2_sparse_local_attn_workspace(const csa2_cache *cache, const csa2_local_cache *local,
                                        int32_t nq, int32_t n_heads, int32_t top_k) {
  if (check_cache(cache, false) != CSA2_OK || check_local(local) != CSA2_OK) return 0;
  if (nq < 0 || n_heads < 16 || n_heads > 128 || n_heads % 16 != 0) return 0;
  if (top_k < 1 || top_k > kMaxTopK) return 0;
  return attn_workspace_layout(*cache, nq, n_heads, top_k, local->window).total;
}

csa2_status csa2_sparse_local_attn(const csa2_cache *cache, const csa2_local_cache *local,
                                   const uint16_t *q, int32_t n_heads, const int32_t *q_seq,
                                   const int32_t *q_pos, int32_t nq, const int32_t *topk,
                                   int32_t top_k, float softmax_scale, float *out, float *lse,
                                   void *workspace, size_t workspace_bytes, void *stream) {
  csa2_status st = check_cache(cache, false);
  if (st != CSA2_OK) return st;
  if ((st = check_local(local)) != CSA2_OK) return st;
  if (local->batch < cache->batch) return CSA2_ERR_SHAPE;
  if (n_heads < 16 || n_heads > 128 || n_heads % 16 != 0) return CSA2_ERR_UNSUPPORTED;
  if (nq < 0 || top_k < 1 || top_k > kMaxTopK || nq > 65535) return CSA2_ERR_SHAPE;
  if (nq == 0) return CSA2_OK;
  if (q == nullptr || q_seq == nullptr || q_pos == nullptr || topk == nullptr || out == nullptr)
    return CSA2_ERR_NULL;
  const AttnWorkspace L = attn_workspace_layout(*cache, nq, n_heads, top_k, local->window);
  if (workspace == nullptr || workspace_bytes < L.total) return CSA2_ERR_WORKSPACE;
  if (launch_sparse_attn(*cache, q, n_heads, q_seq, nq, topk, top_k, softmax_scale, out, lse,
                         static_cast<uint8_t *>(workspace), L, (hipStream_t)stream, local,
                         q_pos) != hipSuccess)
    return CSA2_ERR_HIP;
  return CSA2_OK;
}

csa2_status csa2_local_append(const csa2_local_cache *cache, const uint16_t *k, const uint16_t *v,
                              const int32_t *seq, const int32_t *pos, int32_t n, void *stream) {
  csa2_status st = check_local(cache);
  if (st != CSA2_OK) return st;
  if (n < 0) return CSA2_ERR_SHAPE;
  if (n == 0) return CSA2_OK;
  if (k == nullptr || v == nullptr || seq == nullptr || pos == nullptr) return CSA2_ERR_NULL;
  if (launch_local_append(*cache, k, v, seq, pos, n, (hipStream_t)stream) != hipSuccess)
    return CSA2_ERR_HIP;
  return CSA2_OK;
}

csa2_status csa2_local_attn(const csa2_local_cache *cache, const uint16_t *q, int32_t n_heads,
                            const int32_t *q_seq, const int32_t *q_pos, int32_t nq,
                            float softmax_scale, float *out, float *lse, void *stream) {
  csa2_status st = check_local(cache);
  if (st != CSA2_OK) return st;
  if (n_heads < 16 || n_heads > 128 || n_heads % 16 != 0) return CSA2_ERR_UNSUPPORTED;
  if (nq < 0 || nq > 65535) return CSA2_ERR_SHAPE;
  if (nq == 0) return CSA2_OK;
  if (q == nullptr || q_seq == nullptr || q_pos == nullptr || out == nullptr || lse == nullptr)
    return CSA2_ERR_NULL;
  if (launch_local_attn(*cache, q, n_heads, q_seq, q_pos, nq, softmax_scale, out, lse,
                        (hipStream_t)stream) != hipSuccess)
    return CSA2_ERR_HIP;
  return CSA2_OK;
}

namespace {

struct KvImage {
  size_t codes, scales, idx, total;   // section sizes in bytes
};

KvImage kv_image(const csa2_cache &c, int32_t len) {
  const size_t esz = c.idx_k_dtype == CSA2_FP8_E4M3 ? 1 : 2;
  const int32_t per_tile = 64 / c.idx_heads;
  KvImage im;
  im.codes = (size_t)len * 128;
  im.scales = (size_t)len * 16;
  im.idx = (size_t)((len + per_tile - 1) / per_tile) * 64 * 64 * esz;
  im.total = im.codes + im.scales + im.idx;
  return im;
}

csa2_status check_image_args(const csa2_cache *c, int32_t seq, int32_t len, const void *buf,
                             size_t bytes) {
  csa2_status st = check_cache(c, true);
  if (st != CSA2_OK) return st;
  if (seq < 0 || seq >= c->batch || len < 0 || len > c->capacity) return CSA2_ERR_SHAPE;
  if (len == 0) return CSA2_OK;
  if (buf == nullptr) return CSA2_ERR_NULL;
  if (bytes < kv_image(*c, len).total) return CSA2_ERR_WORKSPACE;
  return CSA2_OK;
}

// The three sections of one sequence's prefix, as (device address, bytes).
void kv_sections(const csa2_cache &c, int32_t seq, int32_t len, uint8_t *dev[3], size_t n[3]) {
  const KvImage im = kv_image(c, len);
  const size_t esz = c.idx_k_dtype == CSA2_FP8_E4M3 ? 1 : 2;
  dev[0] = c.kv_codes + (size_t)seq * c.capacity * 128;
  dev[1] = c.kv_scales + (size_t)seq * c.capacity * 16;
  dev[2] = static_cast<uint8_t *>(c.idx_k) + (size_t)seq * c.capacity * c.idx_heads * 64 * esz;
  n[0] = im.codes;
  n[1] = im.scales;
  n[2] = im.idx;
}

}  // namespace

size_t csa2_kv_export_bytes(const csa2_cache *cache, int32_t len) {
  if (check_cache(cache, true) != CSA2_OK || len < 0 || len > cache->capacity) return 0;
  return kv_image(*cache, len).total;
}

csa2_status csa2_kv_export(const csa2_cache *cache, int32_t seq, int32_t len, void *dst,
                           size_t dst_bytes, void *stream) {
  csa2_status st = check_image_args(cache, seq, len, dst, dst_bytes);
  if (st != CSA2_OK || len == 0) return st;
  uint8_t *dev[3];
  size_t n[3];
  kv_sections(*cache, seq, len, dev, n);
  uint8_t *out = static_cast<uint8_t *>(dst);
  for (int i = 0; i < 3; ++i) {
    if (hipMemcpyAsync(out, dev[i], n[i], hipMemcpyDefault, (hipStream_t)stream) != hipSuccess)
      return CSA2_ERR_HIP;
    out += n[i];
  }
  return CSA2_OK;
}

csa2_status csa2_kv_import(const csa2_cache *cache, int32_t seq, int32_t len, const void *src,
                           size_t src_bytes, void *stream) {
  csa2_status st = check_image_args(cache, seq, len, src, src_bytes);
  if (st != CSA2_OK || len == 0) return st;
  uint8_t *dev[3];
  size_t n[3];
  kv_sections(*cache, seq, len, dev, n);
  const uint8_t *in = static_cast<const uint8_t *>(src);
  for (int i = 0; i < 3; ++i) {
    if (hipMemcpyAsync(dev[i], in, n[i], hipMemcpyDefault, (hipStream_t)stream) != hipSuccess)
      return CSA2_ERR_HIP;
    in += n[i];
  }
  return CSA2_OK;
}

csa2_status csa2_proj_append(const csa2_cache *cache, const uint16_t *x, int32_t d_model,
                             const uint16_t *w, const int32_t *seq, const int32_t *pos, int32_t n,
                             void *stream) {
  csa2_status st = check_cache(cache, true);
  if (st != CSA2_OK) return st;
  if (n < 0 || d_model < 32 || d_model > 65536 || d_model % 32 != 0) return CSA2_ERR_SHAPE;
  if (n == 0) return CSA2_OK;
  if (x == nullptr || w == nullptr || seq == nullptr || pos == nullptr) return CSA2_ERR_NULL;
  if ((n + 63) / 64 > 0x7FFFFFFF) return CSA2_ERR_SHAPE;
  if (launch_proj_append(*cache, x, d_model, w, seq, pos, n, (hipStream_t)stream) != hipSuccess)
    return CSA2_ERR_HIP;
  return CSA2_OK;
}

csa2_status csa2_local_clear(const csa2_local_cache *cache, int32_t seq, void *stream) {
  csa2_status st = check_local(cache);
  if (st != CSA2_OK) return st;
  if (seq < 0 || seq >= cache->batch) return CSA2_ERR_SHAPE;
  if (launch_local_clear(*cache, seq, (hipStream_t)stream) != hipSuccess) return CSA2_ERR_HIP;
  return CSA2_OK;
}

}  // extern "C"
