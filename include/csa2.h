/*
 * csa2.h -- C ABI of the CSA2 hot path on MI355X (gfx950).
 *
 * Compressed Sparse Attention 2 (CSA2) as the pages state the problem:
 *   - model card "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
 *     Compression", Introduction, CSA2 paragraph: per-layer static modes Full,
 *     Reindex and Reuse that share main KV and indexer keys across layers and
 *     recycle Top-K sparse-attention indices; a Hierarchical Sparse Indexer in
 *     the decoder restricting later indexers to a candidate pool built by the
 *     first Full layer; main KV cached in FP4 (E2M1 values, one E4M3 scale per
 *     16 channels);
 *   - aiwiki "DeepSeek V4.1-Flash", section "Compressed Sparse Attention 2":
 *     what each mode computes and reuses; the pool of 8-position blocks ranked
 *     by their maximum index score; section "KV-cache formats and bounded
 *     replay": the main global KV lives in accelerator memory in FP4.
 *
 * Three calls make one layer's step: csa2_kv_append (quantize-and-append new
 * rows), csa2_index_topk (index scoring + Top-K in a mode, optionally building
 * the pool), csa2_sparse_attn (gather + dequantize the selected rows and run
 * softmax attention of every query head over them).
 *
 * Conventions for every call:
 *   - All array arguments are DEVICE pointers (hipMalloc'd or torch-owned),
 *     except the csa2_cache descriptor itself, which is a host struct.
 *   - The library never allocates, frees or synchronizes.  Work is enqueued on
 *     `stream` (a hipStream_t; NULL = the null stream) and returns at once.
 *   - Scalars and pointers are validated on the host before anything is
 *     enqueued; a failed check returns an error and enqueues nothing.
 *     Launch failures return CSA2_ERR_HIP.  Device-side preconditions (listed
 *     per call) are not checked.
 *   - Calls are reentrant; concurrent calls must not share a workspace.
 *   - Finite inputs only: NaN or infinite inputs give unspecified results.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 1

typedef enum {
  CSA2_OK = 0,
  CSA2_ERR_NULL = 1,         /* a required pointer is NULL */
  CSA2_ERR_SHAPE = 2,        /* a size is out of range */
  CSA2_ERR_UNSUPPORTED = 3,  /* a dimension or dtype the library does not implement */
  CSA2_ERR_WORKSPACE = 4,    /* workspace missing or smaller than the query function returns */
  CSA2_ERR_HIP = 5,          /* a HIP launch reported an error */
  CSA2_ERR_ARG = 6           /* inconsistent arguments (e.g. mode vs. pool/reuse pointers) */
} csa2_status;

/* Layer modes (aiwiki, "Compressed Sparse Attention 2"). */
typedef enum {
  CSA2_FULL = 0,     /* score every causally visible position; fresh Top-K; may build the pool */
  CSA2_REINDEX = 1,  /* new index query over earlier index keys; search the pool (or all visible) */
  CSA2_REUSE = 2     /* recycle an earlier layer's Top-K unchanged */
} csa2_mode;

typedef enum {
  CSA2_BF16 = 0,
  CSA2_FP8_E4M3 = 1  /* OCP E4M3FN: bias 7, max 448, 0x7F/0xFF NaN, no infinities */
} csa2_dtype;

/*
 * The shared global cache of one layer group: FP4 main KV plus index keys.
 * Caller-owned device memory; byte layout (part of the ABI):
 *   kv_codes  [batch][capacity][dk/2 + dv/2] bytes.  Bytes 0..dk/2-1 hold the
 *             K codes, then the V codes.  Channel 2i is the low nibble of byte
 *             i, channel 2i+1 the high nibble.  A code is E2M1 (bit 3 sign,
 *             magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6).
 *   kv_scales [batch][capacity][dk/16 + dv/16] bytes, E4M3 codes: the scale
 *             of K channels 16b..16b+15 at byte b, then the V scales.
 *   idx_k     index keys, bf16 bits or E4M3 codes (idx_k_dtype), idx_heads x
 *             idx_dim per position, stored TILED so that the index scan reads
 *             every 1 KB span with one coalesced wave load and each lane gets
 *             one head of one position.  With E = bytes per element (1 or 2),
 *             T = 64 / idx_heads positions per tile and C = 4 * E chunks of
 *             16 bytes per head, element (position p, head h, channel c) of
 *             sequence s lives at byte
 *               s * capacity * idx_heads * idx_dim * E
 *               + (p / T) * (64 * 64 * E)                  -- tile
 *               + ((c * E) / 16) * 1024                    -- chunk
 *               + ((p % T) * idx_heads + h) * 16           -- lane slot
 *               + (c * E) % 16                             -- byte in chunk.
 *             (For 8 heads of E4M3: tiles of 8 positions, 4 KB each.)
 * One cached position = dk/2 + dv/2 + dk/16 + dv/16 bytes of main KV
 * (144 B for dk = dv = 128) plus idx_heads * idx_dim * (1 or 2) bytes.
 * Supported: dk = dv = 128, idx_dim = 64, idx_heads in {4, 8}; capacity a
 * multiple of 16, at most 8388608 (2^23) positions per sequence (the kernels
 * use 32-bit byte offsets within a sequence); a larger capacity is rejected
 * with CSA2_ERR_SHAPE by every call that takes the cache.
 */
typedef struct csa2_cache {
  uint8_t *kv_codes;
  uint8_t *kv_scales;
  void *idx_k;
  int32_t batch;
  int32_t capacity;
  int32_t dk;
  int32_t dv;
  int32_t idx_heads;
  int32_t idx_dim;
  int32_t idx_k_dtype; /* csa2_dtype */
} csa2_cache;

/*
 * Quantize-and-append n new rows (model card, Introduction, CSA2 paragraph:
 * FP4 main KV, E2M1 values with one E4M3 scale per 16 channels).
 *   k, v       [n][dk], [n][dv] bf16 bits: the new main K and V rows.
 *   idx_k_in   [n][idx_heads][idx_dim] bf16 bits, or NULL to leave the index
 *              keys untouched.  Stored verbatim (bf16 cache) or cast to E4M3
 *              (round to nearest even, saturating at +-448, sign kept).
 *   seq, pos   [n] int32: row r goes to sequence seq[r], position pos[r].
 * Per 16-channel block: scale = E4M3 nearest amax/6 (ties to even,
 * saturating at 448); each element = E2M1 nearest x/scale (ties to even,
 * saturating at 6, sign kept; a zero scale gives magnitude 0).
 * Device preconditions: 0 <= seq[r] < batch, 0 <= pos[r] < capacity; no two
 * rows of one call share (seq, pos).
 * Errors: CSA2_ERR_NULL, CSA2_ERR_SHAPE (n < 0), CSA2_ERR_UNSUPPORTED, CSA2_ERR_HIP.
 * n = 0 is a no-op returning CSA2_OK.
 */
csa2_status csa2_kv_append(const csa2_cache *cache, const uint16_t *k, const uint16_t *v,
                           const uint16_t *idx_k_in, const int32_t *seq, const int32_t *pos,
                           int32_t n, void *stream);

/*
 * Bytes of workspace csa2_index_topk needs for these arguments (0 for REUSE).
 * Returns 0 as well when the arguments are invalid; csa2_index_topk then
 * reports the error.
 */
size_t csa2_index_topk_workspace(const csa2_cache *cache, csa2_mode mode, int32_t nq, int32_t top_k,
                                 int32_t pool_len, int32_t pool_blocks);

/*
 * Index scoring and per-query Top-K (aiwiki, "Compressed Sparse Attention 2").
 *   q_idx      [nq][idx_heads][idx_dim] bf16 bits: each query's index query.
 *   q_dtype    precision the index query is scored in: CSA2_BF16 as given, or
 *              CSA2_FP8_E4M3 (cast with round to nearest even, saturating).
 *   q_seq      [nq] int32 sequence of each query.
 *   q_pos      [nq] int32 position of each query; it sees rows [0, q_pos].
 *   top_k      entries per query in topk_out (1 .. 65536).
 *   FULL:      candidates are positions 0..q_pos.  If pool_blocks > 0, also
 *              builds the candidate pool: blocks [8b, 8b+8) ranked by their
 *              maximum score (ties to the lower block), the top pool_blocks
 *              blocks kept; pool_out [nq][8*pool_blocks] receives their visible
 *              positions in ascending order, -1 padded.
 *   REINDEX:   candidates are the entries of pool_in [nq][pool_len] that lie
 *              in [0, q_pos] (-1 = empty slot), a row's positions in ascending
 *              order (as pool_out lists them); pool_in = NULL means all visible
 *              positions (as FULL, no pool).  Entries must be distinct.
 *   REUSE:     topk_out = reuse_src [nq][top_k], copied unchanged; q_idx,
 *              q_seq, q_pos may be NULL.
 * Score of candidate j: sum over indexer heads h of q_h . k_{j,h}, in fp32 in
 * the plain left-to-right order: per head one chain of fused multiply-adds
 * over channels 0 .. idx_dim-1 starting from 0, then the head sums added from
 * head 0 up.  The result is bit-reproducible.
 * Matrix-core scoring: with q_dtype = CSA2_FP8_E4M3 against E4M3 keys and
 * every visible position a candidate (FULL without a pool, REINDEX without
 * pool_in), all queries of the call are scored as one dense E4M3 product on
 * matrix cores.  Each product is exact; the fp32 sums follow the hardware's
 * order (deterministic, but not the order above), so a Top-K may differ from
 * the fixed-order one only among candidates whose exact scores lie within
 * fp32 rounding of the K-th score.  Queries are grouped 512 at a time in
 * index order; a group whose queries share one sequence (a prefill chunk)
 * runs at full rate, a group spanning several sequences makes one pass per
 * sequence.
 * topk_out [nq][top_k] int32: the min(top_k, #candidates) candidates with the
 * largest scores (ties to the lower position, -0 == +0), in ascending
 * position order, then -1 padding.
 * Device preconditions: 0 <= q_seq < batch, 0 <= q_pos < capacity.
 * Errors: CSA2_ERR_NULL, CSA2_ERR_SHAPE, CSA2_ERR_UNSUPPORTED, CSA2_ERR_ARG
 * (pool_out missing with pool_blocks > 0, pool arguments in the wrong mode,
 * reuse_src missing in REUSE), CSA2_ERR_WORKSPACE, CSA2_ERR_HIP.
 * nq = 0 is a no-op returning CSA2_OK (after the checks of mode, top_k and
 * the pool sizes); the query, list, pool and workspace pointers may then be
 * NULL.
 */
csa2_status csa2_index_topk(const csa2_cache *cache, csa2_mode mode, const uint16_t *q_idx,
                            csa2_dtype q_dtype, const int32_t *q_seq, const int32_t *q_pos,
                            int32_t nq, int32_t top_k, const int32_t *pool_in, int32_t pool_len,
                            int32_t pool_blocks, int32_t *pool_out, const int32_t *reuse_src,
                            int32_t *topk_out, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * csa2_kv_append of the n_append rows (k, v, idx_k_in, a_seq, a_pos) followed
 * by csa2_index_topk (every other argument), in one call on one stream, with
 * the same results as the two calls: a decode step's append and its first
 * index layer (aiwiki "DeepSeek V4.1-Flash", section "Compressed Sparse
 * Attention 2": the new token's index key is scored with the rest).
 * Where the index scoring streams the keys in workgroups of 2048 or 4096
 * candidates (FULL, or REINDEX without pool_in, with enough queries x
 * candidates to fill the chip; not the matrix-core scorer) and n_append <=
 * 256, the rows are stored by extra workgroups of the scoring launch and each
 * appended position a query sees is scored from its row's input, so the
 * step needs no separate append launch; otherwise the append runs first as
 * its own launch.  Workspace: csa2_index_topk_workspace's.
 * Preconditions: csa2_kv_append's for the rows, csa2_index_topk's for the rest.
 * Errors: csa2_kv_append's (rows checked first), then csa2_index_topk's.
 */
csa2_status csa2_index_topk_append(const csa2_cache *cache, const uint16_t *k, const uint16_t *v,
                                   const uint16_t *idx_k_in, const int32_t *a_seq,
                                   const int32_t *a_pos, int32_t n_append, csa2_mode mode,
                                   const uint16_t *q_idx, csa2_dtype q_dtype,
                                   const int32_t *q_seq, const int32_t *q_pos, int32_t nq,
                                   int32_t top_k, const int32_t *pool_in, int32_t pool_len,
                                   int32_t pool_blocks, int32_t *pool_out,
                                   const int32_t *reuse_src, int32_t *topk_out, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* Bytes of workspace csa2_sparse_attn needs (0 for invalid arguments). */
size_t csa2_sparse_attn_workspace(const csa2_cache *cache, int32_t nq, int32_t n_heads,
                                  int32_t top_k);

/*
 * Sparse softmax attention over the selected FP4 rows (model card,
 * Introduction, CSA2 paragraph; aiwiki "Compressed Sparse Attention 2": every
 * layer attends over its Top-K positions of the shared FP4 main KV; all query
 * heads share the one KV head).
 *   q          [nq][n_heads][dk] bf16 bits.
 *   q_seq      [nq] int32 sequence each query reads.
 *   topk       [nq][top_k] int32 rows; entries < 0 are skipped; each entry
 *              counts once (duplicates count twice).
 *   softmax_scale  multiplies q.k (pass 1/sqrt(dk) for the usual scaling).
 *   out        [nq][n_heads][dv] fp32: sum_j softmax(z)_j V_j with
 *              z_j = softmax_scale * q_h . K_j, K and V dequantized exactly.
 *   lse        [nq][n_heads] fp32 natural-log sum of exp(z_j), or NULL.
 * An empty selection gives out = 0 and lse = -inf.  Accumulation is fp32 on
 * matrix cores (fp16 q.K products, fp16 probabilities times V).
 * Input range: q is rounded once to fp16, so every |q| element must be at most
 * 65504 (larger finite bf16 values overflow to infinity and make out and lse
 * NaN); elements below 2^-14 in magnitude lose bits below 2^-24.
 * Supported: n_heads a multiple of 16 up to 128; dk = dv = 128.
 * Device preconditions: 0 <= q_seq < batch; topk entries < capacity.
 * Errors: CSA2_ERR_NULL, CSA2_ERR_SHAPE, CSA2_ERR_UNSUPPORTED,
 * CSA2_ERR_WORKSPACE, CSA2_ERR_HIP.
 */
csa2_status csa2_sparse_attn(const csa2_cache *cache, const uint16_t *q, int32_t n_heads,
                             const int32_t *q_seq, int32_t nq, const int32_t *topk, int32_t top_k,
                             float softmax_scale, float *out, float *lse, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * csa2_sparse_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation, arguments and results as csa2_sparse_attn, without a
 * workspace argument.  The split partials go to a static device array of
 * 16 MiB (16777216 bytes) that the library holds on every device it runs on
 * until the process ends; the call allocates nothing.
 *   Limit: csa2_sparse_attn_workspace(cache, nq, n_heads, top_k) must not
 *   exceed 16 MiB (for example 32 queries x 64 heads x top_k 2048 need 8.5
 *   MiB); larger calls return CSA2_ERR_WORKSPACE and enqueue nothing.
 *   The stream must belong to the calling thread's current device (the array
 *   of that device is used).  Every call on one device shares its array:
 *   calls that overlap on one device (concurrent streams, or another thread)
 *   race and give undefined results; calls ordered on one stream are safe.
 *   The first call on a device looks up the array's device address
 *   (hipGetSymbolAddress) once.
 * Errors: as csa2_sparse_attn.
 */
csa2_status csa2_sparse_attn_noalloc(const csa2_cache *cache, const uint16_t *q, int32_t n_heads,
                                     const int32_t *q_seq, int32_t nq, const int32_t *topk,
                                     int32_t top_k, float softmax_scale, float *out, float *lse,
                                     void *stream);

/*
 * The local sliding-window KV of one layer (aiwiki "DeepSeek V4.1-Flash",
 * section "Compressed Sparse Attention 2": besides its query, every CSA2 layer
 * creates its own local sliding-window keys and values; section "KV-cache
 * formats and bounded replay": that local window KV is stored in FP8).
 * Caller-owned device memory, a ring of `window` slots per sequence:
 *   k, v   [batch][window][dk], [batch][window][dv] bytes: E4M3 codes of the
 *          bf16 rows (round to nearest even, saturating at +-448, sign kept,
 *          no scale).
 *   pos    [batch][window] int32: the position a slot holds, -1 = none (fill
 *          with -1 before first use).
 * Position p of sequence s lives in slot p % window.
 * Supported: dk = dv = 128, window 1 .. 1024.
 */
typedef struct csa2_local_cache {
  uint8_t *k;
  uint8_t *v;
  int32_t *pos;
  int32_t batch;
  int32_t window;
  int32_t dk;
  int32_t dv;
} csa2_local_cache;

/*
 * Quantize-and-append n rows into the local window (E4M3 codes as above).
 *   k, v       [n][dk], [n][dv] bf16 bits.
 *   seq, pos   [n] int32: row r is position pos[r] of sequence seq[r]; it
 *              replaces whatever slot pos[r] % window held.
 * Device preconditions: 0 <= seq[r] < batch, pos[r] >= 0; no two rows of one
 * call share a (seq, slot).
 * Errors: CSA2_ERR_NULL, CSA2_ERR_SHAPE (n < 0), CSA2_ERR_UNSUPPORTED, CSA2_ERR_HIP.
 * n = 0 is a no-op returning CSA2_OK.
 */
csa2_status csa2_local_append(const csa2_local_cache *cache, const uint16_t *k, const uint16_t *v,
                              const int32_t *seq, const int32_t *pos, int32_t n, void *stream);

/*
 * The local window branch, merged into the sparse branch's result (the same
 * softmax over both sets of rows, through the sparse branch's lse).
 *   q          [nq][n_heads][dk] bf16 bits (the same queries as the sparse call).
 *   q_seq, q_pos [nq] int32: the window rows of a query are the positions
 *              max(0, q_pos - window + 1) .. q_pos of its sequence whose slot
 *              holds that position.
 *   out, lse   on entry csa2_sparse_attn's out [nq][n_heads][dv] and lse
 *              [nq][n_heads]; on return the softmax attention over the union
 *              of the selected FP4 rows and the window's FP8 rows:
 *              out = sum_j softmax(z)_j V_j, lse = ln sum_j exp(z_j), with
 *              z_j = softmax_scale * q_h . K_j over both sets.
 * Rows of both sets are different cached values (the global FP4 KV and the
 * layer's own FP8 window), so a position in both counts twice.  Accumulation
 * is fp32 on matrix cores (fp16 q.K products, fp16 probabilities times V);
 * q must lie within the fp16 range (|q| <= 65504), as for csa2_sparse_attn.
 * Supported: n_heads a multiple of 16 up to 128; dk = dv = 128.
 * Device preconditions: 0 <= q_seq < batch, q_pos >= 0.
 * Errors: CSA2_ERR_NULL, CSA2_ERR_SHAPE, CSA2_ERR_UNSUPPORTED, CSA2_ERR_HIP.
 */
csa2_status csa2_local_attn(const csa2_local_cache *cache, const uint16_t *q, int32_t n_heads,
                            const int32_t *q_seq, const int32_t *q_pos, int32_t nq,
                            float softmax_scale, float *out, float *lse, void *stream);

/*
 * Both branches of a layer in one pass: the selected FP4 rows (as
 * csa2_sparse_attn) and the layer's FP8 window rows (as csa2_local_attn) in
 * one softmax, written to out and lse directly.  The window rows become extra
 * splits of the same launch, merged with the selected rows' splits by one
 * combine, so the window costs no launch of its own.
 *   cache, q, n_heads, q_seq, nq, topk, top_k, softmax_scale: as for
 *              csa2_sparse_attn; local, q_pos: as for csa2_local_attn
 *              (local->batch >= cache->batch; q_seq indexes both).
 *   out, lse   [nq][n_heads][dv], [nq][n_heads] (lse may be NULL): the
 *              softmax attention over the union of both sets of rows.
 *   workspace  device scratch of csa2_sparse_local_attn_workspace bytes.
 * Supported, input range, device preconditions and errors: as
 * csa2_sparse_attn together with csa2_local_attn (CSA2_ERR_SHAPE also for
 * local->batch < batch).
 */
size_t csa2_sparse_local_attn_workspace(const csa2_cache *cache, const csa2_local_cache *local,
                                        int32_t nq, int32_t n_heads, int32_t top_k);
csa2_status csa2_sparse_local_attn(const csa2_cache *cache, const csa2_local_cache *local,
                                   const uint16_t *q, int32_t n_heads, const int32_t *q_seq,
                                   const int32_t *q_pos, int32_t nq, const int32_t *topk,
                                   int32_t top_k, float softmax_scale, float *out, float *lse,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * The encoder-side projection fused into quantize-and-append (aiwiki
 * "DeepSeek V4.1-Flash", section "Causal Encoder-Decoder": a decoder layer's
 * global keys and values are projected from the final causal-encoder hidden
 * states with that layer's own projection weights).  For each of n tokens:
 *   y = w . x   (fp32 accumulation of bf16 products), rounded to bf16
 * (nearest, ties to even); y's channels are K (0..127), V (128..255) and the
 * index keys (256 .. 256 + idx_heads * 64 - 1, head-major); they are then
 * quantized and stored exactly as csa2_kv_append stores those bf16 rows.
 * The fp32 summation order depends on d_model only: a token's bytes do not
 * depend on n or on the other tokens of the call.
 *   x          [n][d_model] bf16 bits, the hidden states.
 *   w          [256 + idx_heads * 64][d_model] bf16 bits, the projection
 *              weights, one row per output channel.
 *   seq, pos   [n] int32, as for csa2_kv_append.
 * Supported: d_model a multiple of 32, 32 .. 65536.
 * Device preconditions and errors as csa2_kv_append (CSA2_ERR_SHAPE also
 * for d_model).  n = 0 is a no-op returning CSA2_OK.
 */
csa2_status csa2_proj_append(const csa2_cache *cache, const uint16_t *x, int32_t d_model,
                             const uint16_t *w, const int32_t *seq, const int32_t *pos, int32_t n,
                             void *stream);

/*
 * Persistent KV (aiwiki "DeepSeek V4.1-Flash", section "KV-cache formats and
 * bounded replay": the long-lived global state is kept apart from the runtime
 * cache, on SSD or host memory, to resume or reuse a prefix).  The persistent
 * form of positions [0, len) of one sequence is the byte image of its rows,
 * in this order, with no header:
 *   kv_codes  len * 128 bytes          (kv_codes[seq][0 .. len), row-major)
 *   kv_scales len * 16 bytes           (kv_scales[seq][0 .. len))
 *   idx_k     ceil(len / T) whole tiles of 64 * 64 * E bytes (the tiled
 *             layout above; T = 64 / idx_heads positions per tile).
 * A last, partly filled tile also carries the bytes of positions len ..
 * ceil(len / T) * T - 1, which no query sees before they are appended.
 * csa2_kv_export_bytes gives the image's size (0 for an invalid cache or len).
 */
size_t csa2_kv_export_bytes(const csa2_cache *cache, int32_t len);

/*
 * Copies the persistent image of positions [0, len) of sequence seq to dst
 * (device memory or pinned host memory from hipHostMalloc, dst_bytes >=
 * csa2_kv_export_bytes), ordered on the stream; synchronize the stream before
 * reading a host dst.
 * Errors: CSA2_ERR_NULL, CSA2_ERR_SHAPE (seq outside [0, batch), len outside
 * [0, capacity]), CSA2_ERR_UNSUPPORTED, CSA2_ERR_WORKSPACE (dst_bytes too
 * small), CSA2_ERR_HIP.  len = 0 is a no-op returning CSA2_OK.
 */
csa2_status csa2_kv_export(const csa2_cache *cache, int32_t seq, int32_t len, void *dst,
                           size_t dst_bytes, void *stream);

/*
 * Writes a persistent image (from csa2_kv_export of a cache with the same
 * idx_heads and idx_k_dtype; capacity and batch may differ) into positions
 * [0, len) of sequence seq, ordered on the stream; src as for dst above.
 * Appends after it continue at position len.
 * Errors: as csa2_kv_export (src_bytes too small: CSA2_ERR_WORKSPACE).
 */
csa2_status csa2_kv_import(const csa2_cache *cache, int32_t seq, int32_t len, const void *src,
                           size_t src_bytes, void *stream);

/*
 * Empties sequence seq's local window (every slot's position set to -1) by a
 * small kernel on the stream (no memset node, so the call can be captured).
 * With csa2_local_append of the most recent min(window, len) positions this
 * is the bounded replay of the page's section "KV-cache formats and bounded
 * replay": the window is rebuilt from recent tokens instead of being stored.
 * Errors: CSA2_ERR_NULL, CSA2_ERR_SHAPE (seq outside [0, batch)),
 * CSA2_ERR_UNSUPPORTED, CSA2_ERR_HIP.
 */
csa2_status csa2_local_clear(const csa2_local_cache *cache, int32_t seq, void *stream);

/*
 * Profiling hook for callers that measure the index scan against its
 * roofline (bench use; no effect on results).  After a call with non-NULL
 * events (two hipEvent_t), every csa2_index_topk call made later from the same
 * host thread records `before` and `after` on its stream around its scoring:
 * the streaming scorer's one kernel that reads the index keys, or the
 * matrix-core scorer's product passes (the sampled and the emitting pass, or
 * the block-maximum and the emitting pass) with the launches between them.  csa2_profile_index_scan(NULL, NULL) turns the hook off.  The
 * events are caller-owned; the library only records them.
 */
void csa2_profile_index_scan(void *before, void *after);

/* Static description of a status code. */
const char *csa2_strerror(csa2_status status);

/* CSA2_ABI_VERSION of the loaded library. */
int csa2_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
