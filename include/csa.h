/*
 * csa.h -- one layer of compressed sparse attention decode on AMD Instinct
 * MI355X (gfx950): compress -> index/top-k -> sparse K=V attention ->
 * inverse RoPE.
 *
 * Sources (the method is defined by these pages; section names as printed):
 *   [vLLM-V4]      "DeepSeek V4 in vLLM: Efficient Long-context Attention"
 *                  (digest of the vLLM team's blog post): section 2 design
 *                  principles; section 3 part 1 keeping the KV cache packed;
 *                  section 3 part 2 keeping the GPU busy; appendix (why
 *                  inverse RoPE, exact position ranges and causality, exact
 *                  k values, why the short window).
 *   [SGLang-pools] "SGLang KV Cache storage pool architecture": section 3
 *                  (the 576 = 512 + 64 MLA row shared by K and V) and
 *                  section 4 (the 132-byte fp8 indexer row).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked "host".  All memory is owned
 *     by the caller; the library never allocates and never frees.  Scratch
 *     memory is the caller's `workspace`, sized by the *_workspace_size
 *     queries.  A `csa_cache` descriptor itself lives in host memory.
 *   - Every call is asynchronous on `stream` and never synchronises the
 *     host; buffers must stay alive until the stream has passed the call.
 *   - Host-visible arguments are validated before anything is launched; on a
 *     non-zero status nothing was launched.  CSA_EHIP reports a failed launch
 *     (hipGetLastError after launching).  No C++ exception crosses the ABI.
 *   - Device-side contents (lengths, positions, block-table entries, top-k
 *     ids) are trusted: values outside the documented ranges are undefined
 *     behaviour, except where a call states how it treats them.
 *   - The functions keep no state between calls and may be called from
 *     several threads on different streams.
 *   - An array of length zero (total_q = 0, total_new = 0, ...) may be passed
 *     as NULL; a call with no work returns CSA_OK without launching.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 1

/* A hipStream_t (struct ihipStream_t*); NULL is the null stream. */
typedef struct ihipStream_t* csa_stream_t;

/* Element types of stored rows and of query inputs. */
typedef enum {
  CSA_F32 = 0,       /* IEEE float32 */
  CSA_BF16 = 1,      /* bfloat16 */
  CSA_FP8_E4M3 = 2,  /* OCP E4M3 ("e4m3fn") codes with one float32 scale per row */
  CSA_FP4_E2M1 = 3   /* OCP E2M1 codes, two per byte, with one E8M0 scale byte per 16 values */
} csa_dtype;

/* Status codes. */
enum {
  CSA_OK = 0,
  CSA_EINVAL = -1,      /* a required pointer is NULL or a size/argument is out of range */
  CSA_ENOTSUP = -2,     /* a combination of dtype / dim / heads this build does not implement */
  CSA_EWORKSPACE = -3,  /* workspace smaller than the matching *_workspace_size() */
  CSA_EHIP = -4         /* the HIP runtime reported an error while launching */
};

/*
 * One paged cache ([vLLM-V4] section 3 part 1: every compressed layer uses a
 * logical block of 256 native positions).  Logical row r of sequence b --
 * an entry index for compressed caches, a raw token position for window and
 * compressor-state caches -- lives in physical block
 * block_table[b * bt_stride + r / rows_per_block] at slot r % rows_per_block.
 * rows_per_block is therefore 64 for a c4a cache (256 / 4 entries), 2 for a
 * c128a cache (256 / 128) and 256 for window and state caches.
 *
 * Row layout: `dim` contiguous elements.  Main KV rows are the shared key and
 * value, 512 latent dimensions followed by the 64 RoPE dimensions
 * ([SGLang-pools] section 3); indexer rows are 128 dimensions.  FP8 rows keep
 * their float32 scales in a separate [num_blocks][rows_per_block] array
 * (value = code * scale; 128 codes + 4 scale bytes = the 132-byte indexer row
 * of [SGLang-pools] section 4).  Scales must be positive.
 *
 * FP4 rows ([SGLang-pools] section 7, FP4 quantisation: two 4-bit values a
 * byte and one scale per 16 values; [vLLM-V4] section 2 puts the indexer
 * cache in fp4) hold dim / 2 bytes, element 2i in the low nibble of byte i and
 * element 2i + 1 in the high nibble; `scales` then points at uint8 E8M0 bytes
 * [num_blocks][rows_per_block][dim / 16], byte s meaning 2^(s - 127), and
 * value = E2M1(code) * 2^(s - 127).  Scale bytes must lie in 1..254.  `dim`
 * counts elements (128 for an indexer row of 64 + 8 bytes) and is a multiple
 * of 16.  FP4 is accepted for compressed-entry caches written by the
 * compressor and for the indexer cache, not for attention or window caches.
 */
typedef struct csa_cache {
  void*          rows;            /* [num_blocks][rows_per_block][dim] elements of `dtype` (fp8: uint8 codes;
                                     fp4: [..][dim / 2] bytes) */
  void*          scales;          /* float32 [num_blocks][rows_per_block] for CSA_FP8_E4M3, uint8
                                     [num_blocks][rows_per_block][dim / 16] for CSA_FP4_E2M1, else NULL */
  int32_t        dtype;           /* csa_dtype */
  int32_t        dim;             /* elements per row */
  int32_t        rows_per_block;  /* 64 (c4a), 2 (c128a) or 256 (window, state) */
  int32_t        num_blocks;      /* physical blocks in `rows` */
  const int32_t* block_table;     /* [batch][bt_stride] physical block ids, each in [0, num_blocks) */
  int32_t        bt_stride;       /* logical blocks per sequence in block_table */
} csa_cache;

/* CSA_ABI_VERSION of the loaded library. */
int csa_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char* csa_status_str(int status);

/*
 * Host helper: compressed entries after `num_tokens` raw tokens, floor(num_tokens / ratio)
 * ([vLLM-V4] appendix, exact position ranges: entry i of c4a ends at 4i + 3,
 * of c128a at 128i + 127).  Returns -1 if ratio is not 4 or 128 or num_tokens < 0.
 */
int64_t csa_num_entries(int ratio, int64_t num_tokens);

/*
 * csa_compress_insert -- the fused compressor ([vLLM-V4] section 3 part 2,
 * first fusion: compress + RMSNorm + RoPE + cache insert; one instance per
 * head dimension, main KV d = 576 or indexer d = 128).
 *
 * ratio 4 (c4a) or 128 (c128a); coff = 2 or 1; window W = coff * ratio raw rows
 * (8 or 128).  Sequence b held ctx_lens[b] raw tokens before the call and
 * receives new_raw rows [cu_new[b], cu_new[b+1]) at positions ctx_lens[b], ...
 * For every entry j completed by the call (its anchor a_j = ratio*j + ratio - 1
 * is one of the new positions; the call's entries for b are
 * j = n(ctx_lens[b]) .. n(ctx_lens[b] + new_b) - 1, in that order):
 *   x_r = raw row at position s_j + r, r in [0, W), s_j = ratio*j - (coff-1)*ratio,
 *         0 for negative positions ([vLLM-V4] appendix, exact position ranges);
 *   w   = softmax(gate_logits[cu_entries[b] + (j - n(ctx_lens[b]))][0..W));
 *   y   = sum_r w_r x_r;  n = y / sqrt(mean(y^2) + eps) * gamma  (whole row);
 *   c   = RoPE_{a_j}(n): the last rope_dims dimensions rotated in consecutive
 *         pairs (2i, 2i+1) by a_j * rope_base^(-2i/rope_dims) (angles in float64);
 *   out row j = c rounded to out->dtype (fp8: scale = amax/448, codes RNE; fp4: per
 *         block of 16 values the smallest power-of-two scale 2^k with amax / 2^k <= 6,
 *         k clamped to [-126, 127], codes RNE with ties to the even code).
 * Raw rows at positions below ctx_lens[b] are read from `state` (which must hold
 * the last W positions); the new rows among the last W positions after the call
 * are written to `state` (the rolling residual registered as sliding-window KV,
 * [vLLM-V4] section 3 part 1).  If `swa` is not NULL, every new row x_p is also
 * written there as RoPE_p(x_p) in swa->dtype (the uncompressed window rows).
 *
 * Arguments:
 *   ctx_lens   [batch] int32, >= 0.        cu_new [batch+1] int32, cu_new[0] = 0,
 *   total_new  = cu_new[batch] (host).     new_raw [total_new][dim] of raw_dtype (F32 or BF16).
 *   cu_entries [batch+1] int32 prefix sums of the per-sequence entry counts above;
 *   total_entries = cu_entries[batch] (host).  gate_logits [total_entries][W] float32.
 *   gamma [dim] float32 or NULL (= 1).  eps >= 0.  rope_base > 0.  rope_dims even,
 *   2..min(dim, 128).  state: rows_per_block 256, dtype = raw_dtype, same dim.
 *   out: rows_per_block 256 / ratio, dim = state dim, any dtype (FP4_E2M1: dim a
 *   multiple of 16).  swa: NULL or rows_per_block 256, same dim, F32, BF16 or
 *   FP8_E4M3.  dim <= 1024.
 * Cache rows must not alias new_raw; out, state and swa must be distinct memory.
 */
int csa_compress_insert(csa_stream_t stream, int ratio, int batch,
                        const int32_t* ctx_lens, const int32_t* cu_new, int total_new,
                        const void* new_raw, int raw_dtype,
                        const int32_t* cu_entries, int total_entries, const float* gate_logits,
                        const float* gamma, float eps, float rope_base, int rope_dims,
                        const csa_cache* state, const csa_cache* out, const csa_cache* swa);

/*
 * csa_compress_insert_many -- several compressor instances over the same new tokens in one
 * launch: for example a c4a layer's main-KV compressor (d = 576, with window rows) and its
 * indexer-key compressor (d = 128), which [vLLM-V4] section 3 part 2 runs as separate
 * instances per head dimension.  Every job computes exactly what csa_compress_insert computes
 * with the call's ctx_lens / cu_new / total_new and the job's own arguments (its own ratio,
 * entry offsets, logits, caches, dtype and RoPE settings).  1 <= num_jobs <= 4; `jobs` is a
 * host array.  The jobs must not write the same cache rows.  Returns the first job's error if
 * any job is rejected (nothing is launched then).
 */
typedef struct csa_compress_job {
  int32_t            ratio;          /* 4 or 128 */
  const void*        new_raw;        /* [total_new][dim] of raw_dtype */
  int32_t            raw_dtype;      /* CSA_F32 or CSA_BF16 */
  const int32_t*     cu_entries;     /* [batch+1] prefix sums of this job's emitted entries */
  int32_t            total_entries;  /* cu_entries[batch] (host) */
  const float*       gate_logits;    /* [total_entries][coff * ratio] */
  const float*       gamma;          /* [dim] or NULL (= 1) */
  float              eps, rope_base;
  int32_t            rope_dims;
  const csa_cache*   state;          /* host descriptors, as in csa_compress_insert */
  const csa_cache*   out;
  const csa_cache*   swa;            /* or NULL */
} csa_compress_job;

int csa_compress_insert_many(csa_stream_t stream, int batch, const int32_t* ctx_lens,
                             const int32_t* cu_new, int total_new, int num_jobs,
                             const csa_compress_job* jobs);

/*
 * csa_index_topk -- indexer score and top-k over c4a entries ([vLLM-V4]
 * section 2: DeepSeek Sparse Attention, the query attends to the top-k
 * compressed tokens; appendix: causality 4j + 3 <= t and default k).
 *
 * Query i (of sequence b, cu_q[b] <= i < cu_q[b+1]) sits at position
 * t = q_pos[i]; its candidates are the c4a entries j < n(t + 1) (those with
 * anchor 4j + 3 <= t), capped at n(max_context).  Its score for entry j is
 *     s_j = sum_h head_w[i][h] * max(0, q_idx[i][h] . k_j)
 * with k_j the stored indexer key (fp8 code * scale).  The k' = min(k, n)
 * best are written to topk_idx[i][0..k') in ascending entry order; the rest
 * of the row is -1.  Among exactly equal scores lower entry ids win.
 * topk_score (optional) receives the matching float32 scores (0 for padding).
 *
 *   cu_q [batch+1], q_pos [total_q] int32 (0 <= t < max_context).
 *   q_idx [total_q][n_heads_idx][128] of q_dtype: CSA_BF16 (1 <= n_heads_idx <= 64)
 *         or CSA_F32 (any n_heads_idx >= 1).
 *   head_w [total_q][n_heads_idx] float32.
 *   idx_cache: dim 128, rows_per_block 64, dtype FP8_E4M3, FP4_E2M1 or BF16 (any
 *         dtype with CSA_F32 queries).
 *   1 <= k <= 65536.  topk_idx [total_q][k] int32.  topk_score [total_q][k] or NULL.
 *   workspace: csa_index_workspace_size(total_q, max_context, k) bytes take every query in
 *         one pass (one score and one select launch).  Any smaller workspace of at least
 *         csa_index_workspace_size(1, max_context, k) bytes is also accepted: the queries are
 *         then taken in consecutive slices of as many as fit (two launches per slice, same
 *         results), which bounds the memory of long chunked prefills; below that size the
 *         call returns CSA_EWORKSPACE before any launch.
 */
size_t csa_index_workspace_size(int total_q, int max_context, int k);

int csa_index_topk(csa_stream_t stream, int batch, const int32_t* cu_q, const int32_t* q_pos,
                   int total_q, int max_context, const void* q_idx, int q_dtype, int n_heads_idx,
                   const float* head_w, const csa_cache* idx_cache, int k,
                   int32_t* topk_idx, float* topk_score, void* workspace, size_t workspace_bytes);

/*
 * The two halves of csa_index_topk, for callers that schedule or time them
 * separately.  csa_index_score writes every candidate's score (and per-chunk
 * selection bounds) into `workspace`; csa_index_select reads them back and
 * writes topk_idx / topk_score.  Called back to back on one stream with the
 * same arguments and workspace they are exactly csa_index_topk.  Both need the
 * whole call's workspace, csa_index_workspace_size(total_q, max_context, k).
 */
int csa_index_score(csa_stream_t stream, int batch, const int32_t* cu_q, const int32_t* q_pos,
                    int total_q, int max_context, const void* q_idx, int q_dtype, int n_heads_idx,
                    const float* head_w, const csa_cache* idx_cache, int k,
                    void* workspace, size_t workspace_bytes);

int csa_index_select(csa_stream_t stream, int batch, const int32_t* cu_q, const int32_t* q_pos,
                     int total_q, int max_context, int k, int32_t* topk_idx, float* topk_score,
                     void* workspace, size_t workspace_bytes);

/*
 * csa_q_norm_rope_swa -- query normalisation + RoPE and the window keys in one launch
 * ([vLLM-V4] section 3 part 2, third fusion: fused Q norm + KV RoPE + K insert, one warp
 * per query head or key head, no cross-warp communication).
 *
 * For every query i and head h (the pages name the operations only; the reading is the
 * compressor's RMSNorm and RoPE applied per query head):
 *   n = q_in[i][h] / sqrt(mean(q_in[i][h]^2) + eps) * q_gamma   (over the head's dim values);
 *   q_out[i][h] = RoPE_{q_pos[i]}(n): the last rope_dims dimensions rotated in consecutive
 *                 pairs (2j, 2j+1) by q_pos[i] * rope_base^(-2j/rope_dims) (angles in
 *                 float64), rounded to q_dtype.
 * If `swa` is not NULL, every new raw row x_p -- sequence b held ctx_lens[b] raw tokens and
 * receives new_raw rows [cu_new[b], cu_new[b+1]) at positions ctx_lens[b], ... -- is stored
 * in `swa` at p as RoPE_p(x_p) in swa->dtype (fp8: scale = amax/448, codes RNE): the same rows
 * csa_compress_insert writes when it is given a window cache.
 *
 * Arguments:
 *   total_q >= 0.  q_pos [total_q] int32 >= 0.  q_in, q_out [total_q][n_heads][dim] of
 *   q_dtype (F32 or BF16), not overlapping.  n_heads >= 1.  dim a multiple of 8, <= 1024.
 *   q_gamma [dim] float32 or NULL (= 1).  eps >= 0.  rope_base > 0.  rope_dims a multiple
 *   of 8, 8..min(dim, 128).
 *   Window keys (read only when swa != NULL): batch >= 1, ctx_lens [batch] int32 >= 0,
 *   cu_new [batch+1] int32 prefix sums with cu_new[batch] = total_new (host), new_raw
 *   [total_new][dim] of raw_dtype (F32 or BF16); swa: rows_per_block 256, the same dim,
 *   F32, BF16 or FP8_E4M3, not overlapping new_raw or q_out.
 * total_q = 0 and total_new = 0 are valid; with neither, nothing is launched.
 * Returns CSA_EINVAL for inconsistent arguments, CSA_ENOTSUP for an unsupported dtype or
 * dim; a zero-length array may be NULL.
 */
int csa_q_norm_rope_swa(csa_stream_t stream, int total_q, const int32_t* q_pos, const void* q_in,
                        void* q_out, int q_dtype, int n_heads, int dim, const float* q_gamma,
                        float eps, float rope_base, int rope_dims, int batch,
                        const int32_t* ctx_lens, const int32_t* cu_new, int total_new,
                        const void* new_raw, int raw_dtype, const csa_cache* swa);

/*
 * csa_sparse_attn_decode -- multi-query attention with K = V over the selected
 * compressed entries plus the uncompressed sliding window, then inverse RoPE
 * ([vLLM-V4] section 2: shared K/V, top-k sparse attention, window of 128;
 * appendix: Output = Attention(Q, K, V) R_t^{-1}; c128a attends to all of its
 * entries, framed as top-k 8192; window rows [t-127, t]).
 *
 * For query i at position t = q_pos[i] of sequence b the row set is
 *   { kv row j : j in topk_idx[i][0..k), 0 <= j < n_t }   (n_t = n(t + 1) for `ratio`;
 *                                                          ids outside are padding, skipped)
 *   or, when topk_idx is NULL, { kv row j : 0 <= j < min(n_t, n(max_context)) };
 *   plus { swa row p : max(0, t - window + 1) <= p <= t }.
 * Each row serves as key and value.  For every head h:
 *   z_r = softmax_scale * q[i][h] . row_r;  o = sum_r softmax(z)_r row_r  (full dim);
 *   out[i][h] = o with its last rope_dims dimensions rotated by -t (R_t^{-1});
 *   lse[i][h] = log(sum_r exp(z_r)) (natural log; -inf and out = 0 if no rows).
 * List entries should be distinct (a repeated id is attended twice).
 *
 *   q [total_q][n_heads][dim] of q_dtype (CSA_BF16 or CSA_F32), already rotated.
 *   kv: rows_per_block 256 / ratio; swa: rows_per_block 256; both with the same
 *       dim (512 or 576) and the same dtype (F32, BF16 or FP8_E4M3).  rope_dims = 64.
 *   1 <= n_heads <= 128.  topk_idx [total_q][k] int32 or NULL (then k is ignored).
 *   The row count per query, (topk_idx ? k : n(max_context)) + min(window, max_context), must
 *   not exceed 262144 (CSA_ENOTSUP otherwise; the workspace query then returns 0).
 *   0 <= window <= 4096.  out [total_q][n_heads][dim] float32.  lse [total_q][n_heads] or NULL.
 *   workspace of at least csa_sparse_attn_workspace_size(...) bytes with the same
 *   total_q, n_heads, dim, ratio, topk_idx != NULL, k, max_context and window.
 */
size_t csa_sparse_attn_workspace_size(int total_q, int n_heads, int dim, int ratio, int has_topk,
                                      int k, int max_context, int window);

int csa_sparse_attn_decode(csa_stream_t stream, int batch, const int32_t* cu_q,
                           const int32_t* q_pos, int total_q, int max_context,
                           const void* q, int q_dtype, int n_heads,
                           const csa_cache* kv, int ratio, const int32_t* topk_idx, int k,
                           const csa_cache* swa, int window, float softmax_scale,
                           float rope_base, int rope_dims, float* out, float* lse,
                           void* workspace, size_t workspace_bytes);

/*
 * csa_sparse_attn_decode_noalloc -- csa_sparse_attn_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same kernels and results.  Its
 * scratch (the split partials) is a device array inside the library, one per GPU, held until
 * the process ends; the call allocates and frees nothing.  Limit: the workspace the call would
 * need (csa_sparse_attn_workspace_size for its arguments) must not exceed 16 MiB
 * (16,777,216 bytes), else CSA_EWORKSPACE and nothing is launched.  Every call on a GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different host threads) race and give wrong results; calls in
 * one stream are ordered and safe.  No part of the array needs to start at zero.  Returns
 * CSA_EHIP if the array's device address cannot be resolved on the current device.
 */
int csa_sparse_attn_decode_noalloc(csa_stream_t stream, int batch, const int32_t* cu_q,
                                   const int32_t* q_pos, int total_q, int max_context,
                                   const void* q, int q_dtype, int n_heads,
                                   const csa_cache* kv, int ratio, const int32_t* topk_idx, int k,
                                   const csa_cache* swa, int window, float softmax_scale,
                                   float rope_base, int rope_dims, float* out, float* lse);

/*
 * csa_sparse_attn_decode_fp8 -- csa_sparse_attn_decode with the output row quantised to fp8 in
 * the same launch as the inverse RoPE ([vLLM-V4] section 3 part 2, second fusion: inverse RoPE
 * + fp8 quantisation, the input of the output projection's fp8 matrix products).  The pages do
 * not give the fp8 layout; each output row (query, head) is stored like an fp8 cache row:
 * out_scales[i][h] = amax / 448 over the row's dim values (1 for an all-zero row) and
 * out_fp8[i][h][d] = the OCP E4M3 code of out[i][h][d] / scale, rounded to nearest even.
 *
 * Arguments as csa_sparse_attn_decode, plus out_fp8 [total_q][n_heads][dim] uint8 and
 * out_scales [total_q][n_heads] float32 (both required when total_q > 0); `out` may be NULL
 * (only the fp8 row is written) or receive the float32 row the codes were taken from.  The
 * workspace is csa_sparse_attn_workspace_size(...) bytes as for csa_sparse_attn_decode.
 */
int csa_sparse_attn_decode_fp8(csa_stream_t stream, int batch, const int32_t* cu_q,
                               const int32_t* q_pos, int total_q, int max_context,
                               const void* q, int q_dtype, int n_heads,
                               const csa_cache* kv, int ratio, const int32_t* topk_idx, int k,
                               const csa_cache* swa, int window, float softmax_scale,
                               float rope_base, int rope_dims, uint8_t* out_fp8,
                               float* out_scales, float* out, float* lse,
                               void* workspace, size_t workspace_bytes);

/*
 * csa_compress_index_score -- csa_compress_insert_many followed by csa_index_score, with the
 * compressor running beside the score instead of before it ([vLLM-V4] section 3 part 2,
 * multi-stream: the pages overlap the compressor with the indexer on a second stream; here
 * the compressor's workgroups share the score's launch).  The score workgroups read and score
 * only the entries that existed before the call (the first ctx_lens[b] / 4 of sequence b);
 * the indexer-key compressor jobs[idx_job] scores each entry it inserts, from the key it
 * stores, for every query of its sequence that sees the entry.  Scores and chunk bounds land in
 * the workspace as csa_index_score leaves them, so csa_index_select follows unchanged.
 *
 * Arguments: those of csa_compress_insert_many (batch, ctx_lens, cu_new, total_new, num_jobs,
 * jobs) and of csa_index_score (cu_q, q_pos, total_q, max_context, q_idx, q_dtype,
 * n_heads_idx, head_w, idx_cache, k, workspace); jobs[idx_job] must have ratio 4 and write
 * idx_cache (the same rows, dtype and block table).  Queries sit at positions the call
 * inserts or before (q_pos < ctx_lens[b] + new_b).  The single launch is used for bf16 queries,
 * at most 64 indexer heads, ratio-4 jobs and total_entries(jobs[idx_job]) * total_q <= 4096
 * (decode); otherwise the compressor and the score run as two launches with the same result.
 * Returns the status of the first failing check (nothing is launched then).
 */
int csa_compress_index_score(csa_stream_t stream, int batch, const int32_t* ctx_lens,
                             const int32_t* cu_new, int total_new, int num_jobs,
                             const csa_compress_job* jobs, int idx_job, const int32_t* cu_q,
                             const int32_t* q_pos, int total_q, int max_context, const void* q_idx,
                             int q_dtype, int n_heads_idx, const float* head_w,
                             const csa_cache* idx_cache, int k, void* workspace,
                             size_t workspace_bytes);

/*
 * csa_compress_index_score_launches -- how many kernel launches csa_compress_index_score makes
 * for these arguments (host-only, reads no device memory): 1 when the compressors run inside
 * the score launch, 2 when the compressor launch precedes the score launch, 1 or 0 when there
 * are no queries or nothing to compress.  total_new and the jobs' total_entries are the
 * counts the call would receive.  Returns CSA_EINVAL for a missing job array, idx_job out of
 * range or negative counts.
 */
int csa_compress_index_score_launches(int num_jobs, const csa_compress_job* jobs, int idx_job,
                                      int total_new, int total_q, int q_dtype, int n_heads_idx);

/*
 * csa_read_probe -- a measurement utility, not a step of the method: reads `bytes` bytes of the
 * device buffer `buf` once each with 16-byte non-temporal loads (eight in flight per thread)
 * and writes one word per workgroup to `sink`
 * (the XOR of the words it read, so no load can be dropped).  Timed on a buffer larger than
 * the 256 MB infinity cache it gives the device's achievable streaming read bandwidth, the
 * ceiling beside the 8 TB/s peak against which the indexer score kernel is reported.
 *   buf: 16-byte aligned, bytes a positive multiple of 16; sink: csa_read_probe_sink_words()
 *   uint32 words.  Returns CSA_EINVAL otherwise.
 */
int csa_read_probe(csa_stream_t stream, const void* buf, size_t bytes, uint32_t* sink);
int csa_read_probe_sink_words(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
