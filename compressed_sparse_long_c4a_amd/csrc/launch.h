// Internal launch entry points behind the C ABI (arguments already validated by api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

// ---------------------------------------------------------------- compress
constexpr int kMaxCompressJobs = 4;  // compressor instances one launch can run

struct CompressJob {
  int ratio;
  const void* new_raw;
  int raw_dtype;
  const int32_t* cu_entries;
  int total_entries;
  const float* logits;
  const float* gamma;
  float eps, rope_base;
  int rope_dims;
  const csa_cache* state;
  const csa_cache* out;
  const csa_cache* swa;
};

struct CompressLaunch {
  int batch;
  const int32_t* ctx_lens;
  const int32_t* cu_new;
  int total_new;
  int num_jobs;
  CompressJob jobs[kMaxCompressJobs];
};
hipError_t launch_compress(const CompressLaunch& a, hipStream_t stream);

// ---------------------------------------------------------------- query norm + window keys
struct QNormLaunch {
  int total_q;
  const int32_t* q_pos;
  const void* q_in;
  void* q_out;
  int q_dtype, n_heads, dim;
  const float* q_gamma;
  float eps, rope_base;
  int rope_dims;
  int batch;
  const int32_t* ctx_lens;
  const int32_t* cu_new;
  int total_new;
  const void* new_raw;
  int raw_dtype;
  const csa_cache* swa;  // NULL: queries only
};
hipError_t launch_q_norm_rope_swa(const QNormLaunch& a, hipStream_t stream);

// ---------------------------------------------------------------- indexer
// Entries handled by one workgroup of the score / filter kernels.
constexpr int kIndexChunk = 2048;

struct IndexWorkspace {
  float* scores;       // [total_q][n_cap]
  int32_t* new_from;   // [total_q]           first entry id the call's compressor inserted
  uint2* new_cand;     // [total_q][64]       (key, id) of the entries the call's compressor inserted
  uint2* cand;         // [total_q][n_cap]    (key, entry) candidates, chunk-sparse
  int4* cand_info;     // [total_q][chunks]   candidate count, least and largest key, bound
  int chunks;          // per query
  int64_t n_cap;       // chunks * kIndexChunk
};
size_t index_workspace_bytes(int total_q, int max_context, int k);
IndexWorkspace index_workspace_carve(void* ws, int total_q, int max_context, int k);

struct IndexLaunch {
  int batch;
  const int32_t* cu_q;
  const int32_t* q_pos;
  int total_q, max_context;
  const void* q_idx;
  int q_dtype, n_heads;
  const float* head_w;
  const csa_cache* idx_cache;
  int k;
  // A slice of a call's queries: q_pos, q_idx, head_w (and the outputs) point at the slice's
  // first query, total_q counts the slice, and q_base is that query's index in the call (cu_q
  // keeps the call's indices).  0 for a whole call.
  int q_base = 0;
};
hipError_t launch_index_score(const IndexLaunch& a, const IndexWorkspace& ws, hipStream_t stream);
// The compressor jobs of `c` and the index score in one launch (bf16 queries, <= 64 heads, ratio-4
// jobs; jobs[score_job] writes the indexer keys of a.idx_cache).
hipError_t launch_compress_index_score(const IndexLaunch& a, const IndexWorkspace& ws,
                                       const CompressLaunch& c, int score_job, hipStream_t stream);
hipError_t launch_index_select(const IndexLaunch& a, int32_t* topk_idx, float* topk_score,
                               const IndexWorkspace& ws, hipStream_t stream);

// ---------------------------------------------------------------- attention
// Rows (top-k list length or visible entries, plus window) one query may attend to.
constexpr int64_t kAttnMaxRows = 256 * 1024;
// Most rows one attention workgroup takes (their addresses are staged in LDS): the fp8-row
// kernel with bf16 queries holds 1,024, the generic kernel 2,048.
constexpr int kAttnRowsCapFp8 = 1024;
constexpr int kAttnRowsCapGeneric = 2048;
inline int attn_rows_cap(int kv_dtype, int q_dtype) {
  return kv_dtype == CSA_FP8_E4M3 && q_dtype == CSA_BF16 ? kAttnRowsCapFp8 : kAttnRowsCapGeneric;
}

struct AttnPlan {
  int splits;          // row splits per (query, head group)
  int rows_per_split;  // multiple of 32
  int head_groups;     // ceil(n_heads / 16)
  int64_t max_rows;
};
AttnPlan attn_plan(int total_q, int n_heads, int ratio, int has_topk, int k, int max_context,
                   int window, int rows_cap);
size_t attn_workspace_bytes(int total_q, int n_heads, int dim, const AttnPlan& p);

struct AttnLaunch {
  int batch;
  const int32_t* cu_q;
  const int32_t* q_pos;
  int total_q, max_context;
  const void* q;
  int q_dtype, n_heads;
  const csa_cache* kv;
  int ratio;
  const int32_t* topk_idx;
  int k;
  const csa_cache* swa;
  int window;
  float softmax_scale, rope_base;
  int rope_dims;
  float* out;           // [total_q][n_heads][dim] float32, or NULL when only fp8 is wanted
  float* lse;
  uint8_t* out_fp8;     // NULL, or [total_q][n_heads][dim] OCP E4M3 codes of the same rows
  float* out_scales;    // with out_fp8: [total_q][n_heads], one scale per row (amax / 448)
};
hipError_t launch_sparse_attn(const AttnLaunch& a, const AttnPlan& p, void* workspace,
                              hipStream_t stream);

// csa_sparse_attn_decode_noalloc: the largest workspace it serves from the library's own
// device array, and that array's address on the current device (resolved once per device;
// NULL with *err set if the lookup fails).
constexpr size_t kAttnStaticScratchBytes = (size_t)16 << 20;
void* attn_static_scratch(hipError_t* err);

}  // namespace csa
