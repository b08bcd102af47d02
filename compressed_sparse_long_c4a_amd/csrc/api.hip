// The C ABI of libcsa: argument validation, workspace sizing and launch.  Nothing here
// allocates memory or synchronises the host.
#include <algorithm>

#include "csa.h"
#include "launch.h"

namespace {

constexpr int kMaxContextIndex = 8 * 1024 * 1024;  // select kernel: <= 1024 chunks of 2048 entries

bool dtype_ok(int dt) {
  return dt == CSA_F32 || dt == CSA_BF16 || dt == CSA_FP8_E4M3 || dt == CSA_FP4_E2M1;
}

// A cache descriptor with the given geometry (dim < 0: any dim).
bool cache_ok(const csa_cache* c, int rows_per_block, int dim) {
  if (!c || !c->rows || !c->block_table) return false;
  if (!dtype_ok(c->dtype) || c->rows_per_block != rows_per_block) return false;
  if (dim >= 0 && c->dim != dim) return false;
  if (c->dim <= 0 || c->bt_stride <= 0 || c->num_blocks <= 0) return false;
  if ((c->dtype == CSA_FP8_E4M3 || c->dtype == CSA_FP4_E2M1) && !c->scales) return false;
  if (c->dtype == CSA_FP4_E2M1 && (c->dim & 15)) return false;
  return true;
}

int hip_status(hipError_t e) { return e == hipSuccess ? CSA_OK : CSA_EHIP; }

}  // namespace

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_status_str(int status) {
  switch (status) {
    case CSA_OK: return "ok";
    case CSA_EINVAL: return "invalid argument";
    case CSA_ENOTSUP: return "unsupported dtype / dim / head combination";
    case CSA_EWORKSPACE: return "workspace too small";
    case CSA_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int64_t csa_num_entries(int ratio, int64_t num_tokens) {
  if ((ratio != 4 && ratio != 128) || num_tokens < 0) return -1;
  return num_tokens / ratio;
}

// Validates one compressor instance against the call's shared token layout and fills `job`.
static int compress_job_check(const csa_compress_job& j, int batch, int total_new,
                              csa::CompressJob* job) {
  if (j.ratio != 4 && j.ratio != 128) return CSA_EINVAL;
  if (j.total_entries < 0 || !j.cu_entries || !j.state || !j.out) return CSA_EINVAL;
  if (total_new > 0 && !j.new_raw) return CSA_EINVAL;
  if (j.total_entries > 0 && !j.gate_logits) return CSA_EINVAL;
  if (j.raw_dtype != CSA_F32 && j.raw_dtype != CSA_BF16) return CSA_ENOTSUP;
  if (!(j.eps >= 0.f) || !(j.rope_base > 0.f)) return CSA_EINVAL;
  if (!cache_ok(j.state, 256, -1)) return CSA_EINVAL;
  const int dim = j.state->dim;
  if (j.state->dtype != j.raw_dtype) return CSA_EINVAL;
  if (!cache_ok(j.out, 256 / j.ratio, dim)) return CSA_EINVAL;
  if (j.swa && !cache_ok(j.swa, 256, dim)) return CSA_EINVAL;
  if (j.swa && j.swa->dtype == CSA_FP4_E2M1) return CSA_ENOTSUP;
  if (dim < 2 || dim > 1024 || (dim & 1)) return CSA_ENOTSUP;
  if (j.rope_dims < 2 || (j.rope_dims & 1) || j.rope_dims > dim || j.rope_dims > 128) return CSA_EINVAL;
  (void)batch;
  *job = csa::CompressJob{j.ratio, j.new_raw, j.raw_dtype, j.cu_entries, j.total_entries,
                          j.gate_logits, j.gamma, j.eps, j.rope_base, j.rope_dims, j.state,
                          j.out, j.swa};
  return CSA_OK;
}

// Validates a compressor call and fills *L; *work = its workgroup count.
static int compress_prepare(int batch, const int32_t* ctx_lens, const int32_t* cu_new, int total_new,
                            int num_jobs, const csa_compress_job* jobs, csa::CompressLaunch* L,
                            int64_t* work) {
  if (batch <= 0 || total_new < 0 || !ctx_lens || !cu_new) return CSA_EINVAL;
  if (num_jobs < 1 || num_jobs > csa::kMaxCompressJobs || !jobs) return CSA_EINVAL;
  *L = csa::CompressLaunch{};
  L->batch = batch;
  L->ctx_lens = ctx_lens;
  L->cu_new = cu_new;
  L->total_new = total_new;
  L->num_jobs = num_jobs;
  *work = 0;
  for (int i = 0; i < num_jobs; ++i) {
    const int st = compress_job_check(jobs[i], batch, total_new, &L->jobs[i]);
    if (st != CSA_OK) return st;
    *work += (int64_t)jobs[i].total_entries + total_new;
  }
  if (*work > 0x7FFFFFFF) return CSA_ENOTSUP;
  return CSA_OK;
}

int csa_compress_insert_many(csa_stream_t stream, int batch, const int32_t* ctx_lens,
                             const int32_t* cu_new, int total_new, int num_jobs,
                             const csa_compress_job* jobs) {
  csa::CompressLaunch L;
  int64_t work = 0;
  const int st = compress_prepare(batch, ctx_lens, cu_new, total_new, num_jobs, jobs, &L, &work);
  if (st != CSA_OK || work == 0) return st;
  return hip_status(csa::launch_compress(L, (hipStream_t)stream));
}

int csa_compress_insert(csa_stream_t stream, int ratio, int batch, const int32_t* ctx_lens,
                        const int32_t* cu_new, int total_new, const void* new_raw, int raw_dtype,
                        const int32_t* cu_entries, int total_entries, const float* gate_logits,
                        const float* gamma, float eps, float rope_base, int rope_dims,
                        const csa_cache* state, const csa_cache* out, const csa_cache* swa) {
  const csa_compress_job job{ratio,      new_raw, raw_dtype, cu_entries, total_entries, gate_logits,
                             gamma,      eps,     rope_base, rope_dims,  state,         out,
                             swa};
  return csa_compress_insert_many(stream, batch, ctx_lens, cu_new, total_new, 1, &job);
}

size_t csa_index_workspace_size(int total_q, int max_context, int k) {
  if (total_q <= 0 || max_context <= 0 || k <= 0) return 0;
  return csa::index_workspace_bytes(total_q, max_context, k);
}

// ws_queries: how many queries the workspace must hold (the whole call, or one for
// csa_index_topk, which takes the queries in slices that fit)
static int index_check(int batch, const int32_t* cu_q, const int32_t* q_pos, int total_q,
                       int max_context, int k, size_t ws_bytes, const void* ws, int ws_queries) {
  if (batch <= 0 || total_q < 0 || !cu_q) return CSA_EINVAL;
  if (total_q > 0 && !q_pos) return CSA_EINVAL;
  if (max_context <= 0 || max_context > kMaxContextIndex) return CSA_EINVAL;
  if (k <= 0 || k > 65536) return CSA_EINVAL;
  if (total_q > 0 && (!ws || ws_bytes < csa::index_workspace_bytes(ws_queries, max_context, k)))
    return CSA_EWORKSPACE;
  return CSA_OK;
}

// (q_idx and head_w may be NULL when total_q = 0: zero-length arrays are never read)
static int score_check(int total_q, const void* q_idx, int q_dtype, int n_heads_idx,
                       const float* head_w, const csa_cache* idx_cache) {
  if (total_q > 0 && (!q_idx || !head_w)) return CSA_EINVAL;
  if (!cache_ok(idx_cache, 64, 128)) return CSA_EINVAL;
  if (q_dtype == CSA_BF16) {
    if (n_heads_idx < 1 || n_heads_idx > 64) return CSA_ENOTSUP;
    if (idx_cache->dtype == CSA_F32) return CSA_ENOTSUP;
  } else if (q_dtype == CSA_F32) {
    if (n_heads_idx < 1) return CSA_EINVAL;
  } else {
    return CSA_ENOTSUP;
  }
  return CSA_OK;
}

int csa_index_score(csa_stream_t stream, int batch, const int32_t* cu_q, const int32_t* q_pos,
                    int total_q, int max_context, const void* q_idx, int q_dtype, int n_heads_idx,
                    const float* head_w, const csa_cache* idx_cache, int k, void* workspace,
                    size_t workspace_bytes) {
  int st = index_check(batch, cu_q, q_pos, total_q, max_context, k, workspace_bytes, workspace, total_q);
  if (st != CSA_OK) return st;
  st = score_check(total_q, q_idx, q_dtype, n_heads_idx, head_w, idx_cache);
  if (st != CSA_OK || total_q == 0) return st;
  csa::IndexLaunch L{batch, cu_q, q_pos, total_q, max_context, q_idx, q_dtype, n_heads_idx,
                     head_w, idx_cache, k};
  const csa::IndexWorkspace ws = csa::index_workspace_carve(workspace, total_q, max_context, k);
  return hip_status(csa::launch_index_score(L, ws, (hipStream_t)stream));
}

int csa_index_select(csa_stream_t stream, int batch, const int32_t* cu_q, const int32_t* q_pos,
                     int total_q, int max_context, int k, int32_t* topk_idx, float* topk_score,
                     void* workspace, size_t workspace_bytes) {
  int st = index_check(batch, cu_q, q_pos, total_q, max_context, k, workspace_bytes, workspace, total_q);
  if (st != CSA_OK) return st;
  if (total_q == 0) return CSA_OK;
  if (!topk_idx) return CSA_EINVAL;
  csa::IndexLaunch L{batch, cu_q, q_pos, total_q, max_context, nullptr, 0, 0, nullptr, nullptr, k};
  const csa::IndexWorkspace ws = csa::index_workspace_carve(workspace, total_q, max_context, k);
  return hip_status(csa::launch_index_select(L, topk_idx, topk_score, ws, (hipStream_t)stream));
}

int csa_index_topk(csa_stream_t stream, int batch, const int32_t* cu_q, const int32_t* q_pos,
                   int total_q, int max_context, const void* q_idx, int q_dtype, int n_heads_idx,
                   const float* head_w, const csa_cache* idx_cache, int k, int32_t* topk_idx,
                   float* topk_score, void* workspace, size_t workspace_bytes) {
  int st = index_check(batch, cu_q, q_pos, total_q, max_context, k, workspace_bytes, workspace,
                       total_q > 0 ? 1 : 0);
  if (st != CSA_OK) return st;
  st = score_check(total_q, q_idx, q_dtype, n_heads_idx, head_w, idx_cache);
  if (st != CSA_OK) return st;
  if (total_q == 0) return CSA_OK;
  if (!topk_idx) return CSA_EINVAL;
  // the most queries whose workspace fits (the size grows with the query count)
  int slice = total_q;
  if (workspace_bytes < csa::index_workspace_bytes(total_q, max_context, k)) {
    int lo = 1, hi = total_q - 1;
    while (lo < hi) {
      const int mid = lo + (hi - lo + 1) / 2;
      if (csa::index_workspace_bytes(mid, max_context, k) <= workspace_bytes) lo = mid;
      else hi = mid - 1;
    }
    slice = lo;
  }
  const size_t q_row = (size_t)n_heads_idx * 128 * (q_dtype == CSA_BF16 ? 2 : 4);
  for (int q0 = 0; q0 < total_q; q0 += slice) {
    const int n = std::min(slice, total_q - q0);
    csa::IndexLaunch L{batch, cu_q, q_pos + q0, n, max_context, (const char*)q_idx + q0 * q_row, q_dtype,
                       n_heads_idx, head_w + (int64_t)q0 * n_heads_idx, idx_cache, k, q0};
    const csa::IndexWorkspace ws = csa::index_workspace_carve(workspace, n, max_context, k);
    hipError_t e = csa::launch_index_score(L, ws, (hipStream_t)stream);
    if (e != hipSuccess) return CSA_EHIP;
    e = csa::launch_index_select(L, topk_idx + (int64_t)q0 * k, topk_score ? topk_score + (int64_t)q0 * k : nullptr,
                                 ws, (hipStream_t)stream);
    if (e != hipSuccess) return CSA_EHIP;
  }
  return CSA_OK;
}

// One launch for csa_compress_index_score when the entry scoring stays small: every new indexer
// key is scored by its compressor workgroup for each query of its sequence (bf16 queries, at
// most 64 indexer heads, ratio-4 jobs, at most 4,096 (new entry, query) pairs).
static bool single_launch(int num_jobs, const csa_compress_job* jobs, int idx_job, int64_t work,
                          int total_q, int q_dtype, int n_heads_idx) {
  bool fuse = work > 0 && total_q > 0 && q_dtype == CSA_BF16 && n_heads_idx <= 64 &&
              (int64_t)jobs[idx_job].total_entries * total_q <= 4096;
  for (int i = 0; i < num_jobs; ++i) fuse = fuse && jobs[i].ratio == 4;
  return fuse;
}

int csa_compress_index_score_launches(int num_jobs, const csa_compress_job* jobs, int idx_job,
                                      int total_new, int total_q, int q_dtype, int n_heads_idx) {
  if (num_jobs < 1 || num_jobs > csa::kMaxCompressJobs || !jobs || idx_job < 0 ||
      idx_job >= num_jobs || total_new < 0 || total_q < 0)
    return CSA_EINVAL;
  int64_t work = 0;
  for (int i = 0; i < num_jobs; ++i) work += (int64_t)jobs[i].total_entries + total_new;
  if (single_launch(num_jobs, jobs, idx_job, work, total_q, q_dtype, n_heads_idx)) return 1;
  return (work > 0 ? 1 : 0) + (total_q > 0 ? 1 : 0);
}

int csa_compress_index_score(csa_stream_t stream, int batch, const int32_t* ctx_lens,
                             const int32_t* cu_new, int total_new, int num_jobs,
                             const csa_compress_job* jobs, int idx_job, const int32_t* cu_q,
                             const int32_t* q_pos, int total_q, int max_context, const void* q_idx,
                             int q_dtype, int n_heads_idx, const float* head_w,
                             const csa_cache* idx_cache, int k, void* workspace,
                             size_t workspace_bytes) {
  csa::CompressLaunch CL;
  int64_t work = 0;
  int st = compress_prepare(batch, ctx_lens, cu_new, total_new, num_jobs, jobs, &CL, &work);
  if (st != CSA_OK) return st;
  if (idx_job < 0 || idx_job >= num_jobs) return CSA_EINVAL;
  st = index_check(batch, cu_q, q_pos, total_q, max_context, k, workspace_bytes, workspace, total_q);
  if (st != CSA_OK) return st;
  st = score_check(total_q, q_idx, q_dtype, n_heads_idx, head_w, idx_cache);
  if (st != CSA_OK) return st;
  const csa_compress_job& ij = jobs[idx_job];
  if (ij.ratio != 4 || ij.out->rows != idx_cache->rows || ij.out->dtype != idx_cache->dtype ||
      ij.out->block_table != idx_cache->block_table)
    return CSA_EINVAL;
  const hipStream_t s = (hipStream_t)stream;
  if (total_q == 0) return work == 0 ? CSA_OK : hip_status(csa::launch_compress(CL, s));
  const bool fuse = single_launch(num_jobs, jobs, idx_job, work, total_q, q_dtype, n_heads_idx);
  csa::IndexLaunch L{batch, cu_q, q_pos, total_q, max_context, q_idx, q_dtype, n_heads_idx,
                     head_w, idx_cache, k};
  const csa::IndexWorkspace ws = csa::index_workspace_carve(workspace, total_q, max_context, k);
  if (fuse) return hip_status(csa::launch_compress_index_score(L, ws, CL, idx_job, s));
  hipError_t e = work > 0 ? csa::launch_compress(CL, s) : hipSuccess;
  if (e != hipSuccess) return CSA_EHIP;
  return hip_status(csa::launch_index_score(L, ws, s));
}

size_t csa_sparse_attn_workspace_size(int total_q, int n_heads, int dim, int ratio, int has_topk,
                                      int k, int max_context, int window) {
  if (total_q <= 0 || n_heads <= 0 || dim <= 0 || (ratio != 4 && ratio != 128) || max_context <= 0 ||
      window < 0)
    return 0;
  // the larger of the two kernels' plans (the dtypes are not arguments here)
  const csa::AttnPlan p = csa::attn_plan(total_q, n_heads, ratio, has_topk, k, max_context, window,
                                         csa::kAttnRowsCapFp8);
  const csa::AttnPlan p2 = csa::attn_plan(total_q, n_heads, ratio, has_topk, k, max_context, window,
                                          csa::kAttnRowsCapGeneric);
  if (p.max_rows > csa::kAttnMaxRows) return 0;
  return std::max(csa::attn_workspace_bytes(total_q, n_heads, dim, p),
                  csa::attn_workspace_bytes(total_q, n_heads, dim, p2));
}

int csa_q_norm_rope_swa(csa_stream_t stream, int total_q, const int32_t* q_pos, const void* q_in,
                        void* q_out, int q_dtype, int n_heads, int dim, const float* q_gamma,
                        float eps, float rope_base, int rope_dims, int batch,
                        const int32_t* ctx_lens, const int32_t* cu_new, int total_new,
                        const void* new_raw, int raw_dtype, const csa_cache* swa) {
  if (total_q < 0 || n_heads < 1) return CSA_EINVAL;
  if (q_dtype != CSA_F32 && q_dtype != CSA_BF16) return CSA_ENOTSUP;
  if (dim < 8 || dim > 1024 || (dim & 7)) return CSA_ENOTSUP;
  if (rope_dims < 8 || (rope_dims & 7) || rope_dims > dim || rope_dims > 128) return CSA_EINVAL;
  if (!(eps >= 0.f) || !(rope_base > 0.f)) return CSA_EINVAL;
  if (total_q > 0 && (!q_pos || !q_in || !q_out)) return CSA_EINVAL;
  if (swa) {
    if (batch < 1 || total_new < 0 || !ctx_lens || !cu_new) return CSA_EINVAL;
    if (raw_dtype != CSA_F32 && raw_dtype != CSA_BF16) return CSA_ENOTSUP;
    if (total_new > 0 && !new_raw) return CSA_EINVAL;
    if (!cache_ok(swa, 256, dim)) return CSA_EINVAL;
    if (swa->dtype == CSA_FP4_E2M1) return CSA_ENOTSUP;
  }
  csa::QNormLaunch L{};
  L.total_q = total_q;
  L.q_pos = q_pos;
  L.q_in = q_in;
  L.q_out = q_out;
  L.q_dtype = q_dtype;
  L.n_heads = n_heads;
  L.dim = dim;
  L.q_gamma = q_gamma;
  L.eps = eps;
  L.rope_base = rope_base;
  L.rope_dims = rope_dims;
  L.batch = batch;
  L.ctx_lens = ctx_lens;
  L.cu_new = cu_new;
  L.total_new = swa ? total_new : 0;
  L.new_raw = new_raw;
  L.raw_dtype = raw_dtype;
  L.swa = swa;
  return hip_status(csa::launch_q_norm_rope_swa(L, (hipStream_t)stream));
}

// Shared by the float32, fp8 output and no-allocation entry points (static_scratch: the
// library's own device array instead of the caller's workspace).
static int sparse_attn(csa_stream_t stream, int batch, const int32_t* cu_q, const int32_t* q_pos,
                       int total_q, int max_context, const void* q, int q_dtype, int n_heads,
                       const csa_cache* kv, int ratio, const int32_t* topk_idx, int k,
                       const csa_cache* swa, int window, float softmax_scale, float rope_base,
                       int rope_dims, float* out, float* lse, uint8_t* out_fp8, float* out_scales,
                       void* workspace, size_t workspace_bytes, bool static_scratch = false) {
  if (ratio != 4 && ratio != 128) return CSA_EINVAL;
  if (batch <= 0 || total_q < 0 || !cu_q) return CSA_EINVAL;
  if (total_q > 0 && (!q_pos || !q)) return CSA_EINVAL;  // zero-length arrays may be NULL
  if (total_q > 0 && !out && !out_fp8) return CSA_EINVAL;
  if (total_q > 0 && out_fp8 && !out_scales) return CSA_EINVAL;
  if (max_context <= 0 || window < 0 || window > 4096) return CSA_EINVAL;
  if (topk_idx && (k <= 0 || k > 65536)) return CSA_EINVAL;
  if (!cache_ok(kv, 256 / ratio, -1) || !cache_ok(swa, 256, kv->dim)) return CSA_EINVAL;
  if (kv->dtype != swa->dtype || kv->dtype == CSA_FP4_E2M1) return CSA_ENOTSUP;
  if (kv->dim != 576 && kv->dim != 512) return CSA_ENOTSUP;
  if (q_dtype != CSA_BF16 && q_dtype != CSA_F32) return CSA_ENOTSUP;
  if (n_heads < 1 || n_heads > 128) return CSA_ENOTSUP;
  if (rope_dims != 64) return CSA_ENOTSUP;
  if (!(rope_base > 0.f)) return CSA_EINVAL;
  if (total_q == 0) return CSA_OK;
  const int has_topk = topk_idx != nullptr;
  const csa::AttnPlan p =
      csa::attn_plan(total_q, n_heads, ratio, has_topk, has_topk ? k : 0, max_context, window,
                     csa::attn_rows_cap(kv->dtype, q_dtype));
  if (p.max_rows > csa::kAttnMaxRows) return CSA_ENOTSUP;
  const size_t need = csa::attn_workspace_bytes(total_q, n_heads, kv->dim, p);
  if (static_scratch) {  // the no-allocation entry point
    if (need > csa::kAttnStaticScratchBytes) return CSA_EWORKSPACE;
    hipError_t e = hipSuccess;
    workspace = csa::attn_static_scratch(&e);
    if (!workspace) return CSA_EHIP;
    workspace_bytes = csa::kAttnStaticScratchBytes;
  }
  if (!workspace || workspace_bytes < need) return CSA_EWORKSPACE;
  csa::AttnLaunch L{batch, cu_q, q_pos, total_q, max_context, q, q_dtype, n_heads, kv, ratio,
                    topk_idx, has_topk ? k : 0, swa, window, softmax_scale, rope_base, rope_dims,
                    out, lse, out_fp8, out_scales};
  return hip_status(csa::launch_sparse_attn(L, p, workspace, (hipStream_t)stream));
}

int csa_sparse_attn_decode(csa_stream_t stream, int batch, const int32_t* cu_q,
                           const int32_t* q_pos, int total_q, int max_context, const void* q,
                           int q_dtype, int n_heads, const csa_cache* kv, int ratio,
                           const int32_t* topk_idx, int k, const csa_cache* swa, int window,
                           float softmax_scale, float rope_base, int rope_dims, float* out,
                           float* lse, void* workspace, size_t workspace_bytes) {
  if (total_q > 0 && !out) return CSA_EINVAL;
  return sparse_attn(stream, batch, cu_q, q_pos, total_q, max_context, q, q_dtype, n_heads, kv,
                     ratio, topk_idx, k, swa, window, softmax_scale, rope_base, rope_dims, out,
                     lse, nullptr, nullptr, workspace, workspace_bytes);
}

int csa_sparse_attn_decode_noalloc(csa_stream_t stream, int batch, const int32_t* cu_q,
                                   const int32_t* q_pos, int total_q, int max_context,
                                   const void* q, int q_dtype, int n_heads,
                                   const csa_cache* kv, int ratio, const int32_t* topk_idx, int k,
                                   const csa_cache* swa, int window, float softmax_scale,
                                   float rope_base, int rope_dims, float* out, float* lse) {
  if (total_q > 0 && !out) return CSA_EINVAL;
  return sparse_attn(stream, batch, cu_q, q_pos, total_q, max_context, q, q_dtype, n_heads, kv,
                     ratio, topk_idx, k, swa, window, softmax_scale, rope_base, rope_dims, out,
                     lse, nullptr, nullptr, nullptr, 0, true);
}

int csa_sparse_attn_decode_fp8(csa_stream_t stream, int batch, const int32_t* cu_q,
                               const int32_t* q_pos, int total_q, int max_context, const void* q,
                               int q_dtype, int n_heads, const csa_cache* kv, int ratio,
                               const int32_t* topk_idx, int k, const csa_cache* swa, int window,
                               float softmax_scale, float rope_base, int rope_dims,
                               uint8_t* out_fp8, float* out_scales, float* out, float* lse,
                               void* workspace, size_t workspace_bytes) {
  if (total_q > 0 && (!out_fp8 || !out_scales)) return CSA_EINVAL;
  return sparse_attn(stream, batch, cu_q, q_pos, total_q, max_context, q, q_dtype, n_heads, kv,
                     ratio, topk_idx, k, swa, window, softmax_scale, rope_base, rope_dims, out,
                     lse, out_fp8, out_scales, workspace, workspace_bytes);
}

}  // extern "C"
