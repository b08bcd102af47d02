// Fused compressor: weighted window sum -> RMSNorm -> RoPE -> paged insert, plus the rolling
// state append and the window-row write, in one launch.
//
// [vLLM-V4] section 3 part 2 (first fusion): compress, RMSNorm, RoPE and cache insertion are
// almost entirely elementwise and run as one kernel, with separate instances per head dim.
// [vLLM-V4] appendix, exact position ranges: c4a entry j covers raw positions [4j-4, 4j+3]
// (negative positions are 0) with RoPE at 4j+3; c128a entry j covers [128j, 128j+127] with
// RoPE at 128j+127; the group is combined first and rotated once at the anchor.
// [vLLM-V4] section 3 part 1: the compressor keeps the last coff*ratio raw rows per request as
// sliding-window state.
//
// Launch shape: one 256-thread workgroup per emitted entry, then one per new raw row.  Both
// kinds are latency-bound (a decode step emits at most one entry per sequence), so the kernel
// favours few passes over the row: each thread owns the dimensions tid, tid+256, ... and the
// row is staged once in LDS for the pairwise rotation and the fp8 amax.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace csa {
namespace {

constexpr int kMaxDim = 1024;
constexpr int kPerThread = kMaxDim / 256;
constexpr int kLdsBatch = 1024;  // sequences whose offsets are staged in LDS in one load
constexpr int64_t kNoRow = INT64_MIN;  // window slot at a negative position

struct Args {
  int ratio, batch, W, coff, dim, rope_dims, total_entries, has_swa, raw_dtype;
  const int32_t* ctx_lens;
  const int32_t* cu_new;
  const void* new_raw;
  const int32_t* cu_entries;
  const float* logits;
  const float* gamma;
  float eps;
  DevCache state, out, swa;
  RopeTable rope;
};

// Rotate the last rope_dims entries of v_sh (consecutive pairs) by `position`.
__device__ void rope_lds(float* v_sh, int dim, int rope_dims, double position, const RopeTable& rt) {
  const int i = threadIdx.x;
  if (i < rope_dims / 2) {
    float c, s;
    rope_cos_sin(position, rt.theta[i], c, s);
    const int d0 = dim - rope_dims + 2 * i;
    const float x0 = v_sh[d0], x1 = v_sh[d0 + 1];
    v_sh[d0] = x0 * c - x1 * s;
    v_sh[d0 + 1] = x0 * s + x1 * c;
  }
}

// Store the row staged in v_sh at physical row `prow` of cache c, rounded to its dtype.
// FP8 rows get scale = amax / 448 (1 for an all-zero row) and nearest-even codes of v / scale.
__device__ void store_row(const DevCache& c, int64_t prow, const float* v_sh, int dim,
                          float* red_sh) {
  const int tid = threadIdx.x;
  if (c.dtype == CSA_FP8_E4M3) {
    float amax = 0.f;
    for (int d = tid; d < dim; d += 256) amax = fmaxf(amax, fabsf(v_sh[d]));
    amax = block_max256(amax, red_sh);
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    uint8_t* dst = (uint8_t*)c.rows + prow * dim;
    for (int d = tid; d < dim; d += 256) dst[d] = f32_to_fp8(v_sh[d] / scale);
    if (tid == 0) c.scales[prow] = scale;
  } else if (c.dtype == CSA_BF16) {
    uint16_t* dst = (uint16_t*)c.rows + prow * dim;
    for (int d = tid; d < dim; d += 256) dst[d] = f32_to_bf16_bits(v_sh[d]);
  } else {
    float* dst = (float*)c.rows + prow * dim;
    for (int d = tid; d < dim; d += 256) dst[d] = v_sh[d];
  }
}

// Sequence owning flat index i (prefix sums cu[0..batch], staged in LDS when small enough).
__device__ __forceinline__ int seq_lookup(const int* cu_sh, const int32_t* cu, int batch, int i) {
  if (batch > kLdsBatch) return seq_of(cu, batch, i);
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_sh[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// RAW: dtype of the raw rows (CSA_BF16 or CSA_F32).  Every workgroup issues the loads that do
// not depend on its sequence before the sequence lookup, and all rows of a window at once, so
// a task costs about four dependent memory round trips: offsets, sequence length, block
// table, rows.
template <int RAW>
__global__ __launch_bounds__(256) void compress_kernel(Args a) {
  typedef typename std::conditional<RAW == CSA_BF16, uint16_t, float>::type Elem;
  constexpr int ESZ = sizeof(Elem);
  __shared__ float v_sh[kMaxDim];
  __shared__ float w_sh[128];
  // byte offset of window row r from new_raw (kNoRow: no row; a state row may lie below
  // new_raw, so offsets take either sign); addresses derived from a kernel argument compile to
  // global loads, whose waits do not drain LDS traffic
  __shared__ int64_t off_sh[128];
  __shared__ float red_sh[8];
  __shared__ int cu_sh[kLdsBatch + 1];
  const int tid = threadIdx.x;
  const int dim = a.dim;
  const int64_t row_bytes = (int64_t)dim * ESZ;
  const char* raw = (const char*)a.new_raw;
  const bool entry_task = (int)blockIdx.x < a.total_entries;
  auto to_f32 = [](Elem v) -> float {
    if constexpr (RAW == CSA_BF16) return bf16_bits_to_f32(v);
    else return v;
  };

  if (entry_task) {
    // ---- one compressed entry
    const int e = blockIdx.x;
    const int W = a.W;
    const float lg = (tid < W) ? a.logits[(int64_t)e * W + tid] : -INFINITY;
    float gm[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k)
      gm[k] = a.gamma ? a.gamma[min(tid + 256 * k, dim - 1)] : 1.0f;
    if (a.batch <= kLdsBatch)
      for (int i = tid; i <= a.batch; i += 256) cu_sh[i] = a.cu_entries[i];
    __syncthreads();
    const int b = seq_lookup(cu_sh, a.cu_entries, a.batch, e);
    const int64_t L0 = a.ctx_lens[b];
    const int n0 = a.cu_new[b];
    const int e0 = a.batch <= kLdsBatch ? cu_sh[b] : a.cu_entries[b];
    const int64_t j = L0 / a.ratio + (e - e0);
    const int64_t start = (int64_t)a.ratio * j - (int64_t)(a.coff - 1) * a.ratio;
    const int64_t anchor = (int64_t)a.ratio * j + a.ratio - 1;

    // window rows: positions below 0 hold no row, below L0 come from the state cache, the
    // rest are new rows of this sequence
    if (tid < W) {
      const int64_t p = start + tid;
      const int64_t state_off = (int64_t)((uintptr_t)a.state.rows - (uintptr_t)a.new_raw);
      int64_t off = kNoRow;
      if (p >= L0) off = (n0 + (p - L0)) * row_bytes;
      else if (p >= 0) off = state_off + phys_row(a.state, b, p) * row_bytes;
      off_sh[tid] = off;
    }
    const int64_t orow = phys_row(a.out, b, j);
    // w = softmax(logits of this entry)
    const float mx = block_max256(lg, red_sh);
    const float ex = (tid < W) ? expf(lg - mx) : 0.f;
    const float den = block_sum256(ex, red_sh);
    if (tid < W) w_sh[tid] = ex / den;
    __syncthreads();

    // y = sum_r w_r x_r, eight rows' loads in flight together (a missing row loads the first
    // new row, which exists whenever an entry is emitted, and is then discarded)
    float y[kPerThread] = {0.f, 0.f, 0.f, 0.f};
    for (int r0 = 0; r0 < W; r0 += 8) {
      Elem x[8][kPerThread];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t o = off_sh[r0 + u] == kNoRow ? 0 : off_sh[r0 + u];
#pragma unroll
        for (int k = 0; k < kPerThread; ++k)
          x[u][k] = *(const Elem*)(raw + o + (int64_t)min(tid + 256 * k, dim - 1) * ESZ);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool has = off_sh[r0 + u] != kNoRow;
        const float wr = w_sh[r0 + u];
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) y[k] = fmaf(wr, has ? to_f32(x[u][k]) : 0.f, y[k]);
      }
    }

    // n = y / sqrt(mean(y^2) + eps) * gamma
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) ss = tid + 256 * k < dim ? fmaf(y[k], y[k], ss) : ss;
    ss = block_sum256(ss, red_sh);
    const float inv = 1.0f / sqrtf(ss / (float)dim + a.eps);
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int d = tid + 256 * k;
      if (d < dim) v_sh[d] = y[k] * inv * gm[k];
    }
    __syncthreads();
    rope_lds(v_sh, dim, a.rope_dims, (double)anchor, a.rope);
    __syncthreads();
    store_row(a.out, orow, v_sh, dim, red_sh);
  } else {
    // ---- one new raw row: state append (last W positions) and window row RoPE_p(x_p)
    const int r = blockIdx.x - a.total_entries;
    Elem x[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k)
      x[k] = ((const Elem*)a.new_raw)[(int64_t)r * dim + min(tid + 256 * k, dim - 1)];
    if (a.batch <= kLdsBatch)
      for (int i = tid; i <= a.batch; i += 256) cu_sh[i] = a.cu_new[i];
    __syncthreads();
    const int b = seq_lookup(cu_sh, a.cu_new, a.batch, r);
    const int64_t L0 = a.ctx_lens[b];
    const int n0 = a.batch <= kLdsBatch ? cu_sh[b] : a.cu_new[b];
    const int n1 = a.batch <= kLdsBatch ? cu_sh[b + 1] : a.cu_new[b + 1];
    const int64_t p = L0 + (r - n0);
    const int64_t L1 = L0 + (n1 - n0);
    const bool append = p >= L1 - a.W;
    const int64_t srow = append ? phys_row(a.state, b, p) : 0;
    const int64_t wrow = a.has_swa ? phys_row(a.swa, b, p) : 0;
    if (append) {
      Elem* dst = (Elem*)a.state.rows + srow * dim;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
        if (tid + 256 * k < dim) dst[tid + 256 * k] = x[k];
    }
    if (a.has_swa) {
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
        if (tid + 256 * k < dim) v_sh[tid + 256 * k] = to_f32(x[k]);
      __syncthreads();
      rope_lds(v_sh, dim, a.rope_dims, (double)p, a.rope);
      __syncthreads();
      store_row(a.swa, wrow, v_sh, dim, red_sh);
    }
  }
}

}  // namespace

hipError_t launch_compress(const CompressLaunch& c, hipStream_t stream) {
  Args a{};
  a.ratio = c.ratio;
  a.batch = c.batch;
  a.coff = c.ratio == 4 ? 2 : 1;
  a.W = a.coff * c.ratio;
  a.dim = c.state->dim;
  a.rope_dims = c.rope_dims;
  a.total_entries = c.total_entries;
  a.has_swa = c.swa != nullptr;
  a.raw_dtype = c.raw_dtype;
  a.ctx_lens = c.ctx_lens;
  a.cu_new = c.cu_new;
  a.new_raw = c.new_raw;
  a.cu_entries = c.cu_entries;
  a.logits = c.logits;
  a.gamma = c.gamma;
  a.eps = c.eps;
  a.rope = make_rope_table(c.rope_base, c.rope_dims);
  a.state = to_dev(c.state);
  a.out = to_dev(c.out);
  a.swa = to_dev(c.swa);
  const int blocks = c.total_entries + c.total_new;
  if (blocks == 0) return hipSuccess;
  if (c.raw_dtype == CSA_BF16)
    hipLaunchKernelGGL(compress_kernel<CSA_BF16>, dim3(blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(compress_kernel<CSA_F32>, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace csa
