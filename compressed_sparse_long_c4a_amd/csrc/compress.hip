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
#include "common.h"
#include "launch.h"

namespace csa {
namespace {

constexpr int kMaxDim = 1024;
constexpr int kPerThread = kMaxDim / 256;

struct Args {
  int ratio, batch, W, coff, dim, rope_dims, total_entries, has_swa, raw_dtype;
  const int32_t* ctx_lens;
  const int32_t* cu_new;
  const void* new_raw;
  const int32_t* cu_entries;
  const float* logits;
  const float* gamma;
  float eps;
  double rope_base;
  DevCache state, out, swa;
};

__device__ __forceinline__ float load_raw(const void* base, int dtype, int64_t idx) {
  if (dtype == CSA_BF16) return bf16_bits_to_f32(((const uint16_t*)base)[idx]);
  return ((const float*)base)[idx];
}

// Rotate the last rope_dims entries of v_sh (consecutive pairs) by `position`.
__device__ void rope_lds(float* v_sh, int dim, int rope_dims, double position, double base) {
  const int i = threadIdx.x;
  if (i < rope_dims / 2) {
    float c, s;
    rope_cos_sin(position, i, rope_dims, base, c, s);
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

__global__ __launch_bounds__(256) void compress_kernel(Args a) {
  __shared__ float v_sh[kMaxDim];
  __shared__ float w_sh[128];
  __shared__ float red_sh[8];
  const int tid = threadIdx.x;
  const int dim = a.dim;

  if ((int)blockIdx.x < a.total_entries) {
    // ---- one compressed entry
    const int e = blockIdx.x;
    const int b = seq_of(a.cu_entries, a.batch, e);
    const int64_t L0 = a.ctx_lens[b];
    const int64_t j = L0 / a.ratio + (e - a.cu_entries[b]);
    const int64_t start = (int64_t)a.ratio * j - (int64_t)(a.coff - 1) * a.ratio;
    const int64_t anchor = (int64_t)a.ratio * j + a.ratio - 1;
    const int W = a.W;

    // w = softmax(logits of this entry)
    const float lg = (tid < W) ? a.logits[(int64_t)e * W + tid] : -INFINITY;
    const float mx = block_max256(lg, red_sh);
    const float ex = (tid < W) ? expf(lg - mx) : 0.f;
    const float den = block_sum256(ex, red_sh);
    if (tid < W) w_sh[tid] = ex / den;
    __syncthreads();

    // y = sum_r w_r x_r; positions below 0 hold 0, below L0 come from the state cache
    float y[kPerThread] = {0.f, 0.f, 0.f, 0.f};
    const int64_t new0 = a.cu_new[b];
    for (int r = 0; r < W; ++r) {
      const int64_t p = start + r;
      if (p < 0) continue;
      const float wr = w_sh[r];
      const void* base;
      int64_t row;
      if (p >= L0) {
        base = a.new_raw;
        row = new0 + (p - L0);
      } else {
        base = a.state.rows;
        row = phys_row(a.state, b, p);
      }
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) {
        const int d = tid + 256 * k;
        if (d < dim) y[k] = fmaf(wr, load_raw(base, a.raw_dtype, row * dim + d), y[k]);
      }
    }

    // n = y / sqrt(mean(y^2) + eps) * gamma
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) ss = fmaf(y[k], y[k], ss);
    ss = block_sum256(ss, red_sh);
    const float inv = 1.0f / sqrtf(ss / (float)dim + a.eps);
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int d = tid + 256 * k;
      if (d < dim) v_sh[d] = y[k] * inv * (a.gamma ? a.gamma[d] : 1.0f);
    }
    __syncthreads();
    rope_lds(v_sh, dim, a.rope_dims, (double)anchor, a.rope_base);
    __syncthreads();
    store_row(a.out, phys_row(a.out, b, j), v_sh, dim, red_sh);
  } else {
    // ---- one new raw row: state append (last W positions) and window row RoPE_p(x_p)
    const int r = blockIdx.x - a.total_entries;
    const int b = seq_of(a.cu_new, a.batch, r);
    const int64_t L0 = a.ctx_lens[b];
    const int64_t p = L0 + (r - a.cu_new[b]);
    const int64_t L1 = L0 + (a.cu_new[b + 1] - a.cu_new[b]);
    if (p >= L1 - a.W) {
      const int64_t prow = phys_row(a.state, b, p);
      if (a.raw_dtype == CSA_BF16) {
        const uint16_t* src = (const uint16_t*)a.new_raw + (int64_t)r * dim;
        uint16_t* dst = (uint16_t*)a.state.rows + prow * dim;
        for (int d = tid; d < dim; d += 256) dst[d] = src[d];
      } else {
        const float* src = (const float*)a.new_raw + (int64_t)r * dim;
        float* dst = (float*)a.state.rows + prow * dim;
        for (int d = tid; d < dim; d += 256) dst[d] = src[d];
      }
    }
    if (a.has_swa) {
      for (int d = tid; d < dim; d += 256) v_sh[d] = load_raw(a.new_raw, a.raw_dtype, (int64_t)r * dim + d);
      __syncthreads();
      rope_lds(v_sh, dim, a.rope_dims, (double)p, a.rope_base);
      __syncthreads();
      store_row(a.swa, phys_row(a.swa, b, p), v_sh, dim, red_sh);
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
  a.rope_base = (double)c.rope_base;
  a.state = to_dev(c.state);
  a.out = to_dev(c.out);
  a.swa = to_dev(c.swa);
  const int blocks = c.total_entries + c.total_new;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(compress_kernel, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace csa
