// Query normalisation + RoPE, and the window keys: one launch, one wave per query head or new
// raw row.
//
// [vLLM-V4] section 3 part 2, third fusion (fused Q norm + KV RoPE + K insert): before the
// main attention, the queries and the uncompressed sliding-window keys only need elementwise
// work; one kernel does it with a static warp-to-head assignment, each warp handling one query
// head or one key head with no communication between warps.
//
// Wave w of the grid takes query head (w / H, w % H) for w < total_q * H, else new raw row
// w - total_q * H.  The dimensions before the rotated span are held as 8-element chunks, chunk
// c by lane c % 64 in slot c / 64 (at most two slots); the rotated span is held one pair
// (2i, 2i+1) per lane, so every lane evaluates at most one angle.  Query: n = x / sqrt(mean(x^2)
// + eps) * gamma (the sum of squares is a wave sum), then RoPE at the query position; written
// in the query dtype.  Key: RoPE_p(x) stored in the window cache (fp8: scale = amax / 448
// from a wave max, codes rounded to nearest even).  The rotation
// and the fp8 rounding are the compressor's, so either kernel writes the same window rows.
#include "common.h"
#include "launch.h"

namespace csa {
namespace {

constexpr int kSlots = 2;     // 8-element chunks per lane (dim <= 1024)
constexpr int kQWaves = 4;    // waves per workgroup

struct QArgs {
  int batch, total_q, n_heads, dim, rope_dims, q_dtype, total_new, raw_dtype;
  float eps;
  const int32_t* q_pos;
  const void* q_in;
  void* q_out;
  const float* gamma;
  const int32_t* ctx_lens;
  const int32_t* cu_new;
  const void* new_raw;
  DevCache swa;
  RopeTable rope;
};

// The 8 elements starting at element e of a row of `dt` (F32 or BF16) as float32.
__device__ __forceinline__ void load8(const void* row, int dt, int e, float (&x)[8]) {
  if (dt == CSA_BF16) {
    const uint4 v = *(const uint4*)((const uint16_t*)row + e);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *(const float4*)((const float*)row + e), b = *(const float4*)((const float*)row + e + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// The pair at element e of a row of `dt` (F32 or BF16) as float32.
__device__ __forceinline__ float2 load2(const void* row, int dt, int e) {
  if (dt == CSA_BF16) {
    const uint32_t v = *(const uint32_t*)((const uint16_t*)row + e);
    return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xFFFF0000u));
  }
  return *(const float2*)((const float*)row + e);
}

__device__ __forceinline__ void store2(void* row, int dt, int e, float2 v) {
  if (dt == CSA_BF16)
    *(uint32_t*)((uint16_t*)row + e) = (uint32_t)f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16);
  else
    *(float2*)((float*)row + e) = v;
}

// Pair i of the rotated span turned by `position`.
__device__ __forceinline__ float2 rope2(float2 v, int i, double position, const RopeTable& rt) {
  float c, s;
  rope_cos_sin(position, rt.theta[i], c, s);
  return make_float2(v.x * c - v.y * s, v.x * s + v.y * c);
}

__device__ __forceinline__ void store8(void* row, int dt, int e, const float (&x)[8]) {
  if (dt == CSA_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16_bits(x[2 * i]) | ((uint32_t)f32_to_bf16_bits(x[2 * i + 1]) << 16);
    *(uint4*)((uint16_t*)row + e) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *(float4*)((float*)row + e) = make_float4(x[0], x[1], x[2], x[3]);
    *(float4*)((float*)row + e + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
}

__global__ __launch_bounds__(64 * kQWaves) void q_norm_rope_swa_kernel(QArgs a) {
  const int lane = threadIdx.x & 63;
  const int w = (int)blockIdx.x * kQWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nq = a.total_q * a.n_heads;
  if (w >= nq + a.total_new) return;
  const int d = a.dim, r0 = d - a.rope_dims;  // the rotated span starts at element r0
  const int nchunk = r0 >> 3, npair = a.rope_dims >> 1;
  const bool has_pair = lane < npair;
  const int ep = r0 + 2 * lane;               // this lane's pair of the rotated span
  float x[kSlots][8];
  float2 xp = make_float2(0.f, 0.f);
  const bool is_q = w < nq;
  if (is_q) {
    const int qi = w / a.n_heads;
    const int esz = a.q_dtype == CSA_BF16 ? 2 : 4;
    const char* src = (const char*)a.q_in + (int64_t)w * d * esz;
    const double pos = (double)a.q_pos[qi];
    float ss = 0.f;
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      const int c = lane + 64 * sl;
      if (c < nchunk) {
        load8(src, a.q_dtype, 8 * c, x[sl]);
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(x[sl][i], x[sl][i], ss);
      }
    }
    if (has_pair) {
      xp = load2(src, a.q_dtype, ep);
      ss = fmaf(xp.x, xp.x, ss);
      ss = fmaf(xp.y, xp.y, ss);
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)d + a.eps);
    char* dst = (char*)a.q_out + (int64_t)w * d * esz;
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      const int c = lane + 64 * sl;
      if (c < nchunk) {
        const int e = 8 * c;
        float g[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
        if (a.gamma) load8(a.gamma, CSA_F32, e, g);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[sl][i] = x[sl][i] * inv * g[i];
        store8(dst, a.q_dtype, e, x[sl]);
      }
    }
    if (has_pair) {
      const float2 g = a.gamma ? *(const float2*)(a.gamma + ep) : make_float2(1.f, 1.f);
      const float2 n = make_float2(xp.x * inv * g.x, xp.y * inv * g.y);
      store2(dst, a.q_dtype, ep, rope2(n, lane, pos, a.rope));
    }
    return;
  }
  // ---- a new raw row: RoPE at its position, stored in the window cache
  const int r = w - nq;
  const int b = seq_of_wave(a.cu_new, a.batch, r);
  const int64_t p = (int64_t)a.ctx_lens[b] + (r - a.cu_new[b]);
  const int64_t prow = phys_row(a.swa, b, p);
  const int esz = a.raw_dtype == CSA_BF16 ? 2 : 4;
  const char* src = (const char*)a.new_raw + (int64_t)r * d * esz;
  float amax = 0.f;
#pragma unroll
  for (int sl = 0; sl < kSlots; ++sl) {
    const int c = lane + 64 * sl;
    if (c < nchunk) {
      load8(src, a.raw_dtype, 8 * c, x[sl]);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[sl][i]));
    }
  }
  if (has_pair) {
    xp = rope2(load2(src, a.raw_dtype, ep), lane, (double)p, a.rope);
    amax = fmaxf(amax, fmaxf(fabsf(xp.x), fabsf(xp.y)));
  }
  if (a.swa.dtype == CSA_FP8_E4M3) {
    amax = wave_max(amax);
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    uint8_t* dst = (uint8_t*)a.swa.rows + prow * d;
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      const int c = lane + 64 * sl;
      if (c < nchunk) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lo |= (uint32_t)f32_to_fp8(x[sl][i] / scale) << (8 * i);
          hi |= (uint32_t)f32_to_fp8(x[sl][4 + i] / scale) << (8 * i);
        }
        *(uint2*)(dst + 8 * c) = make_uint2(lo, hi);
      }
    }
    if (has_pair)
      *(uint16_t*)(dst + ep) = (uint16_t)(f32_to_fp8(xp.x / scale) | (f32_to_fp8(xp.y / scale) << 8));
    if (lane == 0) a.swa.scales[prow] = scale;
  } else {
    const int sz = a.swa.dtype == CSA_BF16 ? 2 : 4;
    char* dst = (char*)a.swa.rows + prow * d * sz;
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      const int c = lane + 64 * sl;
      if (c < nchunk) store8(dst, a.swa.dtype, 8 * c, x[sl]);
    }
    if (has_pair) store2(dst, a.swa.dtype, ep, xp);
  }
}

}  // namespace

hipError_t launch_q_norm_rope_swa(const QNormLaunch& L, hipStream_t stream) {
  QArgs a{};
  a.batch = L.batch;
  a.total_q = L.total_q;
  a.n_heads = L.n_heads;
  a.dim = L.dim;
  a.rope_dims = L.rope_dims;
  a.q_dtype = L.q_dtype;
  a.total_new = L.swa ? L.total_new : 0;
  a.raw_dtype = L.raw_dtype;
  a.eps = L.eps;
  a.q_pos = L.q_pos;
  a.q_in = L.q_in;
  a.q_out = L.q_out;
  a.gamma = L.q_gamma;
  a.ctx_lens = L.ctx_lens;
  a.cu_new = L.cu_new;
  a.new_raw = L.new_raw;
  a.swa = to_dev(L.swa);
  a.rope = make_rope_table(L.rope_base, L.rope_dims);
  const int64_t waves = (int64_t)a.total_q * a.n_heads + a.total_new;
  if (waves == 0) return hipSuccess;
  const int64_t wgs = (waves + kQWaves - 1) / kQWaves;
  hipLaunchKernelGGL(q_norm_rope_swa_kernel, dim3((unsigned)wgs), dim3(64 * kQWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace csa
