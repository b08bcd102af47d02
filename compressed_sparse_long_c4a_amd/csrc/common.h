// Device helpers shared by the kernels of libcsa (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Device-side copy of a csa_cache descriptor (passed to kernels by value).
struct DevCache {
  void* rows;
  float* scales;
  const int32_t* bt;
  int32_t dtype, dim, rpb, bt_stride;
};

inline DevCache to_dev(const csa_cache* c) {
  DevCache d{};
  if (!c) return d;
  d.rows = c->rows;
  d.scales = c->scales;
  d.bt = c->block_table;
  d.dtype = c->dtype;
  d.dim = c->dim;
  d.rpb = c->rows_per_block;
  d.bt_stride = c->bt_stride;
  return d;
}

// Physical row index of logical row r of sequence b: block_table[b][r / rpb] * rpb + r % rpb
// (256-position logical blocks; 64 or 2 compressed entries, or 256 raw rows, per block).
__device__ __forceinline__ int64_t phys_row(const DevCache& c, int b, int64_t r) {
  const int32_t blk = c.bt[(int64_t)b * c.bt_stride + (int32_t)(r / c.rpb)];
  return (int64_t)blk * c.rpb + (r % c.rpb);
}

// Sequence owning flat index i, given prefix sums cu[0..batch] (empty sequences allowed).
__device__ __forceinline__ int seq_of(const int32_t* cu, int batch, int i) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------- formats

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// Two OCP E4M3 codes (bytes 0,1 if !HI, bytes 2,3 if HI of w) to float32; exact.
template <bool HI>
__device__ __forceinline__ void fp8x2_to_f32(uint32_t w, float& a, float& b) {
  auto v = __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
  a = v[0];
  b = v[1];
}

__device__ __forceinline__ float fp8_to_f32(uint8_t c) {
  auto v = __builtin_amdgcn_cvt_pk_f32_fp8((uint32_t)c, false);
  return v[0];
}

// float32 -> OCP E4M3 code, round to nearest even.  Callers keep |x| <= 448.
__device__ __forceinline__ uint8_t f32_to_fp8(float x) {
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false) & 0xFF);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// Order-preserving map of float32 to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t f2key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Sum / max over a 256-thread block; every thread gets the result.  `sh` holds >= 4 floats.
__device__ __forceinline__ float block_sum256(float v, float* sh) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  return sh[0] + sh[1] + sh[2] + sh[3];
}
__device__ __forceinline__ float block_max256(float v, float* sh) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

// Exclusive prefix sum over a 256-thread block; returns this thread's offset, total in *total.
// `sh` holds >= 5 ints.
__device__ __forceinline__ int block_exscan256(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  __syncthreads();
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += sh[i];
  *total = sh[0] + sh[1] + sh[2] + sh[3];
  return base + incl - v;
}

// RoPE angle position * base^(-2i/rope_dims), formed and reduced in float64.
__device__ __forceinline__ void rope_cos_sin(double position, int i, int rope_dims, double base,
                                             float& c, float& s) {
  const double theta = pow(base, -2.0 * (double)i / (double)rope_dims);
  double sd, cd;
  sincos(position * theta, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace csa
