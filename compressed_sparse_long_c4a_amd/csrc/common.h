// Device helpers shared by the kernels of libcsa (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "csa.h"

namespace csa {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Device-side copy of a csa_cache descriptor (passed to kernels by value).  rows_per_block is
// a power of two (2, 64 or 256) and is kept as its log2 so paged addressing needs no division.
struct DevCache {
  void* rows;
  float* scales;  // float32 per row (fp8) or uint8 E8M0 per 16 values (fp4)
  const int32_t* bt;
  int32_t dtype, dim, rpb_shift, bt_stride;
};

inline int log2_exact(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

inline DevCache to_dev(const csa_cache* c) {
  DevCache d{};
  if (!c) return d;
  d.rows = c->rows;
  d.scales = (float*)c->scales;  // fp4 caches: uint8 E8M0 bytes, read through a cast
  d.bt = c->block_table;
  d.dtype = c->dtype;
  d.dim = c->dim;
  d.rpb_shift = log2_exact(c->rows_per_block);
  d.bt_stride = c->bt_stride;
  return d;
}

// Physical row index of logical row r of sequence b: block_table[b][r / rpb] * rpb + r % rpb
// (256-position logical blocks; 64 or 2 compressed entries, or 256 raw rows, per block).
__device__ __forceinline__ int64_t phys_row(const DevCache& c, int b, int64_t r) {
  const int32_t blk = c.bt[(int64_t)b * c.bt_stride + (int32_t)(r >> c.rpb_shift)];
  return ((int64_t)blk << c.rpb_shift) + (r & ((1 << c.rpb_shift) - 1));
}

// theta_i = rope_base^(-2i/rope_dims) for i < rope_dims/2, computed on the host in float64.
struct RopeTable {
  double theta[64];
};

// (the last table is kept per host thread: a decode loop asks for the same one every call)
inline RopeTable make_rope_table(float base, int rope_dims) {
  thread_local float last_base = 0.f;
  thread_local int last_dims = -1;
  thread_local RopeTable last{};
  if (rope_dims == last_dims && base == last_base) return last;
  RopeTable t{};
  for (int i = 0; i < rope_dims / 2 && i < 64; ++i)
    t.theta[i] = std::pow((double)base, -2.0 * (double)i / (double)rope_dims);
  last = t;
  last_base = base;
  last_dims = rope_dims;
  return t;
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

// Same as seq_of with one round trip for batch <= 64: every lane of the calling wave loads
// one prefix sum (unconditionally, so the load needs no branch and never waits alone) and a
// ballot finds the last sequence starting at or before i.  Split in two so that a kernel can
// issue the load with its other first loads: seq_load, then seq_pick on its value.
__device__ __forceinline__ int seq_load(const int32_t* cu, int batch) {
  return cu[min((int)(threadIdx.x & 63), batch - 1)];
}
__device__ __forceinline__ int seq_pick(const int32_t* cu, int batch, int i, int loaded) {
  if (batch > 64) return seq_of(cu, batch, i);
  const int lane = threadIdx.x & 63;
  const unsigned long long m = __ballot(lane < batch && loaded <= i);
  return m ? 63 - __clzll(m) : 0;
}
__device__ __forceinline__ int seq_of_wave(const int32_t* cu, int batch, int i) {
  return seq_pick(cu, batch, i, seq_load(cu, batch));
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

// Eight OCP E4M3 codes (two words) to eight bfloat16 values; exact (every E4M3 value is a
// bfloat16 value), two codes per conversion instruction.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ float fp8_to_f32(uint8_t c) {
  auto v = __builtin_amdgcn_cvt_pk_f32_fp8((uint32_t)c, false);
  return v[0];
}

// float32 -> OCP E4M3 code, round to nearest even.  Callers keep |x| <= 448.
__device__ __forceinline__ uint8_t f32_to_fp8(float x) {
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false) & 0xFF);
}

// ---- FP4: OCP E2M1 codes (sign, 2 exponent bits, 1 mantissa bit; values 0, 0.5, 1, 1.5, 2,
// 3, 4, 6), two per byte with the lower element in the low nibble, and E8M0 block scales.

// E8M0 scale byte s (1..254) as the float32 2^(s - 127): s is the float's exponent field.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) { return __uint_as_float(s << 23); }

// Eight E2M1 codes (one word, element 2i in the low nibble of byte i) times `scale` (a power of
// two) as eight bfloat16 values; exact.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t w, float scale) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Eight E2M1 codes (one word, as above) times `scale` as float32; exact.
__device__ __forceinline__ void fp4x8_to_f32(uint32_t w, float scale, float* x) {
  const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 0);
  const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 1);
  const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 2);
  const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 3);
  x[0] = v0[0]; x[1] = v0[1]; x[2] = v1[0]; x[3] = v1[1];
  x[4] = v2[0]; x[5] = v2[1]; x[6] = v3[0]; x[7] = v3[1];
}

// float32 -> E2M1 code: nearest value, ties to the even code, saturating at 6; -0 and values
// that round to 0 give code 0.  The seven midpoints between neighbouring magnitudes decide:
// a tie at 0.25, 1.25, 2.5 or 5 goes down (to an even code), at 0.75, 1.75 or 3.5 up.
__device__ __forceinline__ uint32_t f32_to_fp4(float x) {
  const float a = fabsf(x);
  const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return m | ((x < 0.f && m) ? 8u : 0u);
}

// Exponent k of the smallest power-of-two scale with amax / 2^k <= 6, for amax > 0: with
// amax = f * 2^e (f in [0.5, 1)), 6 * 2^k = 0.75 * 2^(k + 3), so k = e - 3, plus one when
// f > 0.75.  Clamped to the E8M0 bytes 1..254 (k in [-126, 127]).
__device__ __forceinline__ int fp4_scale_exp(float amax) {
  int e;
  const float f = frexpf(amax, &e);
  return min(max(e - 3 + (f > 0.75f ? 1 : 0), -126), 127);
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

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations, not for its
// outstanding global loads (which __syncthreads() would drain), so prefetched loads stay in
// flight across the barrier.  Use only where the barrier protects LDS data.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------- cross-lane operations
// Reductions and scans inside a wave use DPP lane moves and the gfx950 permlane swaps (VALU
// instructions), not ds_bpermute: a wave-wide sum costs a few cycles per step instead of an LDS
// round trip.  Every lane of the wave must be active.

__device__ __forceinline__ uint32_t as_u32(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ uint32_t as_u32(uint32_t v) { return v; }
__device__ __forceinline__ uint32_t as_u32(int v) { return (uint32_t)v; }
template <typename T> __device__ __forceinline__ T from_u32(uint32_t v) { return __builtin_bit_cast(T, v); }

// Value of lane (l xor 16) and of lane (l xor 32) combined by op over the four 16-lane rows:
// every lane gets op over lanes {l mod 16 + 16 r}.  (permlane16_swap pairs rows 0-1 and 2-3,
// permlane32_swap the halves; with both operands equal, op of the two results is the pairwise
// combination in every lane.)
template <typename T, typename Op>
__device__ __forceinline__ T rows_reduce(T v, Op op) {
  const auto a = __builtin_amdgcn_permlane16_swap(as_u32(v), as_u32(v), false, false);
  v = op(from_u32<T>(a[0]), from_u32<T>(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(as_u32(v), as_u32(v), false, false);
  return op(from_u32<T>(b[0]), from_u32<T>(b[1]));
}

// Four row sums at once: lane (l mod 16, row r) gets the sum of v_r over the four 16-lane rows
// at lane l mod 16 (three swaps and three adds, where four rows_reduce calls take eight and
// eight).  permlane16_swap(x, y) leaves x = [x0 y0 x2 y2] and y = [x1 y1 x3 y3] (by rows), so
// x + y holds the row pairs (0, 1) and (2, 3) of both; permlane32_swap(a, b) leaves
// a = [a0 a1 b0 b1] and b = [a2 a3 b2 b3], and a + b completes the sums.
__device__ __forceinline__ float rows_sum4(float v0, float v1, float v2, float v3) {
  const auto p = __builtin_amdgcn_permlane16_swap(as_u32(v0), as_u32(v1), false, false);
  const float a = from_u32<float>(p[0]) + from_u32<float>(p[1]);  // [v0 01, v1 01, v0 23, v1 23]
  const auto q = __builtin_amdgcn_permlane16_swap(as_u32(v2), as_u32(v3), false, false);
  const float b = from_u32<float>(q[0]) + from_u32<float>(q[1]);  // [v2 01, v3 01, v2 23, v3 23]
  const auto r = __builtin_amdgcn_permlane32_swap(as_u32(a), as_u32(b), false, false);
  return from_u32<float>(r[0]) + from_u32<float>(r[1]);
}

// DPP move of src within 16-lane rows (lanes without a source read 0).
template <int CTRL, typename T>
__device__ __forceinline__ T dpp(T v) {
  return from_u32<T>(__builtin_amdgcn_update_dpp(0u, as_u32(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within 8
constexpr int kDppRowMirror = 0x140;   // lane i <-> 15 - i within 16
template <int N> constexpr int kDppRowShr = 0x110 + N;

// op over the whole wave; every lane gets the result.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, dpp<kDppQuadXor1>(v));
  v = op(v, dpp<kDppQuadXor2>(v));
  v = op(v, dpp<kDppHalfMirror>(v));
  v = op(v, dpp<kDppRowMirror>(v));
  return rows_reduce(v, op);
}

__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float x, float y) { return x + y; });
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce(v, [](uint32_t x, uint32_t y) { return min(x, y); });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce(v, [](uint32_t x, uint32_t y) { return max(x, y); });
}

// Inclusive prefix sum over the wave (lane order).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp<kDppRowShr<1>>(x);
  x += dpp<kDppRowShr<2>>(x);
  x += dpp<kDppRowShr<4>>(x);
  x += dpp<kDppRowShr<8>>(x);
  const int t0 = __builtin_amdgcn_readlane(x, 15);
  const int t1 = __builtin_amdgcn_readlane(x, 31);
  const int t2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row > 0 ? t0 : 0) + (row > 1 ? t1 : 0) + (row > 2 ? t2 : 0);
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
  const int incl = wave_incl_scan(v);
  __syncthreads();
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += sh[i];
  *total = sh[0] + sh[1] + sh[2] + sh[3];
  return base + incl - v;
}

// cos/sin of the RoPE angle position * theta: the product is formed in float64 and reduced to
// [-pi, pi] there (|angle| reaches ~1e6 at 1M positions, where float32 would be off by ~0.05 rad),
// then the reduced angle is evaluated in float32.
__device__ __forceinline__ void rope_cos_sin(double position, double theta, float& c, float& s) {
  const double two_pi = 6.283185307179586476925286766559;
  const double x = position * theta;
  const double r = x - two_pi * rint(x * (1.0 / two_pi));
  sincosf((float)r, &s, &c);
}

// A load through a global-memory address (device memory): emitted as a global load, never a
// flat one.  Flat loads also count against the LDS wait counter, so an LDS-only wait (as in
// barrier_lds) would wait for them too.
__device__ __forceinline__ uint4 load_global16(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = *(const __attribute__((address_space(1))) u32x4*)p;
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace csa
