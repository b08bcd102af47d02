// Streaming-read probe (a measurement utility beside the method's kernels): every byte of a
// buffer is read once with 16-byte non-temporal loads, eight in flight per thread, 32
// workgroups per compute unit, and each workgroup writes the XOR of what it read, so the loads
// have a use.  (Measured over 2 GiB: plain loads with four in flight and 2,048 workgroups reach
// ~5.5 TB/s, these ~6.3 TB/s.)
#include "csa.h"
#include "common.h"

namespace csa {
namespace {

constexpr int kProbeWGs = 8192;  // 32 256-thread workgroups per compute unit
constexpr int kProbeThreads = 256;
constexpr int kProbeInFlight = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* buf, int64_t n16,
                                                                   uint32_t* sink) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* src = (const u32x4*)buf;
  __shared__ uint32_t red[kProbeThreads / 64];
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + (kProbeInFlight - 1) * stride < n16; i += kProbeInFlight * stride) {
    u32x4 v[kProbeInFlight];
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = src[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  acc = wave_reduce(acc, [](uint32_t x, uint32_t y) { return x ^ y; });
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace
}  // namespace csa

extern "C" {

int csa_read_probe_sink_words(void) { return csa::kProbeWGs; }

int csa_read_probe(csa_stream_t stream, const void* buf, size_t bytes, uint32_t* sink) {
  if (!buf || !sink || bytes == 0 || (bytes & 15) || ((uintptr_t)buf & 15)) return CSA_EINVAL;
  hipLaunchKernelGGL(csa::read_probe_kernel, dim3(csa::kProbeWGs), dim3(csa::kProbeThreads), 0,
                     (hipStream_t)stream, (const uint4*)buf, (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_EHIP;
}

}  // extern "C"
