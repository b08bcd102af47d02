// Streaming-read probe (a measurement utility beside the method's kernels): every byte of a
// buffer is read once with 16-byte loads, four loads in flight per thread, and each workgroup
// writes the XOR of what it read, so the loads have a use.
#include "csa.h"
#include "common.h"

namespace csa {
namespace {

constexpr int kProbeWGs = 2048;  // eight 256-thread workgroups per compute unit
constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* buf, int64_t n16,
                                                                   uint32_t* sink) {
  __shared__ uint32_t red[kProbeThreads / 64];
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
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
