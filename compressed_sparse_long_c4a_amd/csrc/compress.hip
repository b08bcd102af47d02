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
// Launch shape: one launch runs any number (<= kMaxCompressJobs) of compressor instances ("jobs") over
// the same new tokens -- a c4a layer's main-KV and indexer-key compressors together, say --
// with one 256-thread workgroup per emitted entry, then one per new raw row, job after job.
// Every task is latency-bound (a decode step emits at most one entry per sequence and job), so
// the kernel minimises dependent memory trips: the sequence tables (entry and token offsets,
// context lengths) are read in one trip alongside the inputs that need no lookup, then the
// block-table reads, then the rows.  Each thread owns the dimensions tid, tid+256, ... and the
// row is staged once in LDS for the pairwise rotation and the fp8 amax.
#include "compress_dev.h"

namespace csa {
namespace {

__global__ __launch_bounds__(256) void compress_kernel(CompressArgs a) {
  __shared__ CompressSmem<128> sm;
  compress_block<128>(a, blockIdx.x, sm);
}

}  // namespace

hipError_t launch_compress(const CompressLaunch& c, hipStream_t stream) {
  int blocks = 0;
  const CompressArgs a = make_compress_args(c, &blocks);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(compress_kernel, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace csa
