// Copies between device memory and pinned host memory made by a kernel: the GPU's own
// loads (or stores) cross the link, so the copy takes no DMA engine and is not queued
// behind the window's large engine copies, with which it only shares the link.  Used for
// the block-boundary activations parked in host memory ("Poros" research post,
// training-step paragraph: the forward keeps the block boundaries for the backward).
#include <algorithm>

#include "internal.hpp"

namespace msq {
namespace {

constexpr int KCOPY_THREADS = 256;
constexpr int64_t KCOPY_MAX_BLOCKS = 256;  // enough loads in flight to fill the link

__global__ __launch_bounds__(KCOPY_THREADS) void kernel_copy_kernel(const uint4* __restrict__ src,
                                                                   uint4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * KCOPY_THREADS;
  for (int64_t i = (int64_t)blockIdx.x * KCOPY_THREADS + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

// Algorithmic bytes: each byte read once and written once.
hipError_t launch_kernel_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>(KCOPY_MAX_BLOCKS, (n16 + KCOPY_THREADS - 1) / KCOPY_THREADS);
  char shape[32];
  snprintf(shape, sizeof(shape), "%lld", (long long)bytes);
  return timed_launch("kernel_copy", shape, 0.0, 2.0 * bytes, kernel_copy_kernel, dim3((unsigned)blocks),
                      dim3(KCOPY_THREADS), s, (const uint4*)src, (uint4*)dst, n16);
}

}  // namespace msq
