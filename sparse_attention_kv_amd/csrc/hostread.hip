// host_read: streaming zero-copy read of pinned host memory into device memory (gfx950).
//
// The reference rate of the host link for reads the GPU issues itself, next to a
// pinned -> device DMA copy.  The swap-in copy reads the pinned host pool the same way
// (16-byte loads through the pool's device mapping), but gathers 1152-byte rows; this
// kernel streams one contiguous range, so it measures what the link delivers to loads
// when nothing else limits them.  Every thread keeps kUnroll 16-byte loads in flight
// before it stores; consecutive lanes read consecutive 16 bytes.  Not a step of the path.

#include <algorithm>

#include "ops.h"

namespace hs {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int kMaxBlocks = 2048;

__global__ __launch_bounds__(kThreads) void host_read_kernel(const i32x4 *__restrict__ src,
                                                             i32x4 *__restrict__ dst,
                                                             int64_t chunks) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < chunks;
       base += stride) {
    i32x4 v[kUnroll];
    // every load of a round is issued before the first store; chunks past the end re-read
    // the last chunk (no branch around a load) and are not stored
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[min(base + (int64_t)u * kThreads, chunks - 1)];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = base + (int64_t)u * kThreads;
      if (c < chunks) dst[c] = v[u];
    }
  }
}

}  // namespace

hipError_t launch_host_read(const void *host_src_dev, void *dst, int64_t chunks, hipStream_t stream) {
  const int64_t per_block = (int64_t)kThreads * kUnroll;
  const int blocks = (int)std::min<int64_t>((chunks + per_block - 1) / per_block, kMaxBlocks);
  hipLaunchKernelGGL(host_read_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                     static_cast<const i32x4 *>(host_src_dev), static_cast<i32x4 *>(dst), chunks);
  return hipGetLastError();
}

}  // namespace hs
