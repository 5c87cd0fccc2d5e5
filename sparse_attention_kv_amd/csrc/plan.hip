// apply_plan: fill follower caches from the leader's swap plan (gfx950).
//
// P3 "vllm 分析（十二）——Hisparse下篇", resolve_topk listing: a runtime with a leader applies
// the leader's plan instead of swapping on its own; the leader's swap_in produces the plan
// and can prefetch the followers.  The plan of one wave is the leader's hot index per entry
// plus each request's missed entries; a follower (another layer with the same slot
// assignment) needs only those rows copied from its own host pool into its own hot buffer.
//
// Grid (request, kSlices): the slices of a request split its (cache, miss, 16-byte chunk)
// work; each thread keeps kUnroll host-link loads in flight before it stores to HBM.

#include "ops.h"

namespace hs {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int kSlices = 8;

__global__ __launch_bounds__(kThreads) void apply_plan_kernel(
    uint8_t *__restrict__ hot_kv, const uint8_t *__restrict__ host_pool, int64_t host_rows,
    int32_t num_caches, int32_t num_reqs, int32_t capacity, int32_t row_bytes,
    const int32_t *__restrict__ wave_rows, int32_t topk, const int32_t *__restrict__ hot_idx,
    const int32_t *__restrict__ miss_count, const int32_t *__restrict__ miss_pos) {
  const int b = blockIdx.x;
  const int count = min(max(miss_count[b], 0), topk);
  const int chunks = row_bytes >> 4;
  const int64_t per_cache = (int64_t)count * chunks;
  const int64_t total = per_cache * num_caches;
  const int64_t hot_rows = (int64_t)num_reqs * capacity;
  const int64_t base_row = (int64_t)b * topk;
  const int64_t stride = (int64_t)kSlices * kThreads * kUnroll;
  for (int64_t base = (int64_t)blockIdx.y * kThreads * kUnroll + threadIdx.x; base < total;
       base += stride) {
    i32x4 v[kUnroll];
    int64_t dst[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t f = base + (int64_t)u * kThreads;
      dst[u] = -1;
      if (f < total) {
        const int c = (int)(f / per_cache);
        const int64_t rem = f - (int64_t)c * per_cache;
        const int m = (int)(rem / chunks);
        const int part = (int)(rem - (int64_t)m * chunks);
        const int e = miss_pos[base_row + m];
        if (e >= 0 && e < topk) {
          const int row = wave_rows[base_row + e];
          const int g = hot_idx[base_row + e];
          if (row >= 0 && row < host_rows && g >= 0 && g < hot_rows) {
            v[u] = *reinterpret_cast<const i32x4 *>(
                host_pool + ((int64_t)c * host_rows + row) * row_bytes + part * 16);
            dst[u] = ((int64_t)c * hot_rows + g) * row_bytes + part * 16;
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (dst[u] >= 0) *reinterpret_cast<i32x4 *>(hot_kv + dst[u]) = v[u];
  }
}

}  // namespace

hipError_t launch_apply_plan(void *hot_kv, const void *host_pool_dev, int64_t host_rows,
                             int32_t num_caches, int32_t num_reqs, int32_t capacity,
                             int32_t row_bytes, const int32_t *wave_rows, int32_t topk,
                             const int32_t *hot_idx, const int32_t *miss_count,
                             const int32_t *miss_pos, hipStream_t stream) {
  hipLaunchKernelGGL(apply_plan_kernel, dim3(num_reqs, kSlices), dim3(kThreads), 0, stream,
                     static_cast<uint8_t *>(hot_kv), static_cast<const uint8_t *>(host_pool_dev),
                     host_rows, num_caches, num_reqs, capacity, row_bytes, wave_rows, topk,
                     hot_idx, miss_count, miss_pos);
  return hipGetLastError();
}

}  // namespace hs
