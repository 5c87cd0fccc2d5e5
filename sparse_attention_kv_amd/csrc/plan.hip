// apply_plan: fill follower caches from the leader's swap plan (gfx950).
//
// P3 "vllm 分析（十二）——Hisparse下篇", resolve_topk listing: a runtime with a leader applies
// the leader's plan instead of swapping on its own; the leader's swap_in produces the plan
// and can prefetch the followers.  The plan of one wave is the leader's hot index per entry
// plus each request's missed entries; a follower (another layer with the same slot
// assignment) needs only those rows copied from its own host pool into its own hot buffer.
//
// Grid (request, kSlices): the slices of a request split its (cache, miss, 16-byte chunk)
// work; each thread issues its kUnroll host-link loads together before it stores to HBM.

#include "ops.h"

namespace hs {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 2;  // more in flight measured slower (the host link saturates)
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
    // Three phases, every load of a phase issued before any result is used and none behind
    // a branch (the compiler would wait for each before the next): the missed entries, their
    // host rows and hot indices, then the rows' chunks.  Out-of-range positions are clamped
    // and not stored.
    int cache[kUnroll], part[kUnroll], e[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t f = min(base + (int64_t)u * kThreads, total - 1);
      cache[u] = (int)(f / per_cache);
      const int64_t rem = f - (int64_t)cache[u] * per_cache;
      const int m = (int)(rem / chunks);
      part[u] = (int)(rem - (int64_t)m * chunks);
      e[u] = miss_pos[base_row + m];
    }
    int row[kUnroll], g[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int ec = min(max(e[u], 0), topk - 1);
      row[u] = wave_rows[base_row + ec];
      g[u] = hot_idx[base_row + ec];
    }
    i32x4 v[kUnroll];
    int64_t dst[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bool ok = base + (int64_t)u * kThreads < total && e[u] >= 0 && e[u] < topk &&
                      row[u] >= 0 && row[u] < host_rows && g[u] >= 0 && g[u] < hot_rows;
      v[u] = *reinterpret_cast<const i32x4 *>(
          host_pool + ((int64_t)cache[u] * host_rows + (ok ? row[u] : 0)) * row_bytes + part[u] * 16);
      dst[u] = ok ? ((int64_t)cache[u] * hot_rows + g[u]) * row_bytes + part[u] * 16 : -1;
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
