// backup_rows: device -> host copy of KV rows (gfx950).
//
// P3 "vllm 分析（十二）——Hisparse下篇", "数据 back up": the worker turns page transfers into
// per-cache source slots and host destination rows and launches a multi-layer backup op
// that copies those rows from the device cache into the pinned host cache; an event marks
// completion.  P1 "hiSparse-MTP", "3. HiSparse staging": the prefill KV is backed up to the
// host pool asynchronously and the request decodes once that event has fired.
//
// The copy is a zero-copy scatter: every thread reads 16-byte chunks of source rows from
// HBM and writes them with write-through vector stores straight into the pinned host cache
// through its device mapping.  Chunks are numbered (layer, entry, chunk of row) so that consecutive
// lanes write consecutive 16 bytes of one host row and a wave's stores form whole lines
// on the host link.  Each thread keeps kUnroll chunk loads in flight before it stores.

#include <algorithm>

#include "ops.h"

namespace hs {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int kMaxBlocks = 2048;

__global__ __launch_bounds__(kThreads) void backup_rows_kernel(
    const uint8_t *__restrict__ dev_cache, int64_t dev_layer_rows, uint8_t *__restrict__ host_cache,
    int64_t host_layer_rows, int32_t row_bytes, const int32_t *__restrict__ src_slots,
    int32_t src_per_layer, const int32_t *__restrict__ dst_rows, int32_t num_rows,
    int32_t src_block_size, int32_t src_block_stride, int64_t total_chunks) {
  const int chunks = row_bytes >> 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < total_chunks;
       base += stride) {
    // Two phases, every load of a phase issued before any result is used and none behind a
    // branch (the compiler would wait for each before the next): the entries' slot and row
    // indices, then the rows' chunks.  Out-of-range positions are clamped and not stored.
    int src[kUnroll], drow[kUnroll], layer[kUnroll], part[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = min(base + (int64_t)u * kThreads, total_chunks - 1);
      const int64_t r = c / chunks;  // (layer, entry) pair
      part[u] = (int)(c - r * chunks);
      layer[u] = (int)(r / num_rows);
      const int i = (int)(r - (int64_t)layer[u] * num_rows);
      src[u] = src_slots[(src_per_layer ? (int64_t)layer[u] * num_rows : 0) + i];
      drow[u] = dst_rows[i];
    }
    i32x4 v[kUnroll];
    int64_t dst[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int sl = src[u], d = drow[u];
      bool ok = base + (int64_t)u * kThreads < total_chunks && sl >= 0 && d >= 0 &&
                d < host_layer_rows;
      const int64_t p = ok ? (int64_t)(sl / src_block_size) * src_block_stride + sl % src_block_size : 0;
      ok = ok && p < dev_layer_rows;
      v[u] = *reinterpret_cast<const i32x4 *>(
          dev_cache + ((int64_t)layer[u] * dev_layer_rows + (ok ? p : 0)) * row_bytes + part[u] * 16);
      dst[u] = ok ? ((int64_t)layer[u] * host_layer_rows + d) * row_bytes + part[u] * 16 : -1;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (dst[u] >= 0) store_through16(host_cache + dst[u], v[u]);
  }
}

}  // namespace

hipError_t launch_backup_rows(const void *dev_cache, int64_t dev_layer_rows, void *host_cache_dev,
                              int64_t host_layer_rows, int32_t num_layers, int32_t row_bytes,
                              const int32_t *src_slots, int32_t src_per_layer,
                              const int32_t *dst_rows, int32_t num_rows, int32_t src_block_size,
                              int32_t src_block_stride, hipStream_t stream) {
  const int64_t total = (int64_t)num_layers * num_rows * (row_bytes >> 4);
  const int64_t per_block = (int64_t)kThreads * kUnroll;
  const int blocks = (int)std::min<int64_t>((total + per_block - 1) / per_block, kMaxBlocks);
  hipLaunchKernelGGL(backup_rows_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint8_t *>(dev_cache), dev_layer_rows,
                     static_cast<uint8_t *>(host_cache_dev), host_layer_rows, row_bytes, src_slots,
                     src_per_layer, dst_rows, num_rows, src_block_size, src_block_stride, total);
  return hipGetLastError();
}

}  // namespace hs
