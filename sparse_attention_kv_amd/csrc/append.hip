// append_accepted: the draft model's context KV grows by the accepted prefix (gfx950).
//
// P2 "投机解码的 KV 流转：prefill 阶段 DFlash 也要吃下整个 prompt", ⑤: after the target has
// verified a round, the features of the accepted prefix only go through the draft model's
// context K/V branch and are appended to its context cache; ⑥ and the timeline table: the
// context then covers the confirmed positions except the newest token (the next anchor).
//
// One workgroup per request: rows 0..L of the request (wave-major verify rows) are copied
// with 16-byte accesses to positions ctx_len .. ctx_len + L through the request's block
// table, then ctx_len advances by L + 1.

#include "ops.h"

namespace hs {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void append_accepted_kernel(
    uint8_t *__restrict__ ctx_cache, int64_t ctx_rows, int32_t row_bytes,
    const int32_t *__restrict__ bt, int32_t bt_stride, int32_t block_size, int32_t phys_stride,
    int32_t *__restrict__ ctx_len, const uint8_t *__restrict__ new_rows,
    const int32_t *__restrict__ accept_len, int32_t num_reqs, int32_t rows_per_req) {
  const int b = blockIdx.x;
  const int L = min(max(accept_len[b], 0), rows_per_req - 1);
  const int base = ctx_len[b];
  const int chunks = row_bytes >> 4;
  const int total = (L + 1) * chunks;
  for (int c = threadIdx.x; c < total; c += kThreads) {
    const int r = c / chunks;
    const int part = c - r * chunks;
    const int64_t pos = (int64_t)base + r;
    if (pos < 0) continue;
    const int64_t page_idx = pos / block_size;
    if (page_idx >= bt_stride) continue;
    const int page = bt[(int64_t)b * bt_stride + page_idx];
    if (page < 0) continue;
    const int64_t row = (int64_t)page * phys_stride + (pos - page_idx * block_size);
    if (row >= ctx_rows) continue;
    const i32x4 v = *reinterpret_cast<const i32x4 *>(
        new_rows + ((int64_t)r * num_reqs + b) * row_bytes + part * 16);
    *reinterpret_cast<i32x4 *>(ctx_cache + row * row_bytes + part * 16) = v;
  }
  __syncthreads();  // every thread has read ctx_len[b]
  if (threadIdx.x == 0) ctx_len[b] = base + L + 1;
}

}  // namespace

hipError_t launch_append_accepted(void *ctx_cache, int64_t ctx_rows, int32_t row_bytes,
                                  const int32_t *bt, int32_t bt_stride, int32_t block_size,
                                  int32_t phys_stride, int32_t *ctx_len, const void *new_rows,
                                  const int32_t *accept_len, int32_t num_reqs,
                                  int32_t rows_per_req, hipStream_t stream) {
  hipLaunchKernelGGL(append_accepted_kernel, dim3(num_reqs), dim3(kThreads), 0, stream,
                     static_cast<uint8_t *>(ctx_cache), ctx_rows, row_bytes, bt, bt_stride,
                     block_size, phys_stride, ctx_len, static_cast<const uint8_t *>(new_rows),
                     accept_len, num_reqs, rows_per_req);
  return hipGetLastError();
}

}  // namespace hs
