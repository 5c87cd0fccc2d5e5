// resolve_topk: request-local top-k token positions -> physical KV rows (gfx950).
//
// P3 "vllm 分析（十二）——Hisparse下篇", HiSparseCacheHandle.resolve_topk listing: the
// fully-resident branch converts each row's top-k indices to global cache slots through
// the request's block table (block size, physical block stride) and can also return
// per-row valid counts.  P3 "数据 back up": block p spans rows p*block_size + offset.
//
// One 1024-thread workgroup per query row.  Consecutive lanes read consecutive int32
// positions (coalesced); a thread's position loads, then its block-table loads, are all
// issued before any result is used (none behind a branch), so a row costs about two memory
// round trips.  The
// block-table row of a request is small (<= 8 KB) and stays in L2.
// Output keeps -1 in place (no compaction); the valid count is a block reduction.

#include "ops.h"

namespace hs {
namespace {

constexpr int kThreads = 1024;
constexpr int kPer = 4;  // entries per thread per pass; all loads of a pass are issued first

__global__ __launch_bounds__(kThreads) void resolve_topk_kernel(
    const int32_t *__restrict__ topk_pos, int32_t topk, const int32_t *__restrict__ req_id,
    const int32_t *__restrict__ causal_limit, int32_t num_reqs,
    const int32_t *__restrict__ block_table, int32_t bt_stride, int32_t block_size,
    int32_t physical_block_stride, int32_t *__restrict__ out_slots,
    int32_t *__restrict__ out_valid) {
  __shared__ int wave_counts[kThreads / 64];
  const int row = blockIdx.x;
  const int b = req_id[row];
  const int lim = causal_limit[row];
  const bool req_ok = b >= 0 && b < num_reqs;
  const int32_t *in = topk_pos + (int64_t)row * topk;
  int32_t *out = out_slots + (int64_t)row * topk;
  const int32_t *bt = block_table + (int64_t)(req_ok ? b : 0) * bt_stride;

  int count = 0;
  for (int base = 0; base < topk; base += kThreads * kPer) {
    int t[kPer], page_idx[kPer], page[kPer];
    // No load sits behind a branch (the compiler would wait for each before the next):
    // indices are clamped into range and the results masked afterwards.
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = base + k * kThreads + threadIdx.x;
      const int tj = in[min(j, topk - 1)];
      t[k] = j < topk ? tj : -1;
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const bool ok = req_ok && t[k] >= 0 && t[k] < lim;
      page_idx[k] = ok ? t[k] / block_size : 0;
      const int raw = bt[min(page_idx[k], bt_stride - 1)];
      page[k] = raw | -static_cast<int>(!(ok && page_idx[k] < bt_stride));  // OR, not a select
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = base + k * kThreads + threadIdx.x;
      int slot = -1;
      if (page[k] >= 0) {
        const int64_t sl = (int64_t)page[k] * physical_block_stride + (t[k] - page_idx[k] * block_size);
        slot = sl < 0x7fffffffLL ? (int)sl : -1;  // rows must fit int32; fail closed
      }
      if (j < topk) out[j] = slot;
      count += slot >= 0;
    }
  }
  if (out_valid == nullptr) return;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) count += __shfl_xor(count, off, 64);
  if (lane_id() == 0) wave_counts[threadIdx.x / 64] = count;
  __syncthreads();
  if (threadIdx.x == 0) {
    int total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) total += wave_counts[w];
    out_valid[row] = total;
  }
}

}  // namespace

hipError_t launch_resolve_topk(const int32_t *topk_pos, int32_t num_rows, int32_t topk,
                               const int32_t *req_id, const int32_t *causal_limit,
                               int32_t num_reqs, const int32_t *block_table, int32_t bt_stride,
                               int32_t block_size, int32_t physical_block_stride,
                               int32_t *out_slots, int32_t *out_valid, hipStream_t stream) {
  hipLaunchKernelGGL(resolve_topk_kernel, dim3(num_rows), dim3(kThreads), 0, stream, topk_pos,
                     topk, req_id, causal_limit, num_reqs, block_table, bt_stride, block_size,
                     physical_block_stride, out_slots, out_valid);
  return hipGetLastError();
}

}  // namespace hs
