// resolve_topk: request-local top-k token positions -> physical KV rows (gfx950).
//
// P3 "vllm 分析（十二）——Hisparse下篇", HiSparseCacheHandle.resolve_topk listing: the
// fully-resident branch converts each row's top-k indices to global cache slots through
// the request's block table (block size, physical block stride) and can also return
// per-row valid counts.  P3 "数据 back up": block p spans rows p*block_size + offset.
//
// One workgroup per query row.  Consecutive lanes read consecutive int32 positions
// (coalesced); the block-table row of the request is small (<= 8 KB) and stays in L2.
// Output keeps -1 in place (no compaction); the valid count is a block reduction.

#include "common.h"

namespace hs {
namespace {

constexpr int kThreads = 256;

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
  for (int j = threadIdx.x; j < topk; j += kThreads) {
    const int t = in[j];
    int slot = -1;
    if (req_ok && t >= 0 && t < lim) {
      const int page_idx = t / block_size;
      if (page_idx < bt_stride) {
        const int page = bt[page_idx];
        if (page >= 0) {
          const int64_t s = (int64_t)page * physical_block_stride + (t - page_idx * block_size);
          slot = s < 0x7fffffffLL ? (int)s : -1;  // rows must fit int32; fail closed
        }
      }
    }
    out[j] = slot;
    count += slot >= 0;
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
