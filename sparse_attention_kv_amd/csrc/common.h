// Internal declarations shared by the library's translation units (gfx950 only): vector
// types, the attention structs and launchers, small device helpers.  The other kernel
// families' launchers are in ops.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hisparse.h"

namespace hs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

#define HS_LDS __attribute__((address_space(3)))

// ---- size limits the entry points enforce (beyond them: HS_ERR_UNSUPPORTED) ----
constexpr int64_t kMaxRowBytes = 1 << 16;      // one KV row of any cache
constexpr int64_t kMaxRowHeads = 1 << 24;      // attention rows x heads per call
constexpr int32_t kMaxAttnTopk = 1 << 20;      // attention keys per row

// ---- attention launchers; return hipSuccess or the launch error ----
// Block-table description for attention that resolves top-k token positions itself
// (the fully resident batch); null = the indices are already KV rows.
struct PagedMap {
  const int32_t *req_id;        // [num_rows]
  const int32_t *causal_limit;  // [num_rows]
  const int32_t *block_table;   // [num_reqs, bt_stride]
  int32_t num_reqs, bt_stride, block_size, physical_block_stride;
};

// Second (cache, indices) source for attention over a mixed batch: a row with
// row_sel[row] != 0 reads alt kv rows through alt indices (per-request residency: resident
// requests read the paged pool, swapped requests the hot buffer).  row_sel == null: none.
struct AltSource {
  const uint8_t *kv;
  int64_t kv_rows;
  const int32_t *indices;  // [num_rows, topk]
  const int32_t *row_sel;  // [num_rows]
};

struct AttnPlan {
  int heads_per_wg;    // 128 (attn128_kernel), 64 (attn64_kernel) or 32 (attn_bf16_kernel)
  int splits;          // key splits per (row, head group); 1 = no combine pass
  int keys_per_split;  // multiple of the key tile
  size_t workspace;    // bytes
};
constexpr int kNumCUs = 256;  // compute units of the GPU (MI355X)
// Kernel and key splits for these sizes, sized for `max_cus` compute units (kNumCUs: the
// whole GPU; fewer leave the rest to a kernel running beside the call on another stream).
AttnPlan plan_attn_bf16(int32_t num_rows, int32_t num_heads, int32_t topk,
                        int32_t max_cus = kNumCUs);

hipError_t launch_attn_bf16(const void *q, const void *kv, int64_t kv_rows, const int32_t *indices,
                            int32_t num_rows, int32_t num_heads, int32_t topk, float scale,
                            void *out, float *lse, void *workspace, const AttnPlan &plan,
                            const PagedMap *paged, const AltSource *alt, hipStream_t stream);

hipError_t launch_attn64(const void *q, const void *kv, int64_t kv_rows, const int32_t *indices,
                         int32_t num_rows, int32_t num_heads, int32_t topk, float scale, void *out,
                         float *lse, void *workspace, const AttnPlan &plan, const PagedMap *paged,
                         const AltSource *alt, hipStream_t stream);

hipError_t launch_attn128(const void *q, const void *kv, int64_t kv_rows, const int32_t *indices,
                          int32_t num_rows, int32_t num_heads, int32_t topk, float scale, void *out,
                          float *lse, void *workspace, const AttnPlan &plan, const PagedMap *paged,
                          const AltSource *alt, hipStream_t stream);

hipError_t launch_attn_f32(const float *q, const float *kv, int64_t kv_rows, const int32_t *indices,
                           int32_t num_rows, int32_t num_heads, int32_t d_qk, int32_t d_v,
                           int32_t topk, float scale, float *out, float *lse, hipStream_t stream);

// ---- small device helpers ----
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// LDS-only barrier: waits for this wave's LDS traffic, then s_barrier.  Unlike
// __syncthreads(), whose release fence also waits for every outstanding global load and
// store, it publishes LDS data only; the wait and the barrier are one asm statement whose
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Exclusive prefix sum of `v` across the 64 lanes of a wave; `total` receives the sum.
__device__ __forceinline__ int wave_exclusive_scan(int v, int &total) {
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane_id() >= off) x += y;
  }
  total = __shfl(x, 63, 64);
  return x - v;
}

}  // namespace hs
