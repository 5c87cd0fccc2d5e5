// Launchers of the non-attention kernel families (gfx950 only); each returns hipSuccess or
// the launch error.
#pragma once

#include "common.h"

namespace hs {

// 16-byte vector store with the system-scope cache policy (sc0 sc1): written through to
// memory rather than held in L2 until the kernel-end writeback.  For stores into pinned host
// memory, where a held store otherwise crosses the host link only after the kernel's last
// instruction (measured: the finalize call's 280 host rows then cost ~4.5 us of tail).
__device__ __forceinline__ void store_through16(void *p, const i32x4 &v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" : : "v"(p), "v"(v) : "memory");
}

// Largest hot-buffer capacity the swap-in kernel's LDS arrays are sized for.
constexpr int kMaxCapacity = 16384;
// Largest top-k a swap-in call accepts (it is also bounded by the capacity); the
// per-entry LDS arrays of the swap-in kernel are sized by it.
constexpr int kMaxSwapTopk = 4096;

hipError_t launch_resolve_topk(const int32_t *topk_pos, int32_t num_rows, int32_t topk,
                               const int32_t *req_id, const int32_t *causal_limit,
                               int32_t num_reqs, const int32_t *block_table, int32_t bt_stride,
                               int32_t block_size, int32_t physical_block_stride,
                               int32_t *out_slots, int32_t *out_valid, hipStream_t stream);

hipError_t launch_swap_in(const hs_hot_state &st, const void *host_pool_dev,
                          const int32_t *wave_rows, int32_t topk, int32_t tick,
                          int32_t *out_hot_idx, int32_t *out_miss_count, int32_t *out_miss_pos,
                          hipStream_t stream);

// Argmax of each bf16 logit row (lowest index of the maximum, NaN never wins).
hipError_t launch_argmax(const void *logits, int32_t rows, int32_t vocab, int32_t *out_argmax,
                         hipStream_t stream);

// logits == nullptr: out_argmax already holds the rows' argmax (only kernel 2 runs).
hipError_t launch_finalize(const hs_hot_state &st, const void *host_pool_dev, const void *logits,
                           int32_t vocab, const int32_t *draft_ids, const void *new_kv,
                           int32_t rows_per_req, const int32_t *seq_len, const int32_t *block_table,
                           int32_t bt_stride, int32_t block_size, int32_t tick, int32_t *out_argmax,
                           int32_t *out_accept_len, int32_t *out_next_token, hipStream_t stream);

// Device -> host row backup; host_cache_dev is the pinned host cache's device address.
hipError_t launch_backup_rows(const void *dev_cache, int64_t dev_layer_rows, void *host_cache_dev,
                              int64_t host_layer_rows, int32_t num_layers, int32_t row_bytes,
                              const int32_t *src_slots, int32_t src_per_layer,
                              const int32_t *dst_rows, int32_t num_rows, int32_t src_block_size,
                              int32_t src_block_stride, hipStream_t stream);

// Follower caches from the leader's swap plan; host_pool_dev is the pinned pools' device address.
hipError_t launch_apply_plan(void *hot_kv, const void *host_pool_dev, int64_t host_rows,
                             int32_t num_caches, int32_t num_reqs, int32_t capacity,
                             int32_t row_bytes, const int32_t *wave_rows, int32_t topk,
                             const int32_t *hot_idx, const int32_t *miss_count,
                             const int32_t *miss_pos, hipStream_t stream);

// Accepted prefix appended to the draft model's context cache.
hipError_t launch_append_accepted(void *ctx_cache, int64_t ctx_rows, int32_t row_bytes,
                                  const int32_t *bt, int32_t bt_stride, int32_t block_size,
                                  int32_t phys_stride, int32_t *ctx_len, const void *new_rows,
                                  const int32_t *accept_len, int32_t num_reqs,
                                  int32_t rows_per_req, hipStream_t stream);

// hs_sparse_decode_attn's validation and launch (every argument as in the C ABI; max_cus
// as for hs_sparse_decode_attn_cus).
hs_status sparse_decode_attn_checked(const void *q, const void *kv, int64_t kv_rows,
                                     const int32_t *indices, int32_t num_rows, int32_t num_heads,
                                     int32_t d_qk, int32_t d_v, int32_t topk, float scale,
                                     int32_t dtype, void *out, float *lse, void *workspace,
                                     size_t workspace_bytes, void *stream, int32_t max_cus);

// Streaming zero-copy read of pinned host memory (host_src_dev: its device address) into
// device memory, chunks of 16 bytes; the host link's reference read rate.
hipError_t launch_host_read(const void *host_src_dev, void *dst, int64_t chunks, hipStream_t stream);

}  // namespace hs
