// C ABI entry points: argument validation, then kernel launches on the caller's stream.
// Validation never launches anything, so every error return leaves all buffers untouched.

#include <cstring>

#include "ops.h"

namespace hs {
int attn_f32_max_topk();
int attn_f32_max_d();
int finalize_max_rows_per_req();
}  // namespace hs

namespace {

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hs_status from_hip(hipError_t e) { return e == hipSuccess ? HS_OK : HS_ERR_HIP; }

// Device-visible address of a buffer the kernels will read/write directly: device memory
// as is, pinned host memory through its device mapping.  Pageable host memory is refused
// (a kernel touching it would fault).
hs_status device_view(const void *p, const void **out) {
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of the failed query
    return HS_ERR_INVALID_ARG;
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) {
    *out = p;
    return HS_OK;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer != nullptr) {
    *out = attr.devicePointer;
    return HS_OK;
  }
  return HS_ERR_INVALID_ARG;
}

// Attention sizes beyond the kernels' limits (rows x heads, keys per row).
inline bool attn_too_large(int32_t num_rows, int32_t num_heads, int32_t topk) {
  return static_cast<int64_t>(num_rows) * num_heads > hs::kMaxRowHeads || topk > hs::kMaxAttnTopk;
}

hs_status check_state(const hs_hot_state *st) {
  if (st == nullptr) return HS_ERR_INVALID_ARG;
  if (st->num_reqs <= 0 || st->capacity <= 0 || st->host_rows <= 0 || st->row_elems <= 0)
    return HS_ERR_INVALID_ARG;
  if (st->host_rows > 0x7fffffffLL) return HS_ERR_INVALID_ARG;
  if (st->dtype != HS_BF16 && st->dtype != HS_F32) return HS_ERR_INVALID_ARG;
  if (!st->slot_loc || !st->slot_stamp || !st->loc_to_hot || !st->hot_kv || !st->host_pool)
    return HS_ERR_INVALID_ARG;
  const int elem = st->dtype == HS_BF16 ? 2 : 4;
  if ((static_cast<int64_t>(st->row_elems) * elem) % 16 != 0) return HS_ERR_INVALID_ARG;
  if (static_cast<int64_t>(st->row_elems) * elem > hs::kMaxRowBytes) return HS_ERR_UNSUPPORTED;
  if (!aligned16(st->hot_kv) || !aligned16(st->host_pool)) return HS_ERR_INVALID_ARG;
  if (static_cast<int64_t>(st->num_reqs) * st->capacity > 0x7fffffffLL) return HS_ERR_INVALID_ARG;
  return HS_OK;
}

}  // namespace

extern "C" {

hs_status hs_resolve_topk(const int32_t *topk_pos, int32_t num_rows, int32_t topk,
                          const int32_t *req_id, const int32_t *causal_limit, int32_t num_reqs,
                          const int32_t *block_table, int32_t bt_stride, int32_t block_size,
                          int32_t physical_block_stride, int32_t *out_slots, int32_t *out_valid,
                          void *stream) {
  if (num_rows < 0 || topk <= 0 || num_reqs <= 0 || bt_stride <= 0 || block_size <= 0 ||
      physical_block_stride <= 0)
    return HS_ERR_INVALID_ARG;
  if (num_rows == 0) return HS_OK;
  if (!topk_pos || !req_id || !causal_limit || !block_table || !out_slots) return HS_ERR_INVALID_ARG;
  return from_hip(hs::launch_resolve_topk(topk_pos, num_rows, topk, req_id, causal_limit, num_reqs,
                                          block_table, bt_stride, block_size, physical_block_stride,
                                          out_slots, out_valid, static_cast<hipStream_t>(stream)));
}

hs_status hs_swap_in(const hs_hot_state *st, const int32_t *wave_rows, int32_t topk, int32_t tick,
                     int32_t *out_hot_idx, int32_t *out_miss_count, int32_t *out_miss_pos,
                     void *stream) {
  hs_status s = check_state(st);
  if (s != HS_OK) return s;
  if (topk <= 0 || !wave_rows || !out_hot_idx || !out_miss_count) return HS_ERR_INVALID_ARG;
  if (st->capacity > hs::kMaxCapacity) return HS_ERR_UNSUPPORTED;
  if (topk > st->capacity) return HS_ERR_CAPACITY;
  if (topk > hs::kMaxSwapTopk) return HS_ERR_UNSUPPORTED;
  const void *pool = nullptr;
  s = device_view(st->host_pool, &pool);
  if (s != HS_OK) return s;
  return from_hip(hs::launch_swap_in(*st, pool, wave_rows, topk, tick, out_hot_idx, out_miss_count,
                                     out_miss_pos, static_cast<hipStream_t>(stream)));
}

hs_status hs_backup_rows(const void *dev_cache, int64_t dev_layer_rows, void *host_cache,
                         int64_t host_layer_rows, int32_t num_layers, int32_t row_bytes,
                         const int32_t *src_slots, int32_t src_per_layer,
                         const int32_t *dst_rows, int32_t num_rows, int32_t src_block_size,
                         int32_t src_block_stride, void *stream) {
  if (num_rows < 0 || num_layers <= 0 || row_bytes <= 0 || row_bytes % 16 != 0 ||
      dev_layer_rows <= 0 || host_layer_rows <= 0 || src_block_size <= 0 || src_block_stride <= 0)
    return HS_ERR_INVALID_ARG;
  if (num_rows == 0) return HS_OK;
  if (!dev_cache || !host_cache || !src_slots || !dst_rows) return HS_ERR_INVALID_ARG;
  if (dev_layer_rows > 0x7fffffffLL || host_layer_rows > 0x7fffffffLL) return HS_ERR_INVALID_ARG;
  if (!aligned16(dev_cache) || !aligned16(host_cache)) return HS_ERR_INVALID_ARG;
  if (row_bytes > hs::kMaxRowBytes) return HS_ERR_UNSUPPORTED;
  const void *host_dev = nullptr;
  hs_status s = device_view(host_cache, &host_dev);
  if (s != HS_OK) return s;
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  if (hipPointerGetAttributes(&attr, host_cache) != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return HS_ERR_INVALID_ARG;  // the destination must be the pinned host cache
  }
  return from_hip(hs::launch_backup_rows(dev_cache, dev_layer_rows, const_cast<void *>(host_dev),
                                         host_layer_rows, num_layers, row_bytes, src_slots,
                                         src_per_layer, dst_rows, num_rows, src_block_size,
                                         src_block_stride, static_cast<hipStream_t>(stream)));
}

hs_status hs_apply_plan(void *hot_kv, const void *host_pool, int64_t host_rows,
                        int32_t num_caches, int32_t num_reqs, int32_t capacity, int32_t row_bytes,
                        const int32_t *wave_rows, int32_t topk, const int32_t *hot_idx,
                        const int32_t *miss_count, const int32_t *miss_pos, void *stream) {
  if (host_rows <= 0 || num_caches <= 0 || num_reqs <= 0 || capacity <= 0 || row_bytes <= 0 ||
      row_bytes % 16 != 0 || topk <= 0)
    return HS_ERR_INVALID_ARG;
  if (!hot_kv || !host_pool || !wave_rows || !hot_idx || !miss_count || !miss_pos)
    return HS_ERR_INVALID_ARG;
  if (host_rows > 0x7fffffffLL || static_cast<int64_t>(num_reqs) * capacity > 0x7fffffffLL)
    return HS_ERR_INVALID_ARG;
  if (!aligned16(hot_kv) || !aligned16(host_pool)) return HS_ERR_INVALID_ARG;
  if (row_bytes > hs::kMaxRowBytes) return HS_ERR_UNSUPPORTED;
  const void *pool = nullptr;
  hs_status s = device_view(host_pool, &pool);
  if (s != HS_OK) return s;
  return from_hip(hs::launch_apply_plan(hot_kv, pool, host_rows, num_caches, num_reqs, capacity,
                                        row_bytes, wave_rows, topk, hot_idx, miss_count, miss_pos,
                                        static_cast<hipStream_t>(stream)));
}

hs_status hs_append_accepted(void *ctx_cache, int64_t ctx_rows, int32_t row_bytes,
                             const int32_t *ctx_block_table, int32_t bt_stride,
                             int32_t block_size, int32_t physical_block_stride, int32_t *ctx_len,
                             const void *new_rows, const int32_t *accept_len, int32_t num_reqs,
                             int32_t rows_per_req, void *stream) {
  if (ctx_rows <= 0 || row_bytes <= 0 || row_bytes % 16 != 0 || bt_stride <= 0 ||
      block_size <= 0 || physical_block_stride <= 0 || num_reqs <= 0 || rows_per_req <= 0)
    return HS_ERR_INVALID_ARG;
  if (!ctx_cache || !ctx_block_table || !ctx_len || !new_rows || !accept_len)
    return HS_ERR_INVALID_ARG;
  if (ctx_rows > 0x7fffffffLL) return HS_ERR_INVALID_ARG;
  if (!aligned16(ctx_cache) || !aligned16(new_rows)) return HS_ERR_INVALID_ARG;
  if (row_bytes > hs::kMaxRowBytes || rows_per_req > (1 << 16)) return HS_ERR_UNSUPPORTED;
  return from_hip(hs::launch_append_accepted(ctx_cache, ctx_rows, row_bytes, ctx_block_table,
                                             bt_stride, block_size, physical_block_stride, ctx_len,
                                             new_rows, accept_len, num_reqs, rows_per_req,
                                             static_cast<hipStream_t>(stream)));
}

hs_status hs_attn_plan_info(int32_t num_rows, int32_t num_heads, int32_t d_qk, int32_t d_v,
                            int32_t topk, int32_t dtype, int32_t *heads_per_wg,
                            int32_t *splits) {
  return hs_attn_plan_info_cus(num_rows, num_heads, d_qk, d_v, topk, dtype, hs::kNumCUs,
                               heads_per_wg, splits);
}

hs_status hs_attn_plan_info_cus(int32_t num_rows, int32_t num_heads, int32_t d_qk, int32_t d_v,
                                int32_t topk, int32_t dtype, int32_t max_cus,
                                int32_t *heads_per_wg, int32_t *splits) {
  if (max_cus <= 0) return HS_ERR_INVALID_ARG;
  if (num_rows <= 0 || num_heads <= 0 || d_qk <= 0 || d_v <= 0 || topk <= 0)
    return HS_ERR_INVALID_ARG;
  if (dtype == HS_F32) {
    if (heads_per_wg) *heads_per_wg = 1;
    if (splits) *splits = 1;
    return HS_OK;
  }
  if (dtype != HS_BF16) return HS_ERR_INVALID_ARG;
  if (d_qk != 576 || d_v != 512 || num_heads % 32 != 0) return HS_ERR_UNSUPPORTED;
  if (attn_too_large(num_rows, num_heads, topk)) return HS_ERR_UNSUPPORTED;
  const hs::AttnPlan p = hs::plan_attn_bf16(num_rows, num_heads, topk, max_cus);
  if (heads_per_wg) *heads_per_wg = p.heads_per_wg;
  if (splits) *splits = p.splits;
  return HS_OK;
}

size_t hs_attn_workspace_bytes(int32_t num_rows, int32_t num_heads, int32_t d_qk, int32_t d_v,
                               int32_t topk, int32_t dtype) {
  if (dtype != HS_BF16 || num_rows <= 0 || topk <= 0 || num_heads <= 0 || num_heads % 32 != 0 ||
      d_qk != 576 || d_v != 512 || attn_too_large(num_rows, num_heads, topk))
    return 0;
  return hs::plan_attn_bf16(num_rows, num_heads, topk).workspace;
}

hs_status hs_sparse_decode_attn(const void *q, const void *kv, int64_t kv_rows,
                                const int32_t *indices, int32_t num_rows, int32_t num_heads,
                                int32_t d_qk, int32_t d_v, int32_t topk, float scale,
                                int32_t dtype, void *out, float *lse, void *workspace,
                                size_t workspace_bytes, void *stream) {
  return hs::sparse_decode_attn_checked(q, kv, kv_rows, indices, num_rows, num_heads, d_qk, d_v,
                                        topk, scale, dtype, out, lse, workspace, workspace_bytes,
                                        stream, hs::kNumCUs);
}

hs_status hs_sparse_decode_attn_cus(const void *q, const void *kv, int64_t kv_rows,
                                    const int32_t *indices, int32_t num_rows, int32_t num_heads,
                                    int32_t d_qk, int32_t d_v, int32_t topk, float scale,
                                    int32_t dtype, void *out, float *lse, void *workspace,
                                    size_t workspace_bytes, int32_t max_cus, void *stream) {
  if (max_cus <= 0) return HS_ERR_INVALID_ARG;
  return hs::sparse_decode_attn_checked(q, kv, kv_rows, indices, num_rows, num_heads, d_qk, d_v,
                                        topk, scale, dtype, out, lse, workspace, workspace_bytes,
                                        stream, max_cus);
}

}  // extern "C"

// Validation and launch of hs_sparse_decode_attn, shared with the entry point whose
// workspace is the library's own scratch array.
hs_status hs::sparse_decode_attn_checked(const void *q, const void *kv, int64_t kv_rows,
                                         const int32_t *indices, int32_t num_rows,
                                         int32_t num_heads, int32_t d_qk, int32_t d_v, int32_t topk,
                                         float scale, int32_t dtype, void *out, float *lse,
                                         void *workspace, size_t workspace_bytes, void *stream,
                                         int32_t max_cus) {
  if (num_rows < 0 || num_heads <= 0 || d_qk <= 0 || d_v <= 0 || topk <= 0 || kv_rows < 0)
    return HS_ERR_INVALID_ARG;
  if (dtype != HS_BF16 && dtype != HS_F32) return HS_ERR_INVALID_ARG;
  if (num_rows == 0) return HS_OK;
  if (!q || !kv || !indices || !out) return HS_ERR_INVALID_ARG;
  if (kv_rows > 0x7fffffffLL) return HS_ERR_INVALID_ARG;
  if (attn_too_large(num_rows, num_heads, topk)) return HS_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == HS_BF16) {
    if (d_qk != 576 || d_v != 512 || num_heads % 32 != 0) return HS_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(kv) || !aligned16(out)) return HS_ERR_INVALID_ARG;
    const hs::AttnPlan plan = hs::plan_attn_bf16(num_rows, num_heads, topk, max_cus);
    if (plan.workspace > 0 && (workspace == nullptr || workspace_bytes < plan.workspace ||
                               !aligned16(workspace)))
      return HS_ERR_INVALID_ARG;
    return from_hip(hs::launch_attn_bf16(q, kv, kv_rows, indices, num_rows, num_heads, topk, scale,
                                         out, lse, workspace, plan, nullptr, nullptr, st));
  }
  if (d_qk > hs::attn_f32_max_d() || d_v > d_qk || topk > hs::attn_f32_max_topk())
    return HS_ERR_UNSUPPORTED;
  return from_hip(hs::launch_attn_f32(static_cast<const float *>(q), static_cast<const float *>(kv),
                                      kv_rows, indices, num_rows, num_heads, d_qk, d_v, topk, scale,
                                      static_cast<float *>(out), lse, st));
}

extern "C" {

hs_status hs_sparse_decode_attn_paged(const void *q, const void *kv_pool, int64_t kv_rows,
                                      const int32_t *topk_pos, const int32_t *req_id,
                                      const int32_t *causal_limit, int32_t num_reqs,
                                      const int32_t *block_table, int32_t bt_stride,
                                      int32_t block_size, int32_t physical_block_stride,
                                      int32_t num_rows, int32_t num_heads, int32_t d_qk,
                                      int32_t d_v, int32_t topk, float scale, int32_t dtype,
                                      void *out, float *lse, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  if (num_rows < 0 || num_heads <= 0 || d_qk <= 0 || d_v <= 0 || topk <= 0 || kv_rows < 0 ||
      num_reqs <= 0 || bt_stride <= 0 || block_size <= 0 || physical_block_stride <= 0)
    return HS_ERR_INVALID_ARG;
  if (dtype != HS_BF16 && dtype != HS_F32) return HS_ERR_INVALID_ARG;
  if (num_rows == 0) return HS_OK;
  if (!q || !kv_pool || !topk_pos || !req_id || !causal_limit || !block_table || !out)
    return HS_ERR_INVALID_ARG;
  if (kv_rows > 0x7fffffffLL) return HS_ERR_INVALID_ARG;
  if (dtype != HS_BF16 || d_qk != 576 || d_v != 512 || num_heads % 32 != 0)
    return HS_ERR_UNSUPPORTED;
  if (attn_too_large(num_rows, num_heads, topk)) return HS_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(kv_pool) || !aligned16(out)) return HS_ERR_INVALID_ARG;
  const hs::AttnPlan plan = hs::plan_attn_bf16(num_rows, num_heads, topk);
  if (plan.workspace > 0 &&
      (workspace == nullptr || workspace_bytes < plan.workspace || !aligned16(workspace)))
    return HS_ERR_INVALID_ARG;
  const hs::PagedMap pg{req_id, causal_limit, block_table, num_reqs, bt_stride, block_size,
                        physical_block_stride};
  return from_hip(hs::launch_attn_bf16(q, kv_pool, kv_rows, topk_pos, num_rows, num_heads, topk,
                                       scale, out, lse, workspace, plan, &pg, nullptr,
                                       static_cast<hipStream_t>(stream)));
}

hs_status hs_sparse_decode_attn_mixed(const void *q, const void *kv_a, int64_t kv_a_rows,
                                      const int32_t *indices_a, const void *kv_b,
                                      int64_t kv_b_rows, const int32_t *indices_b,
                                      const int32_t *row_sel, int32_t num_rows, int32_t num_heads,
                                      int32_t d_qk, int32_t d_v, int32_t topk, float scale,
                                      int32_t dtype, void *out, float *lse, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  return hs_sparse_decode_attn_mixed_cus(q, kv_a, kv_a_rows, indices_a, kv_b, kv_b_rows,
                                         indices_b, row_sel, num_rows, num_heads, d_qk, d_v, topk,
                                         scale, dtype, out, lse, workspace, workspace_bytes,
                                         hs::kNumCUs, stream);
}

hs_status hs_sparse_decode_attn_mixed_cus(const void *q, const void *kv_a, int64_t kv_a_rows,
                                          const int32_t *indices_a, const void *kv_b,
                                          int64_t kv_b_rows, const int32_t *indices_b,
                                          const int32_t *row_sel, int32_t num_rows,
                                          int32_t num_heads, int32_t d_qk, int32_t d_v,
                                          int32_t topk, float scale, int32_t dtype, void *out,
                                          float *lse, void *workspace, size_t workspace_bytes,
                                          int32_t max_cus, void *stream) {
  if (max_cus <= 0) return HS_ERR_INVALID_ARG;
  if (num_rows < 0 || num_heads <= 0 || d_qk <= 0 || d_v <= 0 || topk <= 0 || kv_a_rows < 0 ||
      kv_b_rows < 0)
    return HS_ERR_INVALID_ARG;
  if (dtype != HS_BF16 && dtype != HS_F32) return HS_ERR_INVALID_ARG;
  if (dtype != HS_BF16) return HS_ERR_UNSUPPORTED;
  if (num_rows == 0) return HS_OK;
  if (!q || !kv_a || !indices_a || !kv_b || !indices_b || !row_sel || !out)
    return HS_ERR_INVALID_ARG;
  if (kv_a_rows > 0x7fffffffLL || kv_b_rows > 0x7fffffffLL) return HS_ERR_INVALID_ARG;
  if (d_qk != 576 || d_v != 512 || num_heads % 32 != 0) return HS_ERR_UNSUPPORTED;
  if (attn_too_large(num_rows, num_heads, topk)) return HS_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(kv_a) || !aligned16(kv_b) || !aligned16(out))
    return HS_ERR_INVALID_ARG;
  const hs::AttnPlan plan = hs::plan_attn_bf16(num_rows, num_heads, topk, max_cus);
  if (plan.workspace > 0 &&
      (workspace == nullptr || workspace_bytes < plan.workspace || !aligned16(workspace)))
    return HS_ERR_INVALID_ARG;
  const hs::AltSource alt{static_cast<const uint8_t *>(kv_b), kv_b_rows, indices_b, row_sel};
  return from_hip(hs::launch_attn_bf16(q, kv_a, kv_a_rows, indices_a, num_rows, num_heads, topk,
                                       scale, out, lse, workspace, plan, nullptr, &alt,
                                       static_cast<hipStream_t>(stream)));
}

hs_status hs_finalize_accepted(const hs_hot_state *st, const void *logits, int32_t vocab,
                               const int32_t *draft_ids, const void *new_kv, int32_t rows_per_req,
                               const int32_t *seq_len, const int32_t *block_table,
                               int32_t bt_stride, int32_t block_size, int32_t tick,
                               int32_t *out_argmax, int32_t *out_accept_len,
                               int32_t *out_next_token, void *stream) {
  hs_status s = check_state(st);
  if (s != HS_OK) return s;
  if ((logits != nullptr && vocab <= 0) || rows_per_req <= 0 || bt_stride <= 0 || block_size <= 0)
    return HS_ERR_INVALID_ARG;
  if (!draft_ids || !new_kv || !seq_len || !block_table || !out_argmax || !out_accept_len ||
      !out_next_token)
    return HS_ERR_INVALID_ARG;
  if (rows_per_req > st->capacity) return HS_ERR_INVALID_ARG;
  if (rows_per_req > hs::finalize_max_rows_per_req()) return HS_ERR_UNSUPPORTED;
  if (!aligned16(new_kv) || (logits != nullptr && !aligned16(logits))) return HS_ERR_INVALID_ARG;
  if (static_cast<int64_t>(st->num_reqs) * rows_per_req > 0x7fffffffLL) return HS_ERR_INVALID_ARG;
  const void *pool = nullptr;
  s = device_view(st->host_pool, &pool);
  if (s != HS_OK) return s;
  return from_hip(hs::launch_finalize(*st, pool, logits, vocab, draft_ids, new_kv, rows_per_req,
                                      seq_len, block_table, bt_stride, block_size, tick, out_argmax,
                                      out_accept_len, out_next_token,
                                      static_cast<hipStream_t>(stream)));
}

hs_status hs_greedy_argmax(const void *logits, int32_t rows, int32_t vocab, int32_t *out_argmax,
                           void *stream) {
  if (rows < 0 || vocab <= 0) return HS_ERR_INVALID_ARG;
  if (rows == 0) return HS_OK;
  if (!logits || !out_argmax || !aligned16(logits)) return HS_ERR_INVALID_ARG;
  return from_hip(hs::launch_argmax(logits, rows, vocab, out_argmax, static_cast<hipStream_t>(stream)));
}

hs_status hs_host_read(const void *host_src, void *dst, int64_t bytes, void *stream) {
  if (bytes < 0 || bytes % 16 != 0) return HS_ERR_INVALID_ARG;
  if (bytes == 0) return HS_OK;
  if (!host_src || !dst || !aligned16(host_src) || !aligned16(dst)) return HS_ERR_INVALID_ARG;
  const void *src_dev = nullptr;
  const hs_status s = device_view(host_src, &src_dev);
  if (s != HS_OK) return s;
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  if (hipPointerGetAttributes(&attr, host_src) != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return HS_ERR_INVALID_ARG;  // the source must be pinned host memory
  }
  return from_hip(hs::launch_host_read(src_dev, dst, bytes / 16, static_cast<hipStream_t>(stream)));
}

const char *hs_status_string(int32_t status) {
  switch (status) {
    case HS_OK: return "ok";
    case HS_ERR_INVALID_ARG: return "invalid argument";
    case HS_ERR_CAPACITY: return "top-k exceeds hot-buffer capacity";
    case HS_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case HS_ERR_HIP: return "HIP runtime error";
    case HS_ERR_SCRATCH: return "shape needs more workspace than the library's fixed scratch";
    default: return "unknown status";
  }
}

const char *hs_version(void) { return "hisparse-gfx950 0.1.0"; }

}  // extern "C"
