/*
 * hisparse.h -- C ABI of the MI355X (gfx950) HiSparse sparse-decode library.
 *
 * The path, per decode step and per query row (the decode anchor plus any draft rows
 * being verified):
 *
 *   hs_resolve_topk       request-local top-k token positions -> physical KV rows
 *   hs_swap_in            hit/miss split against the per-request hot buffer, LRU
 *                         victim choice, copy of the misses from the pinned host pool
 *   hs_sparse_decode_attn attention over only the selected latent KV rows
 *                         (_paged: positions resolved in the same call; _mixed: each
 *                         row reads one of two caches; _cus: planned for part of the
 *                         GPU, beside the next wave's swap-in)
 *   hs_finalize_accepted  greedy acceptance of the draft rows, then keep exactly the
 *                         target-verified prefix's KV (host pool + hot buffer)
 *
 * and around it:
 *
 *   hs_apply_plan         follower caches (other layers) take the leader's swap plan
 *   hs_backup_rows        device -> pinned host copy of new KV rows (staging, spills)
 *   hs_append_accepted    the draft model's context cache takes the accepted prefix
 *
 * Sources (web pages describing the method):
 *   P1  Notion page "hiSparse-MTP" -- summary (six-stage main line ending in accepted-KV
 *       finalize), "1. 启动阶段" (startup: the coordinator's device buffer, host
 *       pool, LRU slots and async stream; the core-state maps) and "3. HiSparse staging"
 *       (prefill KV backed up to the host pool, readiness by event).
 *   P2  blog post "投机解码的 KV 流转：prefill 阶段 DFlash 也要吃下整个 prompt" --
 *       worked example, sections ④ (target verify, greedy acceptance, kept KV), ⑤ (the
 *       draft model's context KV takes the accepted prefix) and ⑥.
 *   P3  CSDN post "vllm 分析（十二）——Hisparse下篇" -- HiSparseCacheHandle.resolve_topk
 *       listing (fully-resident conversion vs. swap-in), HiSparseHotSpec (fixed hot
 *       blocks per request), "数据 back up" (block-row address arithmetic, pinned host
 *       pool, the worker's backup transfers), reclaim_resident_blocks and
 *       build_offload_command (per-batch residency).
 *
 * Conventions for every call:
 *   - All pointers are caller-owned; the library allocates nothing and keeps no state
 *     (hs_sparse_decode_attn_noalloc's fixed scratch array aside).
 *     Pointers are DEVICE pointers unless marked HOST or PINNED HOST.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream) and
 *     returns after the launches are queued.  Validation failures return before any
 *     launch and leave every buffer untouched.
 *   - Query rows are laid out wave-major: row r*num_reqs + b is row r (0 = anchor) of
 *     request b.
 *   - Data-dependent conditions are values, not errors: positions outside the causal
 *     limit, unmapped pages and out-of-range rows become -1 entries.
 *   - Device buffers must not overlap unless stated.  Calls that share state buffers
 *     must be ordered by the caller (same stream, or events).
 *   - Size limits: a KV row of any cache is at most 65536 bytes; an attention call has at
 *     most 2^24 (row, head) pairs and top-k at most 2^20.  Beyond them a call returns
 *     HS_ERR_UNSUPPORTED before any launch (hs_attn_workspace_bytes returns 0).
 */
#ifndef HISPARSE_H
#define HISPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HS_OK = 0,
  HS_ERR_INVALID_ARG = -1,  /* null pointer, bad size, misaligned buffer, bad dtype      */
  HS_ERR_CAPACITY = -2,     /* topk exceeds the hot-buffer capacity; nothing was changed */
  HS_ERR_UNSUPPORTED = -3,  /* shape/dtype combination the kernels are not built for    */
  HS_ERR_HIP = -4,          /* a HIP runtime call or kernel launch failed                */
  HS_ERR_SCRATCH = -5       /* the shape needs more workspace than the fixed scratch     */
} hs_status;

typedef enum { HS_BF16 = 0, HS_F32 = 1 } hs_dtype;

/*
 * Per-request hot buffer ("device buffer" + "LRU slots" of P1 "1. 启动阶段"; fixed
 * blocks per request as P3's HiSparseHotSpec).  Request b owns global slots
 * [b*capacity, (b+1)*capacity).
 *
 *   slot_loc   [num_reqs*capacity] int32  host-pool row held by the slot, -1 = empty
 *                                         (P1: slot -> physical KV loc)
 *   slot_stamp [num_reqs*capacity] int32  tick of the slot's last use, -1 = empty
 *                                         (P1: LRU slots)
 *   loc_to_hot [host_rows]         int32  global slot holding the host row, or -1
 *                                         (P1: logical loc -> physical HiSparse slot)
 *   hot_kv     [num_reqs*capacity, row_elems] of dtype  the KV rows in the slots
 *   host_pool  PINNED HOST [host_rows, row_elems] of dtype, device-accessible
 *              (P3 "数据 back up": host cache in pinned DRAM)
 *
 * Invariants kept by hs_swap_in / hs_finalize_accepted: slot_loc and loc_to_hot are
 * inverse on occupied slots; hot_kv[s] equals host_pool[slot_loc[s]] bit for bit.
 * Each host row belongs to at most one request.
 */
typedef struct hs_hot_state {
  int32_t num_reqs;
  int32_t capacity;
  int32_t *slot_loc;
  int32_t *slot_stamp;
  int32_t *loc_to_hot;
  int64_t host_rows;
  int32_t row_elems;
  int32_t dtype;          /* hs_dtype */
  void *hot_kv;
  void *host_pool;
} hs_hot_state;

/*
 * hs_resolve_topk -- P3, HiSparseCacheHandle.resolve_topk: in the fully-resident case
 * the request-local top-k indices are converted to global cache slots through the
 * request's block table (block size, physical block stride), with optional per-row
 * valid counts.  P3 "数据 back up" fixes the rows of block p as p*block_size + offset.
 *
 *   topk_pos      [num_rows, topk] int32  token positions, -1 = padding
 *   req_id        [num_rows] int32        request of each row
 *   causal_limit  [num_rows] int32        positions >= limit are masked (future tokens)
 *   block_table   [num_reqs, bt_stride] int32  physical page per logical page, -1 = none
 *   out_slots     [num_rows, topk] int32  physical row, or -1 (in place, no compaction)
 *   out_valid     [num_rows] int32 or NULL   number of non-negative out_slots entries
 *
 * Entry j of row i maps to block_table[b, t/block_size]*physical_block_stride +
 * t%block_size when 0 <= t < causal_limit[i], t/block_size < bt_stride, the table entry
 * is >= 0 and 0 <= b=req_id[i] < num_reqs; otherwise to -1.
 * Errors: HS_ERR_INVALID_ARG for null required pointers or non-positive sizes
 * (num_rows == 0 is a no-op returning HS_OK).
 */
hs_status hs_resolve_topk(const int32_t *topk_pos, int32_t num_rows, int32_t topk,
                          const int32_t *req_id, const int32_t *causal_limit, int32_t num_reqs,
                          const int32_t *block_table, int32_t bt_stride, int32_t block_size,
                          int32_t physical_block_stride, int32_t *out_slots, int32_t *out_valid,
                          void *stream);

/*
 * hs_swap_in -- P3 resolve_topk listing: when the batch is not fully resident the
 * selected KV is swapped into the hot cache and indices into it are returned; P1
 * startup: device buffer, pinned host pool, LRU slots, async stream.  One call handles
 * one wave: row b of wave_rows holds request b's resolved host rows (all -1 if the
 * request has no row in this wave).
 *
 *   wave_rows      [num_reqs, topk] int32  host rows (hs_resolve_topk output), -1 = none
 *   tick           LRU clock value stamped on every slot this wave uses
 *   out_hot_idx    [num_reqs, topk] int32  b*capacity + slot holding the entry, or -1
 *   out_miss_count [num_reqs] int32        number of misses copied for the request
 *   out_miss_pos   [num_reqs, topk] int32 or NULL  entry indices of the misses in
 *                                          ascending order, -1 after miss_count
 *
 * Precondition: a host row belongs to one request (no shared prefix pages), so
 * loc_to_hot[row] is -1 or a slot of the request that selects the row.  Outside it the
 * results are not defined (every access still stays in bounds).
 * Rule (the pages print none; this is the library's definition): an entry hits iff
 * loc_to_hot[row] names a slot of its request; hit slots are pinned; the victims are the
 * #misses unpinned slots with the smallest (stamp, slot); miss m (ascending entry index)
 * takes the m-th victim in ascending slot order.  Applied in that order: the evicted
 * row's loc_to_hot entry is cleared if it names the evicted slot, the miss's row is
 * mapped to its slot, and the host row is copied bit for bit into hot_kv.  Every used
 * slot gets stamp `tick`.
 * Repeated host rows within one request (top-k sets have none): each copy of a hit uses
 * that hit's slot; each copy of a miss is a miss of its own (counted and listed) and takes
 * its own victim, so every hot index names a slot that holds its row, and the row's map
 * entry names the copy installed last (the highest of those slots).  A copy the map does
 * not name stays resident until it is evicted; evicting it leaves the map alone.
 * hot_kv is written only by work queued on `stream`.  It may run concurrently with
 * attention over the previous wave when capacity >= 2*topk and `tick` is above every
 * stamp that was in the state before that wave: the previous wave's slots then hold the
 * newest stamp and are never victims.
 * Errors: HS_ERR_CAPACITY if topk > capacity; HS_ERR_INVALID_ARG for null pointers,
 * non-positive sizes, row bytes not a multiple of 16 or misaligned hot_kv/host_pool,
 * or a host_pool that is not device-accessible pinned memory; HS_ERR_UNSUPPORTED for
 * capacity > 16384.
 */
hs_status hs_swap_in(const hs_hot_state *st, const int32_t *wave_rows, int32_t topk, int32_t tick,
                     int32_t *out_hot_idx, int32_t *out_miss_count, int32_t *out_miss_pos,
                     void *stream);

/*
 * hs_apply_plan -- P3 resolve_topk listing: a runtime that has a leader does not swap
 * on its own but applies the leader's plan (apply_plan); the leader's swap_in produces
 * that plan for its followers and, with prefetch_followers, fills their caches too.
 * Here the plan is what hs_swap_in returned for one wave: the hot index of every entry
 * and, per request, the entries that missed.  A follower cache (another layer, same
 * slot assignment) then needs only the missed rows copied from its own host pool into
 * its own hot buffer; classification and victim choice are not repeated.
 *
 * For cache c < num_caches, request b and m < miss_count[b]:
 *   e = miss_pos[b, m],  row = wave_rows[b, e],  g = hot_idx[b, e]
 *   hot_kv[c, g] <- host_pool[c, row]   (row_bytes bytes, bit for bit)
 * Entries whose e, row or g is out of range write nothing.
 *
 *   hot_kv     [num_caches, num_reqs*capacity, row_bytes] bytes, the followers' hot buffers
 *   host_pool  PINNED HOST [num_caches, host_rows, row_bytes] bytes, device-accessible
 *   wave_rows, hot_idx, miss_pos  [num_reqs, topk] int32; miss_count [num_reqs] int32:
 *              the leader's hs_swap_in input and outputs for the wave (miss_pos required)
 *
 * Afterwards each follower's hot_kv[c, s] equals host_pool[c, slot_loc[s]] for the slots
 * the wave filled, so attention over layer c can use hot_idx as it is.  Plan rows for a
 * subset of query rows (the pages' plan_row_offset) are passed by offsetting the
 * pointers.  Runs on `stream` after the leader's swap (order them with the stream or an
 * event).
 * Errors: HS_ERR_INVALID_ARG (null pointers, non-positive sizes, row_bytes not a multiple
 * of 16, misaligned buffers, host_pool not pinned, counts beyond int32 rows).
 */
hs_status hs_apply_plan(void *hot_kv, const void *host_pool, int64_t host_rows,
                        int32_t num_caches, int32_t num_reqs, int32_t capacity, int32_t row_bytes,
                        const int32_t *wave_rows, int32_t topk, const int32_t *hot_idx,
                        const int32_t *miss_count, const int32_t *miss_pos, void *stream);

/*
 * hs_sparse_decode_attn -- P1 startup: the DSA attention backend reads KV through
 * HiSparse; P3 resolve_topk: attention receives the cache and per-row indices.  For each
 * row i and head h, over S_i = {j : 0 <= indices[i,j] < kv_rows}:
 *   s_j = scale * <q[i,h,:d_qk], kv[indices[i,j], :d_qk]>,  p = softmax(s),
 *   out[i,h,:] = sum_j p_j * kv[indices[i,j], :d_v]   (value = leading d_v entries),
 *   lse[i,h] = log(sum_j exp(s_j)).
 * An empty S_i gives out = 0 and lse = -inf.  Duplicate indices count as separate keys.
 *
 *   q        [num_rows, num_heads, d_qk] of dtype (row stride num_heads*d_qk)
 *   kv       [kv_rows, d_qk] of dtype (the paged device pool, or hs_hot_state.hot_kv)
 *   indices  [num_rows, topk] int32 (hs_resolve_topk or hs_swap_in output)
 *   out      [num_rows, num_heads, d_v] of dtype
 *   lse      [num_rows, num_heads] float32 or NULL (natural log)
 *   workspace, workspace_bytes  device scratch of at least hs_attn_workspace_bytes(...)
 *            bytes (may be NULL when that is 0)
 *
 * Supported: dtype HS_BF16 with d_qk = 576, d_v = 512, num_heads a multiple of 32 (MFMA
 * path, fp32 accumulation, bf16 output); dtype HS_F32 with d_qk <= 1024, d_v <= d_qk,
 * topk <= 8192 (fp32 path).  KV rows referenced by indices must hold finite values.
 * Errors: HS_ERR_INVALID_ARG (null pointers, sizes, workspace too small, misalignment);
 * HS_ERR_UNSUPPORTED (other shapes).
 */
hs_status hs_sparse_decode_attn(const void *q, const void *kv, int64_t kv_rows,
                                const int32_t *indices, int32_t num_rows, int32_t num_heads,
                                int32_t d_qk, int32_t d_v, int32_t topk, float scale,
                                int32_t dtype, void *out, float *lse, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * hs_sparse_decode_attn_cus -- hs_sparse_decode_attn sized for part of the GPU, for a call
 * that runs beside another kernel on another stream: on the swap path the next wave's
 * swap-in runs during this wave's attention (P1 "1. 启动阶段": the hot buffer is filled on
 * an async stream), and that swap-in needs compute units of its own.  Every attention
 * workgroup holds one compute unit (its LDS), so a whole-GPU launch takes all 256 and a
 * kernel started beside it waits for them to drain.  This call computes exactly what
 * hs_sparse_decode_attn computes (same arguments, same results up to the order in which
 * fp32 partial sums are added), with its kernel and key splits chosen for `max_cus`
 * compute units:
 *
 *   max_cus   > 0; 256 or more is the whole GPU (the plain call).  The launch takes at most
 *             max_cus workgroups when the kernel chosen has at most max_cus (row,
 *             head-group) units times ceil(topk / 2048) (a key split holds at most 2048
 *             keys); larger batches take one workgroup per unit and split.
 *   workspace the size hs_attn_workspace_bytes returns for the same sizes always suffices.
 *
 * The fp32 path (dtype HS_F32) launches as the plain call does.
 * Errors: as hs_sparse_decode_attn; HS_ERR_INVALID_ARG for max_cus <= 0.
 */
hs_status hs_sparse_decode_attn_cus(const void *q, const void *kv, int64_t kv_rows,
                                    const int32_t *indices, int32_t num_rows, int32_t num_heads,
                                    int32_t d_qk, int32_t d_v, int32_t topk, float scale,
                                    int32_t dtype, void *out, float *lse, void *workspace,
                                    size_t workspace_bytes, int32_t max_cus, void *stream);

/*
 * hs_sparse_decode_attn_paged -- the fully resident batch in one call: P3 resolve_topk
 * listing (when every request's KV is resident, the top-k positions are converted to
 * cache rows through the block table and attention reads the paged cache directly).
 * Computes exactly hs_resolve_topk(topk_pos, ..., out_slots) followed by
 * hs_sparse_decode_attn(q, kv_pool, kv_rows, out_slots, ...), without writing the rows:
 * position t of row i (request req_id[i]) selects pool row
 * block_table[b, t / block_size] * physical_block_stride + t % block_size when
 * 0 <= t < causal_limit[i] and that table entry is >= 0; other entries select nothing.
 *
 *   q, out, lse, workspace  as for hs_sparse_decode_attn (same workspace size)
 *   kv_pool      [kv_rows, d_qk] of dtype, the paged device cache
 *   topk_pos, req_id, causal_limit, block_table, bt_stride, block_size,
 *   physical_block_stride, num_reqs   as for hs_resolve_topk
 *
 * Supported: dtype HS_BF16, d_qk = 576, d_v = 512, num_heads a multiple of 32 (other
 * shapes: resolve, then hs_sparse_decode_attn).  Valid counts are not produced; use
 * hs_resolve_topk where they are needed.
 * Errors: as hs_resolve_topk and hs_sparse_decode_attn; HS_ERR_UNSUPPORTED for other shapes.
 */
hs_status hs_sparse_decode_attn_paged(const void *q, const void *kv_pool, int64_t kv_rows,
                                      const int32_t *topk_pos, const int32_t *req_id,
                                      const int32_t *causal_limit, int32_t num_reqs,
                                      const int32_t *block_table, int32_t bt_stride,
                                      int32_t block_size, int32_t physical_block_stride,
                                      int32_t num_rows, int32_t num_heads, int32_t d_qk,
                                      int32_t d_v, int32_t topk, float scale, int32_t dtype,
                                      void *out, float *lse, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * hs_attn_plan_info -- the launch hs_sparse_decode_attn(_paged, _mixed) makes for these
 * sizes: *heads_per_wg = 32, 64 or 128 (the bf16 kernel the call runs), or 1 for the fp32
 * path (one wave per (row, head)); *splits = key splits per row (1: no split, no
 * workspace).  Either output may be NULL.  For tuning and tests; it launches nothing.
 * Errors: HS_ERR_INVALID_ARG for non-positive sizes or an unknown dtype;
 * HS_ERR_UNSUPPORTED for bf16 shapes the attention calls reject.
 */
hs_status hs_attn_plan_info(int32_t num_rows, int32_t num_heads, int32_t d_qk, int32_t d_v,
                            int32_t topk, int32_t dtype, int32_t *heads_per_wg,
                            int32_t *splits);

/* hs_attn_plan_info for hs_sparse_decode_attn_cus with `max_cus` compute units (> 0;
 * HS_ERR_INVALID_ARG otherwise). */
hs_status hs_attn_plan_info_cus(int32_t num_rows, int32_t num_heads, int32_t d_qk, int32_t d_v,
                                int32_t topk, int32_t dtype, int32_t max_cus,
                                int32_t *heads_per_wg, int32_t *splits);

/*
 * hs_sparse_decode_attn_noalloc -- hs_sparse_decode_attn for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and arguments without workspace, workspace_bytes.  The
 * key-split partials go to a scratch array the library keeps in device memory, one per GPU
 * for the life of the process (HS_NOALLOC_SCRATCH_BYTES = 32 MiB; enough for every shape
 * with topk <= 2048).  The call allocates nothing.  All calls on one GPU share that GPU's
 * scratch: calls that may overlap on one GPU (different streams without ordering) race and
 * must be ordered by the caller.  Its contents persist between calls and need no clearing
 * (every partial is written before it is read).
 * Errors: as hs_sparse_decode_attn; HS_ERR_SCRATCH when hs_attn_workspace_bytes(...) for
 * these sizes exceeds HS_NOALLOC_SCRATCH_BYTES (nothing is launched); HS_ERR_HIP if the
 * scratch array's device address cannot be obtained.
 */
#define HS_NOALLOC_SCRATCH_BYTES (32u << 20)
hs_status hs_sparse_decode_attn_noalloc(const void *q, const void *kv, int64_t kv_rows,
                                        const int32_t *indices, int32_t num_rows,
                                        int32_t num_heads, int32_t d_qk, int32_t d_v, int32_t topk,
                                        float scale, int32_t dtype, void *out, float *lse,
                                        void *stream);

/* Device workspace hs_sparse_decode_attn(_paged) needs for these sizes (0 when none). */
size_t hs_attn_workspace_bytes(int32_t num_rows, int32_t num_heads, int32_t d_qk, int32_t d_v,
                               int32_t topk, int32_t dtype);

/*
 * hs_sparse_decode_attn_mixed -- attention over a batch whose rows read two caches.
 * P3 resolve_topk listing: a fully resident batch reads the resident (paged) cache
 * directly, any other batch swaps into the hot cache; P3 reclaim_resident_blocks: once
 * part of a request's resident KV is reclaimed the request is no longer fully resident,
 * and build_offload_command / are_requests_fully_resident make the choice for the whole
 * batch.  This call lets each row take its own source, so resident requests keep reading
 * the resident pool while reclaimed ones go through hs_swap_in and the hot buffer.
 *
 * Row i is computed exactly as hs_sparse_decode_attn computes it over
 *   (kv_a, kv_a_rows, indices_a[i])  when row_sel[i] == 0, or
 *   (kv_b, kv_b_rows, indices_b[i])  otherwise.
 *
 *   kv_a, kv_b            [kv_*_rows, d_qk] bf16 (e.g. resident pool and hot buffer)
 *   indices_a, indices_b  [num_rows, topk] int32 rows into their cache, -1 = none
 *   row_sel               [num_rows] int32 source of each row
 *   workspace             as hs_sparse_decode_attn (hs_attn_workspace_bytes)
 *
 * Errors: as hs_sparse_decode_attn; HS_ERR_UNSUPPORTED for fp32 or shapes other than
 * d_qk 576, d_v 512, heads a multiple of 32.
 */
hs_status hs_sparse_decode_attn_mixed(const void *q, const void *kv_a, int64_t kv_a_rows,
                                      const int32_t *indices_a, const void *kv_b,
                                      int64_t kv_b_rows, const int32_t *indices_b,
                                      const int32_t *row_sel, int32_t num_rows, int32_t num_heads,
                                      int32_t d_qk, int32_t d_v, int32_t topk, float scale,
                                      int32_t dtype, void *out, float *lse, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * hs_sparse_decode_attn_mixed_cus -- hs_sparse_decode_attn_mixed planned for `max_cus`
 * compute units, for a mixed batch whose attention runs beside the next wave's swap-in
 * (P1 "1. 启动阶段": the hot buffer is filled on an async stream); as
 * hs_sparse_decode_attn_cus is to hs_sparse_decode_attn (same results, the same workspace
 * size serves).
 * Errors: as hs_sparse_decode_attn_mixed; HS_ERR_INVALID_ARG for max_cus <= 0.
 */
hs_status hs_sparse_decode_attn_mixed_cus(const void *q, const void *kv_a, int64_t kv_a_rows,
                                          const int32_t *indices_a, const void *kv_b,
                                          int64_t kv_b_rows, const int32_t *indices_b,
                                          const int32_t *row_sel, int32_t num_rows,
                                          int32_t num_heads, int32_t d_qk, int32_t d_v,
                                          int32_t topk, float scale, int32_t dtype, void *out,
                                          float *lse, void *workspace, size_t workspace_bytes,
                                          int32_t max_cus, void *stream);

/*
 * hs_finalize_accepted -- P2 ④: the target verifies [anchor, drafts] in one causal pass;
 * row r's logits judge draft r+1; drafts are kept while they equal the target's greedy
 * choice; only the accepted prefix's KV is kept and the replacement (or bonus) token has
 * no KV yet.  P2 ⑥/timeline table: the next anchor follows the kept prefix.  P1 summary:
 * accepted-KV finalize ends the main line.
 *
 *   logits        [rows, vocab] bf16, rows = st->num_reqs * rows_per_req (wave-major);
 *                 or NULL when out_argmax already holds every row's argmax (from
 *                 hs_greedy_argmax, run earlier on any stream ordered before this call):
 *                 the call then only accepts and finalizes (vocab is then ignored)
 *   draft_ids     [rows] int32 (the anchor rows' entries are ignored)
 *   new_kv        [rows, st->row_elems] of st->dtype: the verified KV of each row
 *   seq_len       [num_reqs] int32: committed length + rows_per_req (row r of request b
 *                 sits at position seq_len[b] - rows_per_req + r)
 *   block_table   [num_reqs, bt_stride] int32 (physical block stride = block_size)
 *   out_argmax    [rows] int32: lowest index of each row's maximum (NaN never wins);
 *                 an input instead when logits is NULL
 *   out_accept_len [num_reqs] int32: L_b = longest l <= rows_per_req-1 with
 *                 draft_ids[row(b,k)] == argmax[row(b,k-1)] for 1 <= k <= l
 *   out_next_token [num_reqs] int32: argmax[row(b, L_b)]
 *
 * Then per request: rows r > L_b are dropped (a hot slot holding that position is
 * emptied; the host row is left as is); rows r <= L_b have new_kv written to their
 * host-pool row (PINNED HOST, device stores) and to the hot buffer (overwrite if
 * resident, else installed with the hs_swap_in victim rule, the slots of the request's
 * resident kept rows pinned, an evicted row's map entry cleared only if it names the
 * evicted slot), stamp `tick`.  Dropped rows are processed first.  The hs_swap_in
 * precondition applies: a verify row's host row is unmapped or mapped into its request.
 * Errors: HS_ERR_INVALID_ARG (null pointers, sizes, rows_per_req < 1 or >
 * st->capacity, vocab < 1); HS_ERR_UNSUPPORTED (rows_per_req > 64).
 */
hs_status hs_finalize_accepted(const hs_hot_state *st, const void *logits, int32_t vocab,
                               const int32_t *draft_ids, const void *new_kv, int32_t rows_per_req,
                               const int32_t *seq_len, const int32_t *block_table,
                               int32_t bt_stride, int32_t block_size, int32_t tick,
                               int32_t *out_argmax, int32_t *out_accept_len,
                               int32_t *out_next_token, void *stream);

/*
 * hs_greedy_argmax -- the greedy choice of P2 ④ on its own: out_argmax[i] = the lowest
 * index of the maximum of logits row i (bf16, compared exactly; NaN never wins; a row of
 * only NaN and -inf gives 0).  It depends on the logits alone, so a decode step can run it
 * ahead of the swap waves and pass its result to hs_finalize_accepted with logits = NULL.
 *
 *   logits      [rows, vocab] bf16, 16-byte aligned
 *   out_argmax  [rows] int32
 *
 * Errors: HS_ERR_INVALID_ARG (null or misaligned pointers, rows < 0, vocab < 1); rows == 0
 * is a no-op.
 */
hs_status hs_greedy_argmax(const void *logits, int32_t rows, int32_t vocab, int32_t *out_argmax,
                           void *stream);

/*
 * Device -> host backup of KV rows: the copy behind prefill staging and page spills.
 * P3 "数据 back up": HiSparseWorker._enqueue_transfers turns page transfers into source
 * slots (block id * kernel block size + offset, one list per cache) and destination host
 * rows ((destination block * blocks per KV block + page offset) * kernel block size +
 * offset), then launches hisparse_backup_layers, which copies those rows of every layer
 * from the device cache into the pinned host cache, and records an event.  P1 "3.
 * HiSparse staging": admit_request_into_staging backs a prefill's KV up to the host pool
 * asynchronously; collect_ready_reqs polls that event before the request decodes.
 *
 * For layer l < num_layers and entry i < num_rows:
 *   s = src_slots[(src_per_layer ? l * num_rows : 0) + i]    slot in the device cache
 *   p = (s / src_block_size) * src_block_stride + s % src_block_size   its physical row
 *   d = dst_rows[i]                                          row of the host cache
 *   host_cache row (l * host_layer_rows + d) <- dev_cache row (l * dev_layer_rows + p),
 *   row_bytes bytes, bit for bit.
 * Entries with s < 0, d < 0, p >= dev_layer_rows or d >= host_layer_rows write nothing,
 * so row lists may be padded with -1.  Nothing else of the host cache is written.
 *
 *   dev_cache    [num_layers * dev_layer_rows, row_bytes] bytes
 *   host_cache   PINNED HOST [num_layers * host_layer_rows, row_bytes] bytes,
 *                device-accessible; written by device stores over the host link
 *   src_slots    [src_per_layer ? num_layers : 1, num_rows] int32
 *   dst_rows     [num_rows] int32.  Its non-negative entries must be distinct (the
 *                pages' planner gives every transfer its own host page).  With a
 *                duplicate, each 16-byte part of that host row comes from one of its
 *                sources, and the parts may come from different ones.
 *
 * Completion: the host rows hold the copies once the work queued on `stream` up to this
 * call has finished (record an event after the call; poll or wait on it before the host
 * reads them).  Returns HS_OK at once when num_rows == 0.
 * Errors: HS_ERR_INVALID_ARG (null pointers, non-positive sizes, row_bytes not a multiple
 * of 16, misaligned caches, host_cache not pinned, row counts beyond int32).
 */
hs_status hs_backup_rows(const void *dev_cache, int64_t dev_layer_rows, void *host_cache,
                         int64_t host_layer_rows, int32_t num_layers, int32_t row_bytes,
                         const int32_t *src_slots, int32_t src_per_layer,
                         const int32_t *dst_rows, int32_t num_rows, int32_t src_block_size,
                         int32_t src_block_stride, void *stream);

/*
 * hs_append_accepted -- P2 ⑤: after target verification only the accepted prefix's
 * target features go through the draft model's context K/V branch and are appended to
 * its context KV cache (KV_D(P) -> KV_D(P + [a0, b1]) in the worked example; the KV the
 * draft round made for itself is not used).  ⑥ and the timeline table: the context then
 * covers every confirmed position except the newest token, which is the next anchor.
 *
 * For request b with L = clamp(accept_len[b], 0, rows_per_req - 1) and r = 0 .. L:
 *   pos = ctx_len[b] + r,  page = ctx_block_table[b, pos / block_size]
 *   ctx_cache row (page * physical_block_stride + pos % block_size)
 *       <- new_rows row (r * num_reqs + b)          (row_bytes bytes, bit for bit)
 * then ctx_len[b] += L + 1.  A position whose page is unmapped (-1, or past bt_stride)
 * or whose row is past ctx_rows is not written (the caller maps pages ahead); ctx_len
 * still advances.
 *
 *   ctx_cache        [ctx_rows, row_bytes] bytes, the draft model's context KV
 *   ctx_block_table  [num_reqs, bt_stride] int32
 *   ctx_len          [num_reqs] int32, read and advanced in place
 *   new_rows         [num_reqs*rows_per_req, row_bytes] bytes, wave-major verify rows
 *                    (context K/V of each row from the target's features)
 *   accept_len       [num_reqs] int32 (hs_finalize_accepted's out_accept_len)
 *
 * Errors: HS_ERR_INVALID_ARG (null pointers, non-positive sizes, row_bytes not a multiple
 * of 16, misaligned buffers, ctx_rows beyond int32).
 */
hs_status hs_append_accepted(void *ctx_cache, int64_t ctx_rows, int32_t row_bytes,
                             const int32_t *ctx_block_table, int32_t bt_stride,
                             int32_t block_size, int32_t physical_block_stride, int32_t *ctx_len,
                             const void *new_rows, const int32_t *accept_len, int32_t num_reqs,
                             int32_t rows_per_req, void *stream);

/*
 * hs_host_read -- the host link's reference read rate (not a step of the path): copies
 * `bytes` from pinned host memory into device memory with a streaming zero-copy kernel,
 * the same kind of access the swap-in copy makes to the pinned host pool (P1 "1. 启动阶段":
 * pinned host pool; P3 "数据 back up": host cache in pinned DRAM), but over one contiguous
 * range.  Asynchronous on `stream`.
 *
 *   host_src  PINNED HOST, 16-byte aligned, device-accessible
 *   dst       device memory, 16-byte aligned, at least `bytes` long
 *   bytes     a multiple of 16 (0 is a no-op)
 *
 * Errors: HS_ERR_INVALID_ARG (null or misaligned pointers, bytes not a multiple of 16 or
 * negative, host_src not pinned host memory).
 */
hs_status hs_host_read(const void *host_src, void *dst, int64_t bytes, void *stream);

/* Static description of a status code. */
const char *hs_status_string(int32_t status);

/* Library version string. */
const char *hs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HISPARSE_H */
