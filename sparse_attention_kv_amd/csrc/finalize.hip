// finalize_accepted: greedy acceptance of the verified draft rows, then keep exactly the
// accepted prefix's KV (gfx950).
//
// P2 "投机解码的 KV 流转：prefill 阶段 DFlash 也要吃下整个 prompt", ④: the target runs the
// anchor and the drafts through one causal pass; the logits of row r decide draft r+1;
// drafts are accepted while they match the target's greedy choice, the first mismatch
// is replaced by that choice and the rest is dropped; only the accepted prefix keeps its
// KV, the replacement token has none yet.  ⑥ and the timeline table: the next anchor is
// the position right after the kept prefix.  P1 "hiSparse-MTP", summary: accepted-KV
// finalize closes the main line.
//
// Kernel 1 (one workgroup per row): argmax over the vocabulary, lowest index on ties,
//   16-byte loads of 8 bf16 logits (HBM-bound streaming read).  It depends on the logits
//   only, so a caller may run it on its own (hs_greedy_argmax) ahead of the rest of the
//   step and hand its result to kernel 2.
// Kernel 2 (one workgroup per request): acceptance length, then
//   dropped rows -> hot slots holding them are emptied;
//   kept rows    -> new KV stored to the pinned host pool (device stores over the host
//                   link) and into the hot buffer (overwrite, or install into the LRU
//                   victim with the kept hits pinned).

#include "ops.h"

namespace hs {
namespace {

constexpr int kArgThreads = 512;
constexpr int kArgUnroll = 4;  // 16-byte loads per thread and pass (more measured slower)
constexpr int kFinThreads = 256;
constexpr int kMaxRowsPerReq = 64;
constexpr int kKeysPerThread = 16;  // victim keys held in registers up to 4096 slots

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// One workgroup per row; several workgroups share a CU (small footprint), so the 384 rows
// of a verify batch stream concurrently.  Each thread keeps kArgUnroll 16-byte loads in
// flight and walks its chunks in increasing index order (first maximum kept).
__global__ __launch_bounds__(kArgThreads) void argmax_kernel(const uint16_t *__restrict__ logits,
                                                             int32_t vocab,
                                                             int32_t *__restrict__ out_argmax) {
  __shared__ float s_v[kArgThreads / 64];
  __shared__ int s_i[kArgThreads / 64];
  const int64_t row = blockIdx.x;
  const uint16_t *lr = logits + row * vocab;
  const int tid = threadIdx.x;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if ((vocab & 7) == 0) {
    const int chunks = vocab >> 3;  // >= 1: the host rejects vocab <= 0
    for (int c0 = tid; c0 < chunks; c0 += kArgThreads * kArgUnroll) {
      // Every load of the pass is issued before any is used: chunks past the end re-load
      // the last chunk (no branch around a load) and are skipped below.
      i32x4 raw[kArgUnroll];
#pragma unroll
      for (int k = 0; k < kArgUnroll; ++k) {
        const int c = min(c0 + k * kArgThreads, chunks - 1);
        raw[k] = *reinterpret_cast<const i32x4 *>(lr + 8 * c);
      }
#pragma unroll
      for (int k = 0; k < kArgUnroll; ++k) {
        const int c = c0 + k * kArgThreads;
        if (c >= chunks) break;
        // chunk maximum first (v_max_f32 returns the non-NaN operand, so NaN never wins);
        // the index is searched only when the chunk beats the running best
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v[e] = __uint_as_float((e & 1) ? (static_cast<uint32_t>(raw[k][e >> 1]) & 0xffff0000u)
                                         : (static_cast<uint32_t>(raw[k][e >> 1]) << 16));
        const float cm = __builtin_fmaxf(
            __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), __builtin_fmaxf(v[2], v[3])),
            __builtin_fmaxf(__builtin_fmaxf(v[4], v[5]), __builtin_fmaxf(v[6], v[7])));
        if (cm > bv) {
          int e0 = 7;
#pragma unroll
          for (int e = 7; e >= 0; --e) e0 = v[e] == cm ? e : e0;
          bv = cm;
          bi = 8 * c + e0;
        } else if (bi == 0x7fffffff) {
          bi = 8 * c;  // every value so far is -inf or NaN: the lowest index stands
        }
      }
    }
  } else {
    for (int i = tid; i < vocab; i += kArgThreads) {
      float v = bf16_bits_to_float(lr[i]);
      v = v != v ? -INFINITY : v;
      if (better(v, i, bv, bi)) { bv = v; bi = i; }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off, 64);
    const int oi = __shfl_xor(bi, off, 64);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if (lane_id() == 0) { s_v[tid >> 6] = bv; s_i[tid >> 6] = bi; }
  __syncthreads();
  if (tid == 0) {
    for (int wv = 1; wv < kArgThreads / 64; ++wv)
      if (better(s_v[wv], s_i[wv], bv, bi)) { bv = s_v[wv]; bi = s_i[wv]; }
    out_argmax[row] = bi == 0x7fffffff ? 0 : bi;
  }
}

// One step of a wave minimum over 64-bit keys: each lane takes the minimum of its key and
// the key of the lane that the DPP control selects (lanes without a source, or in rows the
// mask leaves out, keep their own).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint64_t dpp_min_step(uint64_t v) {
  const int lo = static_cast<int>(v), hi = static_cast<int>(v >> 32);
  const uint32_t plo = __builtin_amdgcn_update_dpp(lo, lo, kCtrl, kRowMask, 0xf, false);
  const uint32_t phi = __builtin_amdgcn_update_dpp(hi, hi, kCtrl, kRowMask, 0xf, false);
  const uint64_t p = (static_cast<uint64_t>(phi) << 32) | plo;
  return p < v ? p : v;
}

// Wave minimum: row_shr 1, 2, 4, 8 leave each 16-lane row's minimum in its lane 15;
// row_bcast 15 then 31 carry it across rows, so lane 63 ends with the wave's minimum.
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  v = dpp_min_step<0x111, 0xf>(v);
  v = dpp_min_step<0x112, 0xf>(v);
  v = dpp_min_step<0x114, 0xf>(v);
  v = dpp_min_step<0x118, 0xf>(v);
  v = dpp_min_step<0x142, 0xa>(v);
  v = dpp_min_step<0x143, 0xc>(v);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(v), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), 63);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Block-wide minimum of (stamp, slot) keys packed in 64 bits.
__device__ __forceinline__ uint64_t block_min_u64(uint64_t v, uint64_t *s_red) {
  v = wave_min_u64(v);
  if (lane_id() == 0) s_red[threadIdx.x >> 6] = v;
  lds_barrier();
  uint64_t r = s_red[0];
  for (int wv = 1; wv < kFinThreads / 64; ++wv) r = s_red[wv] < r ? s_red[wv] : r;
  lds_barrier();
  return r;
}

__global__ __launch_bounds__(kFinThreads) void finalize_kernel(
    int32_t num_reqs, int32_t capacity, int32_t *__restrict__ slot_loc,
    int32_t *__restrict__ slot_stamp, int32_t *__restrict__ loc_to_hot, int64_t host_rows,
    int32_t row_bytes, uint8_t *__restrict__ hot_kv, uint8_t *__restrict__ host_pool,
    const int32_t *__restrict__ draft_ids, const uint8_t *__restrict__ new_kv,
    int32_t rows_per_req, const int32_t *__restrict__ seq_len,
    const int32_t *__restrict__ block_table, int32_t bt_stride, int32_t block_size, int32_t tick,
    const int32_t *__restrict__ argmax, int32_t *__restrict__ out_accept_len,
    int32_t *__restrict__ out_next_token) {
  __shared__ int s_L;
  __shared__ int s_loc[kMaxRowsPerReq];    // host row of each verify row, -1 none
  __shared__ int s_hit[kMaxRowsPerReq];    // slot within the request holding the row, -1 none
  __shared__ int s_slot[kMaxRowsPerReq];   // slot within the request for kept rows, -1 none
  __shared__ int s_owner[kMaxRowsPerReq];  // host row the slot of a missed kept row held
  __shared__ int s_miss[kMaxRowsPerReq];   // kept rows that must be installed
  __shared__ int s_vic[kMaxRowsPerReq];    // victims in LRU order
  __shared__ int s_vown[kMaxRowsPerReq];   // host row each victim held
  __shared__ int s_nmiss;
  __shared__ uint64_t s_red[kFinThreads / 64];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int R = rows_per_req;
  const int64_t slot_base = (int64_t)b * capacity;
  auto slot_key = [&](int sl, int stamp) -> uint64_t {
    return (static_cast<uint64_t>(static_cast<uint32_t>(stamp) ^ 0x80000000u) << 32) |
           static_cast<uint32_t>(sl);
  };

  // Loads first, uses after: the acceptance inputs, the verify rows' block-table entries,
  // then (up to 4096 slots) the request's (stamp, slot) keys and slot owners, which depend
  // on nothing here.  Loads complete in issue order, so the key loads go last and do not
  // delay the reads the acceptance length and host rows wait for.  This kernel's own slot
  // updates are applied to the register copies as it makes them.
  // (Row indices are clamped into range so that no load sits behind a branch; the
  // clamped lanes' values are masked when used.)
  const int draft_next = draft_ids[(int64_t)min(tid + 1, R - 1) * num_reqs + b];
  const int am_row = argmax[(int64_t)min(tid, R - 1) * num_reqs + b];
  // host row of position seq_len - R + tid (same block-table mapping as resolve_topk)
  const int pos = seq_len[b] - R + tid;
  const int pi = pos >= 0 ? pos / block_size : 0;
  const int page_raw = block_table[(int64_t)b * bt_stride + min(pi, bt_stride - 1)];
  // masked with an OR, not a select (a select on a load's value compiles to a branch
  // around the load)
  const int page = page_raw | -static_cast<int>(!(tid < R && pos >= 0 && pi < bt_stride));
  // this thread's first chunk of the verify rows' new KV (chunk tid of rows 0 .. R-1)
  const int chunks = row_bytes >> 4;
  const int c_first = min(tid, R * chunks - 1);
  const int r_first = c_first / chunks;
  const i32x4 kv_first = *reinterpret_cast<const i32x4 *>(
      new_kv + ((int64_t)r_first * num_reqs + b) * row_bytes + (c_first - r_first * chunks) * 16);
  const bool in_regs = capacity <= kFinThreads * kKeysPerThread;
  uint64_t keys[kKeysPerThread];
  int owner[kKeysPerThread];
  if (in_regs) {
    // slots past the capacity re-read the last slot (no branch around a load: every load
    // is issued before the first wait) and are masked after
    int stamp[kKeysPerThread];
#pragma unroll
    for (int i = 0; i < kKeysPerThread; ++i) {
      const int64_t g = slot_base + min(tid + i * kFinThreads, capacity - 1);
      stamp[i] = slot_stamp[g];
      owner[i] = slot_loc[g];
    }
#pragma unroll
    for (int i = 0; i < kKeysPerThread; ++i) {
      const int sl = tid + i * kFinThreads;
      keys[i] = sl < capacity ? slot_key(sl, stamp[i]) : ~0ull;
      owner[i] = sl < capacity ? owner[i] : -1;
    }
  }

  // Acceptance length, wave-parallel (R <= 64): lane r checks draft r+1 against the argmax
  // of row r; L is the number of leading matches.
  if (tid < 64) {
    const bool match = tid < R - 1 && draft_next == am_row;
    const uint64_t mism = ~__builtin_amdgcn_ballot_w64(match);
    const int L = min(static_cast<int>(__builtin_ctzll(mism)), R - 1);
    if (tid == 0) {
      out_accept_len[b] = L;
      out_next_token[b] = argmax[(int64_t)L * num_reqs + b];
      s_L = L;
    }
  }
  if (tid < R) {
    int loc = -1;
    if (page >= 0) {
      const int64_t r = (int64_t)page * block_size + (pos - pi * block_size);
      loc = r < host_rows ? (int)r : -1;
    }
    s_loc[tid] = loc;
  }
  lds_barrier();
  const int L = s_L;

  // The slot each verify row occupies, looked up once (the rows' host rows are distinct,
  // so emptying a dropped row's slot cannot change a kept row's lookup).
  if (tid < R) {
    const int loc = s_loc[tid];
    const int64_t g = loc >= 0 ? loc_to_hot[loc] : -1;
    s_hit[tid] = g >= slot_base && g < slot_base + capacity ? (int)(g - slot_base) : -1;
    s_slot[tid] = -1;
  }

  // kept rows' new KV -> their host-pool rows (device stores written through over the host
  // link); issued early so the link transfer overlaps the slot bookkeeping below
  for (int c = tid; c < (L + 1) * chunks; c += kFinThreads) {
    const int r = c / chunks;
    const int part = c - r * chunks;
    const int loc = s_loc[r];
    if (loc < 0) continue;
    const i32x4 v = c == tid ? kv_first : *reinterpret_cast<const i32x4 *>(
        new_kv + ((int64_t)r * num_reqs + b) * row_bytes + part * 16);
    store_through16(host_pool + (int64_t)loc * row_bytes + part * 16, v);
  }
  lds_barrier();

  // dropped rows: empty the slot that holds them (host rows untouched)
  if (tid < R && tid > L && s_hit[tid] >= 0) {
    const int64_t g = slot_base + s_hit[tid];
    slot_loc[g] = -1;
    slot_stamp[g] = -1;
    loc_to_hot[s_loc[tid]] = -1;
  }
  if (in_regs) {
    for (int r = L + 1; r < R; ++r) {
      const int sl = s_hit[r];
#pragma unroll
      for (int i = 0; i < kKeysPerThread; ++i)
        if (sl >= 0 && tid + i * kFinThreads == sl) {
          keys[i] = slot_key(sl, -1);
          owner[i] = -1;
        }
    }
  }
  // kept rows (wave-parallel): hit -> its slot (pinned), miss -> listed in row order
  if (tid < 64) {
    const int r = tid;
    const bool kept = r <= L && r < R && s_loc[r] >= 0;
    const bool miss = kept && s_hit[r] < 0;
    if (kept && !miss) s_slot[r] = s_hit[r];
    const uint64_t mm = __builtin_amdgcn_ballot_w64(miss);
    if (miss) s_miss[__builtin_popcountll(mm & ((1ull << r) - 1))] = r;
    if (tid == 0) s_nmiss = __builtin_popcountll(mm);
  }
  // (the slow victim search below re-reads stamps and owners from memory, which the
  // dropped-row clears above wrote: it needs the full barrier)
  if (in_regs) lds_barrier(); else __syncthreads();
  const int nmiss = s_nmiss;

  // victims: repeatedly the least-recently-used unpinned, unchosen slot (nmiss <= R).  (A
  // candidate always exists when rows_per_req <= capacity, which the host checks.)
  if (nmiss > 0 && in_regs) {
    for (int r = 0; r <= L; ++r) {  // kept hits are pinned
      const int ps = s_slot[r];
#pragma unroll
      for (int i = 0; i < kKeysPerThread; ++i)
        if (tid + i * kFinThreads == ps) keys[i] = ~0ull;
    }
    for (int k = 0; k < nmiss; ++k) {
      uint64_t best = ~0ull;
#pragma unroll
      for (int i = 0; i < kKeysPerThread; ++i) best = keys[i] < best ? keys[i] : best;
      best = block_min_u64(best, s_red);
      if (tid == 0 && best == ~0ull) s_vic[k] = -1;
#pragma unroll
      for (int i = 0; i < kKeysPerThread; ++i)
        if (keys[i] == best && best != ~0ull) {  // chosen: not a candidate again
          keys[i] = ~0ull;
          s_vic[k] = tid + i * kFinThreads;
          s_vown[k] = owner[i];
        }
    }
    lds_barrier();
  } else if (nmiss > 0) {
    for (int k = 0; k < nmiss; ++k) {
      uint64_t best = ~0ull;
      for (int sl = tid; sl < capacity; sl += kFinThreads) {
        bool taken = false;
        for (int r = 0; r <= L; ++r) taken |= s_slot[r] == sl;
        for (int j = 0; j < k; ++j) taken |= s_vic[j] == sl;
        if (taken) continue;
        const uint64_t key = slot_key(sl, slot_stamp[slot_base + sl]);
        best = key < best ? key : best;
      }
      best = block_min_u64(best, s_red);
      if (tid == 0) {
        const int v = best == ~0ull ? -1 : static_cast<int>(best & 0xffffffffu);
        s_vic[k] = v;
        s_vown[k] = v >= 0 ? slot_loc[slot_base + v] : -1;
      }
      __syncthreads();
    }
  }
  // Victims were chosen in LRU order; pair them with the misses in ascending slot order:
  // miss k takes the victim of rank k (victims are distinct slots).
  if (tid < nmiss) {
    const int v = s_vic[tid];
    int rank = 0;
    for (int j = 0; j < nmiss; ++j) rank += s_vic[j] < v;
    s_slot[s_miss[rank]] = v;
    s_owner[s_miss[rank]] = s_vown[tid];
  }
  lds_barrier();
  if (tid < nmiss && s_slot[s_miss[tid]] >= 0) {
    const int r = s_miss[tid];
    const int64_t g = slot_base + s_slot[r];
    const int old = s_owner[r];
    // the evicted row is unmapped only while the map names this slot (a stale copy leaves
    // its row's live mapping alone); the kept row's own entry is never this slot's value
    // before the store below, so the compare-and-swap and the store commute
    if (old >= 0 && old < host_rows && old != s_loc[r]) atomicCAS(&loc_to_hot[old], (int32_t)g, -1);
    slot_loc[g] = s_loc[r];
    loc_to_hot[s_loc[r]] = (int32_t)g;
  }
  if (tid <= L && tid < R && s_slot[tid] >= 0) slot_stamp[slot_base + s_slot[tid]] = tick;
  // kept rows' new KV -> their hot slots (16 bytes per lane access)
  for (int c = tid; c < (L + 1) * chunks; c += kFinThreads) {
    const int r = c / chunks;
    const int part = c - r * chunks;
    if (s_loc[r] < 0 || s_slot[r] < 0) continue;
    const i32x4 v = c == tid ? kv_first : *reinterpret_cast<const i32x4 *>(
        new_kv + ((int64_t)r * num_reqs + b) * row_bytes + part * 16);
    *reinterpret_cast<i32x4 *>(hot_kv + (slot_base + s_slot[r]) * row_bytes + part * 16) = v;
  }
}

}  // namespace

hipError_t launch_argmax(const void *logits, int32_t rows, int32_t vocab, int32_t *out_argmax,
                         hipStream_t stream) {
  hipLaunchKernelGGL(argmax_kernel, dim3(rows), dim3(kArgThreads), 0, stream,
                     static_cast<const uint16_t *>(logits), vocab, out_argmax);
  return hipGetLastError();
}

hipError_t launch_finalize(const hs_hot_state &st, const void *host_pool_dev, const void *logits,
                           int32_t vocab, const int32_t *draft_ids, const void *new_kv,
                           int32_t rows_per_req, const int32_t *seq_len, const int32_t *block_table,
                           int32_t bt_stride, int32_t block_size, int32_t tick, int32_t *out_argmax,
                           int32_t *out_accept_len, int32_t *out_next_token, hipStream_t stream) {
  if (logits != nullptr) {  // else out_argmax already holds every row's argmax
    const hipError_t e = launch_argmax(logits, st.num_reqs * rows_per_req, vocab, out_argmax, stream);
    if (e != hipSuccess) return e;
  }
  const int elem = st.dtype == HS_BF16 ? 2 : 4;
  hipLaunchKernelGGL(finalize_kernel, dim3(st.num_reqs), dim3(kFinThreads), 0, stream, st.num_reqs,
                     st.capacity, st.slot_loc, st.slot_stamp, st.loc_to_hot, st.host_rows,
                     st.row_elems * elem, static_cast<uint8_t *>(st.hot_kv),
                     static_cast<uint8_t *>(const_cast<void *>(host_pool_dev)), draft_ids,
                     static_cast<const uint8_t *>(new_kv), rows_per_req, seq_len, block_table,
                     bt_stride, block_size, tick, out_argmax, out_accept_len, out_next_token);
  return hipGetLastError();
}

int finalize_max_rows_per_req() { return kMaxRowsPerReq; }

}  // namespace hs
