// swap_in: hit/miss split, LRU victim choice and host->HBM copy for one wave (gfx950).
//
// P3 "vllm 分析（十二）——Hisparse下篇", resolve_topk listing: when a batch is not fully
// resident the selected KV is swapped into the per-request hot cache and the returned
// indices point into it.  P1 "hiSparse-MTP", "1. 启动阶段": the coordinator owns a
// device buffer, a pinned host pool, LRU slots and an async stream; the state maps are
// slot -> physical KV loc and logical loc -> physical HiSparse slot.
//
// One workgroup (16 waves) per request; requests never share slots or host rows, so
// workgroups touch disjoint state.  Phases, each separated by a workgroup barrier:
//   A  classify: each thread owns a contiguous run of entries; hit iff loc_to_hot >= 0;
//      hit slots are marked pinned in LDS; misses are compacted in entry order with a
//      wave-ballot/prefix-sum scan.
//   B  LRU threshold: the need-th smallest (stamp, slot) key among unpinned slots via a
//      4-pass, 8-bit radix select over LDS histograms.  Each thread owns a run of slots
//      whose stamps and held rows it loaded into registers before the first copy round's
//      host reads went out, so B-E wait on no memory load while those reads are in flight.
//   C  victims in ascending slot order: a second ordered scan over slot runs picks every
//      unpinned slot below the threshold stamp plus the lowest-numbered ones at it.
//   D  install: miss m takes victim m (done by the victim slot's owner).  The evicted row's
//      map entry is cleared only while it names the evicted slot (a compare-and-swap), and
//      the new row's entry takes the largest slot installed for it (an atomic max), so a
//      row repeated within a request maps to its last install in pairing order.  Both are
//      atomics whose results are unused: nothing waits for them, and their outcome does not
//      depend on the order in which they reach memory.
//   E  stamp every used slot with `tick`, emit hot indices.
//   F  copy the miss rows from the pinned host pool into the hot buffer with 16-byte
//      loads (the host link is the bound; many independent loads per thread are kept
//      in flight).

#include "ops.h"

namespace hs {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
static_assert(kMaxCapacity <= 16 * kThreads, "a thread holds at most 16 slots in registers");

struct SwapLds {
  int *hist;           // [256]
  int *scan;           // [kWaves + 1]
  int *sel;            // [2]
  int *slot_of_entry;  // [topk]  slot (within the request) used by entry j; -1 invalid
  int *miss_entry;     // [topk]  entry index of miss m
  int *miss_row;       // [topk]  host row of miss m
  int *victim;         // [topk]  slot of victim m (ascending)
  uint8_t *pinned;     // [capacity]
};

__device__ __forceinline__ SwapLds carve(uint8_t *base, int topk) {
  SwapLds s;
  int *p = reinterpret_cast<int *>(base);
  s.hist = p; p += 256;
  s.scan = p; p += kWaves + 1;
  s.sel = p; p += 3;
  s.slot_of_entry = p; p += topk;
  s.miss_entry = p; p += topk;
  s.miss_row = p; p += topk;
  s.victim = p; p += topk;
  s.pinned = reinterpret_cast<uint8_t *>(p);
  return s;
}

size_t lds_bytes(int topk, int capacity) {
  return sizeof(int) * (256 + kWaves + 1 + 3 + 4 * (size_t)topk) + (size_t)capacity;
}

// Exclusive scan of one int per thread across the workgroup (ordered by thread id).
__device__ __forceinline__ int block_exclusive_scan(int v, int *scan, int &total) {
  int wave_total;
  const int ex = wave_exclusive_scan(v, wave_total);
  const int w = threadIdx.x / 64;
  if (lane_id() == 0) scan[w] = wave_total;
  __syncthreads();
  if (w == 0) {
    const int t = lane_id() < kWaves ? scan[lane_id()] : 0;
    int all;
    const int wex = wave_exclusive_scan(t, all);
    if (lane_id() < kWaves) scan[lane_id()] = wex;
    if (lane_id() == 0) scan[kWaves] = all;
  }
  __syncthreads();
  const int res = ex + scan[w];
  total = scan[kWaves];
  __syncthreads();
  return res;
}

__device__ __forceinline__ uint32_t order_key(int32_t stamp) {
  return static_cast<uint32_t>(stamp) ^ 0x80000000u;  // signed order as unsigned order
}

template <int kSper>
__global__ __launch_bounds__(kThreads) void swap_in_kernel(
    int32_t capacity, int32_t *__restrict__ slot_loc, int32_t *__restrict__ slot_stamp,
    int32_t *__restrict__ loc_to_hot, int64_t host_rows, int32_t row_bytes,
    uint8_t *__restrict__ hot_kv, const uint8_t *__restrict__ host_pool,
    const int32_t *__restrict__ wave_rows, int32_t topk, int32_t tick,
    int32_t *__restrict__ out_hot_idx, int32_t *__restrict__ out_miss_count,
    int32_t *__restrict__ out_miss_pos) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  SwapLds sm = carve(lds_raw, topk);
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t slot_base = (int64_t)b * capacity;
  const int32_t *rows = wave_rows + (int64_t)b * topk;

  for (int s = tid; s < capacity; s += kThreads) sm.pinned[s] = 0;
  __syncthreads();

  // ---- A: classify (thread owns entries [j0, j0 + per)) ----
  const int per = (topk + kThreads - 1) / kThreads;
  const int j0 = tid * per;
  int my_miss = 0;
  for (int k = 0; k < per; ++k) {
    const int j = j0 + k;
    if (j >= topk) break;
    const int row = rows[j];
    int slot = -1;
    if (row >= 0 && row < host_rows) {
      const int g = loc_to_hot[row];
      if (g >= slot_base && g < slot_base + capacity) {
        slot = (int)(g - slot_base);
        sm.pinned[slot] = 1;
      } else {
        slot = -2;  // miss: slot assigned in phase D
        ++my_miss;
      }
    }
    sm.slot_of_entry[j] = slot;
  }
  int need;
  int m = block_exclusive_scan(my_miss, sm.scan, need);
  for (int k = 0; k < per; ++k) {
    const int j = j0 + k;
    if (j >= topk) break;
    if (sm.slot_of_entry[j] == -2) {
      sm.miss_entry[m] = j;
      sm.miss_row[m] = rows[j];
      if (out_miss_pos) out_miss_pos[(int64_t)b * topk + m] = j;
      ++m;
    }
  }
  if (out_miss_pos)
    for (int i = need + tid; i < topk; i += kThreads) out_miss_pos[(int64_t)b * topk + i] = -1;
  if (tid == 0) out_miss_count[b] = need;
  __syncthreads();

  // ---- this thread's slots [s0, s0 + sper): stamps and held rows into registers, so that
  // victim choice loads nothing from memory once the copy's first host reads are out (the
  // wait for such a load would also wait for every host read issued before it) ----
  const int sper = (capacity + kThreads - 1) / kThreads;  // <= kSper
  const int s0 = tid * sper;
  const int s_last = max(0, min(s0 + sper, capacity) - 1);
  int32_t st_own[kSper], held[kSper];
  if (need > 0) {
#pragma unroll
    for (int k = 0; k < kSper; ++k) {
      const int s = min(s0 + k, s_last);  // slots past the thread's run re-read its last one
      st_own[k] = slot_stamp[slot_base + s];
      held[k] = slot_loc[slot_base + s];
    }
  }

  // ---- F, first round: host reads of the miss rows (known since A) go out now ----
  const int chunks = row_bytes >> 4;
  const int total = need * chunks;
  constexpr int kUnroll = 8;
  i32x4 v[kUnroll];
  // All kUnroll loads are issued before the first store: chunks past the end re-read the
  // last chunk (no branch around a load, which would make each load wait for the one before
  // it) and are not stored.
  auto load_round = [&](int base) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = min(base + u * kThreads + tid, total - 1);
      const int mi = c / chunks;
      const int part = c - mi * chunks;
      v[u] = *reinterpret_cast<const i32x4 *>(host_pool + (int64_t)sm.miss_row[mi] * row_bytes + part * 16);
    }
  };
  if (need > 0) load_round(0);

  if (need > 0) {
    // ---- B: radix select of the need-th smallest key among unpinned slots ----
    uint32_t prefix = 0;
    int remaining = need;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < 256; i += kThreads) sm.hist[i] = 0;
      if (tid == 0) { sm.sel[0] = 0; sm.sel[1] = remaining; }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kSper; ++k) {
        const int s = s0 + k;
        if (k >= sper || s >= capacity || sm.pinned[s]) continue;
        const uint32_t key = order_key(st_own[k]);
        if (pass == 0 || (key >> (shift + 8)) == (prefix >> (shift + 8)))
          atomicAdd(&sm.hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {
        int c[4], sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) { c[i] = sm.hist[4 * tid + i]; sum += c[i]; }
        int all;
        const int ex = wave_exclusive_scan(sum, all);
        if (ex < remaining && remaining <= ex + sum) {
          int acc = ex;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (remaining <= acc + c[i]) {
              sm.sel[0] = 4 * tid + i;
              sm.sel[1] = remaining - acc;
              break;
            }
            acc += c[i];
          }
        }
      }
      __syncthreads();
      prefix |= (uint32_t)sm.sel[0] << shift;
      remaining = sm.sel[1];
      __syncthreads();
    }
    const uint32_t tau = prefix;
    const int take_eq = remaining;  // slots with key == tau to take, lowest slot first

    // ---- C: victims in ascending slot order ----
    int my_eq = 0;
#pragma unroll
    for (int k = 0; k < kSper; ++k) {
      const int s = s0 + k;
      if (k < sper && s < capacity && !sm.pinned[s] && order_key(st_own[k]) == tau) ++my_eq;
    }
    int unused;
    int eq_rank = block_exclusive_scan(my_eq, sm.scan, unused);
    int my_vic = 0;
    uint32_t flags = 0;
#pragma unroll
    for (int k = 0; k < kSper; ++k) {
      const int s = s0 + k;
      if (k >= sper || s >= capacity || sm.pinned[s]) continue;
      const uint32_t key = order_key(st_own[k]);
      bool vk = false;
      if (key < tau) {
        vk = true;
      } else if (key == tau) {
        vk = eq_rank < take_eq;
        ++eq_rank;
      }
      if (vk) { flags |= 1u << k; ++my_vic; }
    }
    int vrank = block_exclusive_scan(my_vic, sm.scan, unused);

    // ---- D: the slot's owner installs miss vrank into it.  Misses map to -1 before the
    // wave (a mapping into this request's slots is a hit; other requests' rows are never
    // selected), so the max over the wave's installs of one row is its highest victim slot.
    // An entry naming this slot belongs to a row this wave does not select (it would be a
    // hit and the slot pinned), so no install races with the clear; a slot whose stale copy
    // is the row it now receives skips the clear. ----
#pragma unroll
    for (int k = 0; k < kSper; ++k) {
      if (!(flags & (1u << k)) || vrank >= need) continue;
      const int i = vrank++;
      const int vs = s0 + k;
      const int row = sm.miss_row[i];
      const int64_t g = slot_base + vs;
      const int old = held[k];
      if (old >= 0 && old < host_rows && old != row) atomicCAS(&loc_to_hot[old], (int32_t)g, -1);
      slot_loc[g] = row;
      atomicMax(&loc_to_hot[row], (int32_t)g);
      sm.victim[i] = vs;
      sm.slot_of_entry[sm.miss_entry[i]] = vs;
    }
    __syncthreads();
  }

  // ---- E: stamps and hot indices ----
  for (int j = tid; j < topk; j += kThreads) {
    const int slot = sm.slot_of_entry[j];
    int32_t out = -1;
    if (slot >= 0) {
      slot_stamp[slot_base + slot] = tick;
      out = (int32_t)(slot_base + slot);
    }
    out_hot_idx[(int64_t)b * topk + j] = out;
  }

  // ---- F: copy miss rows host pool -> hot buffer, 16 bytes per lane access ----
  for (int base = 0; base < total; base += kThreads * kUnroll) {
    if (base > 0) load_round(base);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = base + u * kThreads + tid;
      if (c < total) {
        const int mi = c / chunks;
        const int part = c - mi * chunks;
        *reinterpret_cast<i32x4 *>(hot_kv + (slot_base + sm.victim[mi]) * row_bytes + part * 16) = v[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_swap_in(const hs_hot_state &st, const void *host_pool_dev,
                          const int32_t *wave_rows, int32_t topk, int32_t tick,
                          int32_t *out_hot_idx, int32_t *out_miss_count, int32_t *out_miss_pos,
                          hipStream_t stream) {
  const int elem = st.dtype == HS_BF16 ? 2 : 4;
  const int32_t row_bytes = st.row_elems * elem;
  const size_t lds = lds_bytes(topk, st.capacity);
  // slots per thread held in registers: 4 up to 4096 slots, else up to 16 (16384 slots)
  const auto kern = st.capacity <= 4 * kThreads ? swap_in_kernel<4> : swap_in_kernel<16>;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(st.num_reqs), dim3(kThreads), lds, stream, st.capacity,
                     st.slot_loc, st.slot_stamp, st.loc_to_hot, st.host_rows, row_bytes,
                     static_cast<uint8_t *>(st.hot_kv), static_cast<const uint8_t *>(host_pool_dev),
                     wave_rows, topk, tick, out_hot_idx, out_miss_count, out_miss_pos);
  return hipGetLastError();
}

}  // namespace hs
