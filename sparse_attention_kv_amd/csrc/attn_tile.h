// Shared pieces of the bf16 sparse-attention kernels (gfx950): tile geometry, the
// direct-to-LDS gather of selected KV rows, and LDS-only synchronisation.
//
// A tile is 64 selected latent rows (64 x 1152 B = 72 KiB) gathered with direct-to-LDS
// 16-byte loads; each kernel chooses the placement of the 16-byte chunks in LDS.
#pragma once

#include "common.h"

namespace hs {
namespace tile {

constexpr int kD = 576;                       // latent row width (q . k)
constexpr int kDV = 512;                      // value width
constexpr int kTK = 64;                       // keys per tile
constexpr int kThreads = 256;
constexpr int kRowBytes = kD * 2;             // 1152
constexpr int kRowChunks = kRowBytes / 16;    // 72
constexpr int kTileBytes = kTK * kRowBytes;   // 73728
constexpr int kLoadsPerThread = kTK * kRowChunks / kThreads;  // 18
constexpr int kMaxKeysPerSplit = 2048;
constexpr int kWaves = kThreads / 64;
constexpr float kLn2 = 0.69314718055994530942f;

// The kernels synchronise with lds_barrier() (common.h): outstanding global loads (the
// next tile's direct-to-LDS gathers) are deliberately not waited for there, since an LDS
// release fence would make the compiler wait for them too (they write LDS).  Code that
// needs a gathered tile waits with wait_vmem() first.
// Direct-to-LDS 16-byte load: lane l's 16 bytes from src land at LDS byte lds_base + 16 l.
// Written as inline asm so that the compiler's wait-count insertion does not treat every
// later LDS read of either tile buffer as dependent on it (it cannot tell the buffers
// apart and would wait for the whole in-flight prefetch).  Readers of a DMA'd buffer wait
// explicitly (wait_vmem / vmcnt_imm) before the barrier that publishes it.  The s_nop is
// the wait state required between an M0 write and an LDS DMA.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; nothing else here uses it
__device__ __forceinline__ void dma16(const void *src, const void *lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>((uintptr_t)(HS_LDS const void *)lds_dst));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x3f70); }  // vmcnt(0)
// s_waitcnt immediate for vmcnt(n), expcnt and lgkmcnt left at their maxima (gfx9 encoding:
// vmcnt bits [3:0] and [15:14]).
constexpr int vmcnt_imm(int n) { return ((n >> 4) & 3) << 14 | 0x3f70 | (n & 15); }

// Exclusive prefix sum across the wave of v in [0, 15] (a lane's count of valid keys), and
// the wave total: one ballot per bit of v and a count of the set bits below the lane, in
// place of a six-round shuffle scan on the path to the first gather.
constexpr int kSmallScanMax = 15;
__device__ __forceinline__ int wave_exclusive_scan_small(int v, int &total) {
  int ex = 0, tot = 0;
#pragma unroll
  for (int bit = 0; bit < 4; ++bit) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(((v >> bit) & 1) != 0);
    const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
    ex += below << bit;
    tot += __builtin_popcountll(m) << bit;
  }
  total = tot;
  return ex;
}

// v_max_f32 (inputs here are finite or -inf)
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_fmaxf(a, b); }

// Maximum and sum of a lane's value and that of lane l ^ 32 (l ^ 16), in every lane, with
// one VALU lane swap instead of an LDS permute: the gfx950 permlane swaps return the lane's
// own value in one result and its partner's in the other (which one depends on the half),
// so combining the two results is the same for every lane.  a + b = b + a exactly, so the
// sums equal those of a shuffle.
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Load this thread's share of a split's indices: entry j = tid * per + k (k < per) of
// `irow`.  With kPaged the entries are request-local token positions, resolved here exactly
// as hs_resolve_topk does (P3 "vllm 分析（十二）——Hisparse下篇", resolve_topk listing:
// position t of a row of request b is kept iff 0 <= t < causal_limit, its page t / block_size
// is inside the table row and mapped; it becomes page * physical_block_stride + t % block_size;
// P3 "数据 back up": rows of page p are p * block_size + offset).  All position loads are
// issued before the block-table loads.  Invalid entries come back as -1.
template <bool kPaged, int kN>
__device__ __forceinline__ void load_split_indices(const int32_t *__restrict__ irow, int per,
                                                   int kcnt, int tid, const PagedMap &pg, int row,
                                                   int (&vals)[kN]) {
#pragma unroll
  for (int k = 0; k < kN; ++k) {
    const int j = tid * per + k;
    vals[k] = (k < per && j < kcnt) ? irow[j] : -1;
  }
  if constexpr (kPaged) {
    const int b = pg.req_id[row];
    const int lim = pg.causal_limit[row];
    const bool req_ok = b >= 0 && b < pg.num_reqs;
    const int32_t *bt = pg.block_table + (int64_t)(req_ok ? b : 0) * pg.bt_stride;
    int pidx[kN], page[kN];
#pragma unroll
    for (int k = 0; k < kN; ++k) {
      const int t = vals[k];
      const bool ok = req_ok && t >= 0 && t < lim;
      pidx[k] = ok ? t / pg.block_size : pg.bt_stride;
      page[k] = pidx[k] < pg.bt_stride ? bt[pidx[k]] : -1;
    }
#pragma unroll
    for (int k = 0; k < kN; ++k) {
      int slot = -1;
      if (page[k] >= 0) {
        const int64_t r = (int64_t)page[k] * pg.physical_block_stride +
                          (vals[k] - pidx[k] * pg.block_size);
        slot = r < 0x7fffffffLL ? (int)r : -1;
      }
      vals[k] = slot;
    }
  }
}

// Scores are kept relative to a reference max m_ref per head (log2 domain).  P is formed
// as 2^(s - m_ref) without re-normalising O every tile; only when a score exceeds m_ref
// by more than kRescaleSlack (P would exceed 2^kRescaleSlack) is a new reference taken
// and O and the running sum rescaled.  The arithmetic is exact for any reference; the
// slack only bounds P (bf16) and the fp32 accumulators.
constexpr float kRescaleSlack = 64.f;

}  // namespace tile

// Split-KV combine (attn.hip): merges normalised bf16 partials with fp32 (max, sum).
void launch_attn_combine(const __bf16 *ws_o, const float *ws_ml, int32_t splits, int32_t num_rows,
                         int32_t num_heads, __bf16 *out, float *lse, hipStream_t stream);

}  // namespace hs
