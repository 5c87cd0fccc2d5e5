// sparse_decode_attn: attention over only the selected latent KV rows (gfx950).
//
// P1 "hiSparse-MTP", "1. 启动阶段": the DSA attention backend reads KV through
// HiSparse.  P3 "vllm 分析（十二）——Hisparse下篇", resolve_topk listing: attention gets
// the cache plus per-row indices (-1 padded) and reads only those rows.
//
// bf16 path (MLA decode shape: 576-wide latent rows, value = leading 512 entries, heads
// share the row):
//   * workgroup = 8 waves = (query row, group of 32 heads, key split).  The four head
//     groups of one (row, split) are placed on the same XCD (consecutive dispatches on
//     one XCD) so the selected rows are fetched from HBM once and re-read from L2.  Head
//     groups go in pairs, and the second pair walks the split's tiles in reverse order,
//     so a tile is requested by two workgroups at a time, not four, and the second visit
//     finds it in L2.
//   * the split's valid indices are compacted into LDS first; KV tiles of 64 selected
//     rows (72 KiB) are gathered with direct-to-LDS 16-byte loads, double buffered, and
//     XOR-swizzled in 16-byte units so MFMA operand reads are bank-conflict free.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (keys as M, 16 heads as N, Q resident
//     in registers); each wave owns 16 keys x 16 heads of the tile.
//   * online softmax in the exp2 domain, max shared across waves through LDS.
//   * O^T = V^T P^T with v_mfma_f32_32x32x16_bf16 (32 heads as N); each wave owns 64 of
//     the 512 value dims; V is read with ds_read_b64_tr_b16 (LDS transpose) so no second
//     copy of the tile is needed.
//   * with several key splits, normalised bf16 partials + fp32 (max, sum) go to a
//     workspace and a combine kernel merges them (log-sum-exp weights).
//
// f32 path: straightforward vector-ALU kernel (one wave per (row, head)), used for the
// small fp32 validation shapes.

#include "attn_tile.h"

namespace hs {
namespace {

constexpr int kHG = 32;                       // heads per workgroup
// (row, 64-head) groups from which attn64 runs on the whole GPU.  With 128 heads (top-k
// 2048) the 32-head kernel measures faster up to 20 rows (8-20 rows: 4-9 %), the 64-head
// one from 24 rows (24-31 rows: 6-10 %).  With fewer CUs the threshold scales with them.
constexpr int kMinGroups64 = 48;
// attn128 runs with more (row, 128-head) groups than half the CUs the call may use.  It
// reads each KV row once per row instead of twice; above 128 groups on the whole GPU the
// 64-head kernel needs a second round of workgroups (160-224 rows: 15-21 % slower than
// attn128), at 128 the two measure the same.
constexpr int kThreads8 = 512;                // 8 waves: two per SIMD
constexpr int kWaves8 = kThreads8 / 64;
constexpr int kSlots8 = tile::kTK * tile::kRowChunks / kThreads8;  // 9 gather slots per wave
constexpr int kOStride = 64 * 2 + 16;         // epilogue staging: a wave's 64 dims of one head
constexpr int kPStride = tile::kTK * 2 + 16;  // P tile row stride in bytes (padded)
constexpr int kQSlots = kHG * tile::kRowBytes / 1024;  // 36 one-KiB DMA slots of Q per workgroup
using namespace tile;

// Tile layout: physical 16-byte chunk c holds (key c/72, logical part (c%72) ^ swz(key)).
// Rows are 1152 bytes, so key bit 0 alone moves a chunk by half the 256-byte bank period.
// A transposed PV read of a half wave touches keys k0 + {0..3} and four parts, and needs 16
// distinct 16-byte bank slots: swz puts key bit 1 on part bit 2, which no lane of the half
// varies.  Key bit 2 goes to part bit 1, which keeps the row-wise QK^T reads (lane octet
// pairs (0,3), (1,2), (4,7), (5,6) of a 16-byte read share a cycle) conflict free too.
__device__ __forceinline__ int swz(int key) { return ((key << 1) & 4) | ((key >> 1) & 2); }

// Gather tile t (selected rows t*64 .. t*64+63 of the compacted list) into LDS buffer dst.
// Keys past n_valid re-load the last valid row; their scores are masked to -inf.  Wave w
// issues the 9 one-KiB slots n = 9w .. 9w+8 (lane l's chunk in slot n is c = 64n + l).
template <int kFirst, int kCount>
__device__ __forceinline__ void gather_part(const uint8_t *__restrict__ kv, const int32_t *sidx,
                                            int n_valid, int t, uint8_t *dst, int w, int l) {
  // All row-index reads first, then the DMA issues.
  const int last = n_valid - 1;
  int rows[kCount], parts[kCount];
#pragma unroll
  for (int i = 0; i < kCount; ++i) {
    const int c = (w * kSlots8 + kFirst + i) * 64 + l;
    const int key = c / kRowChunks;
    const int kk = t * kTK + key;
    rows[i] = sidx[kk < last ? kk : last];
    parts[i] = (c - key * kRowChunks) ^ swz(key);
  }
#pragma unroll
  for (int i = 0; i < kCount; ++i) {
    const uint8_t *src = kv + (int64_t)rows[i] * kRowBytes + parts[i] * 16;
    dma16(src, dst + (w * kSlots8 + kFirst + i) * 1024);
  }
}

template <bool kSplit, bool kPaged>
__global__ __launch_bounds__(kThreads8, 1) void attn_bf16_kernel(
    const __bf16 *__restrict__ q, const uint8_t *__restrict__ kv, int64_t kv_rows,
    const int32_t *__restrict__ indices, int32_t num_rows, int32_t num_heads, int32_t topk,
    int32_t keys_per_split, int32_t splits, float scale_log2, __bf16 *__restrict__ out,
    float *__restrict__ lse, __bf16 *__restrict__ ws_o, float *__restrict__ ws_ml, PagedMap pg,
    AltSource alt) {
  __shared__ __attribute__((aligned(16))) uint8_t s_kv0[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_kv1[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[kHG * kPStride];
  __shared__ __attribute__((aligned(16))) int32_t s_sidx[kMaxKeysPerSplit];
  __shared__ __attribute__((aligned(16))) float s_red[4][kHG];
  __shared__ __attribute__((aligned(16))) float s_alpha[kHG];
  __shared__ __attribute__((aligned(16))) float s_fm[kHG];
  __shared__ __attribute__((aligned(16))) float s_fl[kHG];
  __shared__ int s_scan[kWaves8];
  __shared__ int s_flag[kWaves8];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int kq = w & 3;   // QK^T: this wave's 16 keys of the tile
  const int hh = w >> 2;  // QK^T: this wave's 16 heads of the 32
  const int n_hg = num_heads / kHG;
  // Dispatch i runs on XCD i % 8; XCD x takes units [x * per, (x + 1) * per).  Units are
  // ordered (row, split, head group): the head groups of a (row, split) read the same KV
  // rows and the splits of a row the same Q, so each is fetched from HBM once per row.
  const int units = num_rows * splits * n_hg;
  const int per_xcd = (units + 7) / 8;
  const int u = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (u >= units) return;
  const int hg = u % n_hg;
  const int split = (u / n_hg) % splits;
  const int row = u / (n_hg * splits);
  if (alt.row_sel != nullptr && alt.row_sel[row] != 0) {  // this row reads the second source
    kv = alt.kv;
    kv_rows = alt.kv_rows;
    indices = alt.indices;
  }
  const int h0 = hg * kHG;
  const int kbeg = split * keys_per_split;
  const int kcnt = max(0, min(keys_per_split, topk - kbeg));

  // ---- indices (or token positions) of this split: they gate the first KV gather ----
  const int32_t *irow = indices + (int64_t)row * topk + kbeg;
  const int per = (kcnt + kThreads8 - 1) / kThreads8;  // <= 4
  int vals[kMaxKeysPerSplit / kThreads8];
  load_split_indices<kPaged>(irow, per, kcnt, tid, pg, row, vals);

  // ---- Q (32 heads x 576), one copy per workgroup, staged through the second tile buffer.
  // Slot 18hb + ks (1 KiB) holds, at 16l, lane l's chunk of the B operand for head block hb:
  // head 16hb + (l&15), elements 32ks + 8(l>>4) .. +7.  Wave w issues slots w, w+8, ...
  {
    const uint8_t *qrow = reinterpret_cast<const uint8_t *>(q + ((int64_t)row * num_heads + h0) * kD);
#pragma unroll
    for (int i = 0; i < (kQSlots + kWaves8 - 1) / kWaves8; ++i) {
      const int slot = w + kWaves8 * i;
      if (slot < kQSlots) {
        const int hb = slot / (kD / 32), ks = slot - hb * (kD / 32);
        const uint8_t *src = qrow + (16 * hb + (l & 15)) * kRowBytes + 64 * ks + 16 * (l >> 4);
        dma16(src, s_kv1 + slot * 1024);
      }
    }
  }

  // ---- compact the valid indices into LDS (order preserved) ----
  int n_valid;
  {
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kMaxKeysPerSplit / kThreads8; ++k) {
      const bool ok = vals[k] >= 0 && vals[k] < kv_rows;
      vals[k] = ok ? vals[k] : -1;
      cnt += ok;
    }
    int wave_total;
    static_assert(kMaxKeysPerSplit / kThreads8 <= kSmallScanMax, "per-lane key count fits the scan");
    const int ex = wave_exclusive_scan_small(cnt, wave_total);
    if (l == 0) s_scan[w] = wave_total;
    lds_barrier();
    int base = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kWaves8; ++i) {
      const int c = s_scan[i];
      base += i < w ? c : 0;
      total += c;
    }
    int pos = base + ex;
#pragma unroll
    for (int k = 0; k < kMaxKeysPerSplit / kThreads8; ++k)
      if (vals[k] >= 0) s_sidx[pos++] = vals[k];
    n_valid = total;
    lds_barrier();
  }

  // Step t of the loop works on tile tile_at(t).  Head groups 2, 3 (mod 4) take the tiles
  // last to first: each tile is then requested by two workgroups at once instead of four,
  // and the other pair reads it again from L2 later (1 to 31 rows of 128 heads measured
  // 2-3 % faster than all four head groups in the same order).
  const int ntiles = (n_valid + kTK - 1) / kTK;
  const bool backwards = (hg & 2) != 0;
  auto tile_at = [&](int t) { return backwards ? ntiles - 1 - t : t; };
  if (ntiles > 0) gather_part<0, kSlots8>(kv, s_sidx, n_valid, tile_at(0), s_kv0, w, l);
  // This thread's Q slots were issued before the tile-0 gather: wait for all but those 9.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(kSlots8));
  lds_barrier();
  bf16x8 qreg[kD / 32];  // B operand of this wave's head block
#pragma unroll
  for (int ks = 0; ks < kD / 32; ++ks)
    qreg[ks] = *reinterpret_cast<const bf16x8 *>(s_kv1 + (hh * (kD / 32) + ks) * 1024 + 16 * l);

  float m_ref = -INFINITY;  // reference max of head 16hh + (l & 15) (log2 domain)
  float l_run = 0.f;        // this lane's share of that head's softmax sum
  f32x16 oacc[2];           // O^T: this wave's 64 value dims (2 blocks of 32) x 32 heads
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[nb][i] = 0.f;

  // O^T (this wave's 64 dims x 32 heads) += V^T P^T for the tile in `cur`: the MFMA A
  // operand is V^T (a lane's 8 keys at one value dim, two transposed LDS reads) and B is
  // P^T, so a lane ends with one head (l & 31) and, per 32-dim block nb, the dims
  // 8(i>>2) + 4(l>>5) + (i&3).  Operands of the next 16-key step are issued before the
  // MFMAs of the current one.
  auto pv_tile = [&](const uint8_t *cur) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const int g = l >> 4, j = l & 15, r = j >> 2, c = j & 3;
    const uint8_t *prow = s_p + (l & 31) * kPStride + 16 * (l >> 5);
    int voff[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) voff[nb] = 64 * w + 32 * nb + 16 * (g & 1) + 4 * c;
    bf16x8 pa[2];
    s16x4 vlo[2][2], vhi[2][2];
    auto load_step = [&](int ks, int buf) {
      pa[buf] = *reinterpret_cast<const bf16x8 *>(prow + 32 * ks);
      const int key0 = 16 * ks + 8 * (g >> 1) + r;
      const int key1 = key0 + 4;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int part = voff[nb] >> 3, off = (voff[nb] & 7) * 2;
        vlo[buf][nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (HS_LDS s16x4 *)(cur + key0 * kRowBytes + ((part ^ swz(key0)) << 4) + off));
        vhi[buf][nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (HS_LDS s16x4 *)(cur + key1 * kRowBytes + ((part ^ swz(key1)) << 4) + off));
      }
    };
    load_step(0, 0);
#pragma unroll
    for (int ks = 0; ks < kTK / 16; ++ks) {
      if (ks + 1 < kTK / 16) load_step(ks + 1, (ks + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      const int b = ks & 1;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 vv = {vlo[b][nb][0], vlo[b][nb][1], vlo[b][nb][2], vlo[b][nb][3],
                          vhi[b][nb][0], vhi[b][nb][1], vhi[b][nb][2], vhi[b][nb][3]};
        oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pa[b],
                                                           oacc[nb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The inner loop touches O only through MFMA; a tile whose scores need a new reference
  // (always the first one) leaves it, O is rescaled once outside, and the loop resumes.
  int t = 0;
  while (t < ntiles) {
    bool renorm = false;
    for (; t < ntiles; ++t) {
      const uint8_t *cur = (t & 1) ? s_kv1 : s_kv0;
      uint8_t *nxt = (t & 1) ? s_kv0 : s_kv1;
      wait_vmem();
      lds_barrier();
      const bool more = t + 1 < ntiles;
      const int tnext = more ? tile_at(t + 1) : 0;

      // ---- S^T (this wave's 16 keys x 16 heads), K fragments read 3 at a time ahead; the
      // next tile's 9 DMA slots go out 2, 1, 2, 1, 2, 1 after the six batches of 3 MFMAs ----
      f32x4 sacc;
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[i] = 0.f;
      {
        const int key = 16 * kq + (l & 15);
        const uint8_t *krow = cur + key * kRowBytes;
        const int sw = swz(key);
        constexpr int kB = 3;
        bf16x8 kf[2][kB];
#pragma unroll
        for (int j = 0; j < kB; ++j)
          kf[0][j] = *reinterpret_cast<const bf16x8 *>(krow + (((4 * j + (l >> 4)) ^ sw) << 4));
#pragma unroll
        for (int bt = 0; bt < kD / 32 / kB; ++bt) {
          if (bt + 1 < kD / 32 / kB) {
#pragma unroll
            for (int j = 0; j < kB; ++j) {
              const int ks = (bt + 1) * kB + j;
              kf[(bt + 1) & 1][j] =
                  *reinterpret_cast<const bf16x8 *>(krow + (((4 * ks + (l >> 4)) ^ sw) << 4));
            }
          }
          __builtin_amdgcn_sched_barrier(0);  // keep the next batch's reads ahead of these MFMAs
#pragma unroll
          for (int j = 0; j < kB; ++j)
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[bt & 1][j], qreg[bt * kB + j], sacc, 0, 0, 0);
          if (more) {
            if (bt == 0) gather_part<0, 2>(kv, s_sidx, n_valid, tnext, nxt, w, l);
            if (bt == 1) gather_part<2, 1>(kv, s_sidx, n_valid, tnext, nxt, w, l);
            if (bt == 2) gather_part<3, 2>(kv, s_sidx, n_valid, tnext, nxt, w, l);
            if (bt == 3) gather_part<5, 1>(kv, s_sidx, n_valid, tnext, nxt, w, l);
            if (bt == 4) gather_part<6, 2>(kv, s_sidx, n_valid, tnext, nxt, w, l);
            if (bt == 5) gather_part<8, 1>(kv, s_sidx, n_valid, tnext, nxt, w, l);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- softmax numerators against the reference max (head 16hh + (l&15), keys
      // 16kq + 4(l>>4) + i of the tile) ----
      const int h = 16 * hh + (l & 15);
      const int kfirst = tile_at(t) * kTK + 16 * kq + 4 * (l >> 4);
      float s[4];
      float mw = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = (kfirst + i < n_valid) ? sacc[i] * scale_log2 : -INFINITY;
        mw = vmax(mw, s[i]);
      }
      const bool any_over = __builtin_amdgcn_ballot_w64(mw > m_ref + kRescaleSlack) != 0;
      float psum = 0.f;
      if (!any_over) {
        bf16x4 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(s[i] - m_ref);
          psum += p;
          pk[i] = (__bf16)p;
        }
        *reinterpret_cast<bf16x4 *>(s_p + h * kPStride + (16 * kq + 4 * (l >> 4)) * 2) = pk;
      }
      // publish this wave's per-head maxima and whether it needs a new reference
      mw = xor32_max(xor16_max(mw));
      if (l < 16) s_red[kq][h] = mw;
      if (l == 0) s_flag[w] = any_over;
      lds_barrier();
      int flags = 0;
#pragma unroll
      for (int i = 0; i < kWaves8; ++i) flags |= s_flag[i];
      if (flags) {
        // new reference from all key quarters' maxima; running sum rescaled, P redone
        const float tm = vmax(vmax(s_red[0][h], s_red[1][h]), vmax(s_red[2][h], s_red[3][h]));
        const float m_new = vmax(m_ref, tm);
        const bool none = m_new == -INFINITY;
        const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        float ps = 0.f;
        bf16x4 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = none ? 0.f : __builtin_amdgcn_exp2f(s[i] - m_new);
          ps += p;
          pk[i] = (__bf16)p;
        }
        l_run = l_run * alpha + ps;
        m_ref = m_new;
        *reinterpret_cast<bf16x4 *>(s_p + h * kPStride + (16 * kq + 4 * (l >> 4)) * 2) = pk;
        if (kq == 0 && l < 16) s_alpha[h] = alpha;
        renorm = true;
        break;
      }
      l_run += psum;
      pv_tile(cur);
    }
    if (!renorm) break;
    // ---- rare path: rescale O by alpha (O is still zero on the first tile), then PV ----
    lds_barrier();
    if (t > 0) {
      const float a = s_alpha[l & 31];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[nb][i] *= a;
    }
    pv_tile((t & 1) ? s_kv1 : s_kv0);
    ++t;
  }

  // ---- epilogue: total softmax sums, normalise, write ----
  {
    float lr = l_run;
    lr = xor32_sum(xor16_sum(lr));
    const int h = 16 * hh + (l & 15);
    if (l < 16) s_red[kq][h] = lr;
    if (kq == 0 && l < 16) s_fm[h] = m_ref;
  }
  lds_barrier();
  if (tid < kHG) s_fl[tid] = s_red[0][tid] + s_red[1][tid] + s_red[2][tid] + s_red[3][tid];
  lds_barrier();

  {
    // lane: head l & 31; per block nb and group q, dims 32nb + 8q + 4(l>>5) .. +3 of this
    // wave's 64.  Staged through LDS (tile buffer 0 is free: the barriers above follow the
    // last tile) so each store instruction writes eight whole 128-byte head slices.
    const float lt = s_fl[l & 31];
    const float inv = lt > 0.f ? __builtin_amdgcn_rcpf(lt) : 0.f;
    uint8_t *stg = s_kv0 + w * kHG * kOStride;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(oacc[nb][4 * qd + e] * inv);
        *reinterpret_cast<bf16x4 *>(stg + (l & 31) * kOStride + 2 * (32 * nb + 8 * qd + 4 * (l >> 5))) = v;
      }
    __bf16 *dst = kSplit ? ws_o + (int64_t)split * num_rows * num_heads * kDV : out;
    dst += ((int64_t)row * num_heads + h0 + (l >> 3)) * kDV + 64 * w + 8 * (l & 7);
#pragma unroll
    for (int i = 0; i < kHG / 8; ++i)
      *reinterpret_cast<i32x4 *>(dst + 8 * i * kDV) =
          *reinterpret_cast<const i32x4 *>(stg + (8 * i + (l >> 3)) * kOStride + 16 * (l & 7));
  }
  if (tid < kHG) {
    const float m = s_fm[tid], lt = s_fl[tid];
    const int64_t hi = (int64_t)row * num_heads + h0 + tid;
    if constexpr (kSplit) {
      ws_ml[((int64_t)split * num_rows * num_heads + hi) * 2 + 0] = m;
      ws_ml[((int64_t)split * num_rows * num_heads + hi) * 2 + 1] = lt;
    } else if (lse != nullptr) {
      lse[hi] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

// Merge key-split partials: o = sum_s w_s o_s / sum_s w_s, w_s = l_s * 2^(m_s - max m).
// Partials o_s are normalised per split and stored in bf16; weights and sums stay fp32.
// Split-KV combine: one wave per (row, head); lane l owns value dims 8l..8l+7.  Splits are
// taken eight at a time with every load of a chunk issued before any is used; the running
// maximum moves up per chunk (weights are l_s * 2^(m_s - M)).
constexpr int kCombineChunk = 8;

__global__ __launch_bounds__(64) void attn_combine_kernel(const __bf16 *__restrict__ ws_o,
                                                         const float *__restrict__ ws_ml,
                                                         int32_t splits, int32_t num_rows,
                                                         int32_t num_heads,
                                                         __bf16 *__restrict__ out,
                                                         float *__restrict__ lse) {
  // (row, head) units in row-major order, XCD x (dispatch i runs on XCD i % 8) taking units
  // [x * per, (x + 1) * per): the XCD the attention kernel ran a row's splits on.
  const int64_t plane = (int64_t)num_rows * num_heads;
  const int64_t per = (plane + 7) / 8;
  const int64_t hi = (blockIdx.x & 7) * per + (blockIdx.x >> 3);  // row * num_heads + head
  if (hi >= plane) return;
  const int l = threadIdx.x;
  float M = -INFINITY, wsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += kCombineChunk) {
    float m[kCombineChunk], lt[kCombineChunk];
    bf16x8 v[kCombineChunk];
#pragma unroll
    for (int k = 0; k < kCombineChunk; ++k) {
      const int sk = s0 + k < splits ? s0 + k : splits - 1;
      const float2 ml = *reinterpret_cast<const float2 *>(ws_ml + (sk * plane + hi) * 2);
      m[k] = s0 + k < splits ? ml.x : -INFINITY;
      lt[k] = s0 + k < splits ? ml.y : 0.f;
      v[k] = *reinterpret_cast<const bf16x8 *>(ws_o + (sk * plane + hi) * kDV + 8 * l);
    }
    float Mc = M;
#pragma unroll
    for (int k = 0; k < kCombineChunk; ++k) Mc = vmax(Mc, m[k]);
    if (Mc == -INFINITY) continue;
    const float r = __builtin_amdgcn_exp2f(M - Mc);  // 0 when M was -inf
    wsum *= r;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= r;
    M = Mc;
#pragma unroll
    for (int k = 0; k < kCombineChunk; ++k) {
      const float wgt = lt[k] > 0.f ? lt[k] * __builtin_amdgcn_exp2f(m[k] - M) : 0.f;
      wsum += wgt;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wgt * (float)v[k][e];
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (__bf16)(acc[e] * inv);
  *reinterpret_cast<bf16x8 *>(out + hi * kDV + 8 * l) = o;
  if (lse != nullptr && l == 0) lse[hi] = wsum > 0.f ? (M + __log2f(wsum)) * kLn2 : -INFINITY;
}

// ---- fp32 path: one wave per (row, head) ----
constexpr int kF32MaxTopk = 8192;
constexpr int kF32MaxD = 1024;

__global__ __launch_bounds__(64) void attn_f32_kernel(const float *__restrict__ q,
                                                      const float *__restrict__ kv, int64_t kv_rows,
                                                      const int32_t *__restrict__ indices,
                                                      int32_t num_heads, int32_t d_qk, int32_t d_v,
                                                      int32_t topk, float scale,
                                                      float *__restrict__ out,
                                                      float *__restrict__ lse) {
  __shared__ float s_score[kF32MaxTopk];
  const int64_t hi = blockIdx.x;  // row * num_heads + head
  const int64_t row = hi / num_heads;
  const int l = threadIdx.x;
  const float *qv = q + hi * d_qk;
  const int32_t *idx = indices + row * topk;
  float qr[kF32MaxD / 64];
#pragma unroll
  for (int k = 0; k < kF32MaxD / 64; ++k) qr[k] = (64 * k + l < d_qk) ? qv[64 * k + l] : 0.f;

  float m = -INFINITY;
  for (int j = 0; j < topk; ++j) {
    const int r = idx[j];
    float sc = -INFINITY;
    if (r >= 0 && r < kv_rows) {
      const float *kr = kv + (int64_t)r * d_qk;
      float part = 0.f;
#pragma unroll
      for (int k = 0; k < kF32MaxD / 64; ++k)
        if (64 * k + l < d_qk) part = fmaf(qr[k], kr[64 * k + l], part);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
      sc = part * scale;
    }
    if (l == 0) s_score[j] = sc;
    m = vmax(m, sc);
  }
  __syncthreads();
  float lsum = 0.f;
  for (int j = l; j < topk; j += 64) lsum += s_score[j] == -INFINITY ? 0.f : expf(s_score[j] - m);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, 64);
  float acc[kF32MaxD / 64];
#pragma unroll
  for (int k = 0; k < kF32MaxD / 64; ++k) acc[k] = 0.f;
  for (int j = 0; j < topk; ++j) {
    const float sc = s_score[j];
    if (sc == -INFINITY) continue;
    const float p = expf(sc - m);
    const float *vr = kv + (int64_t)idx[j] * d_qk;
#pragma unroll
    for (int k = 0; k < kF32MaxD / 64; ++k)
      if (64 * k + l < d_v) acc[k] = fmaf(p, vr[64 * k + l], acc[k]);
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
  for (int k = 0; k < kF32MaxD / 64; ++k)
    if (64 * k + l < d_v) out[hi * d_v + 64 * k + l] = acc[k] * inv;
  if (lse != nullptr && l == 0) lse[hi] = lsum > 0.f ? m + logf(lsum) : -INFINITY;
}

}  // namespace

void launch_attn_combine(const __bf16 *ws_o, const float *ws_ml, int32_t splits, int32_t num_rows,
                         int32_t num_heads, __bf16 *out, float *lse, hipStream_t stream) {
  const int units = num_rows * num_heads;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((units + 7) / 8 * 8), dim3(64), 0, stream, ws_o,
                     ws_ml, splits, num_rows, num_heads, out, lse);
}

// The launch for `cus` compute units: every attention workgroup holds one CU (its LDS), so
// the grid is sized for one round of `cus` workgroups where the batch allows.
static AttnPlan plan_for(int64_t rows, int64_t heads, int64_t keys, int64_t cus,
                         int64_t max_splits) {
  AttnPlan p;
  // 64 heads per workgroup (each gathered tile serves twice as many heads) once there are
  // enough (row, 64-head) groups; the 32-head kernel has the shorter critical path for
  // small batches.
  p.heads_per_wg = (heads % 64 == 0 && rows * (heads / 64) * kNumCUs >= kMinGroups64 * cus) ? 64 : kHG;
  if (heads % 128 == 0 && 2 * rows * (heads / 128) > cus) p.heads_per_wg = 128;
  const int64_t groups = rows * (heads / p.heads_per_wg);
  // Key splits: as many as still fit the CUs in one round of workgroups (a workgroup more
  // would wait for a second round), none shorter than two tiles, and at least enough that
  // no split holds more than kMaxKeysPerSplit keys.  Doubling the split count while the grid
  // was below 256 gave 384-496 workgroups at 12-31 and 40-96 rows of 128 heads; one round
  // instead measured 12-30 % faster there (1 and 2 rows 7-10 % faster with two-tile splits
  // instead of four), and the same at 8, 16, 32 and 64 rows.
  const int64_t min_keys = 2 * kTK;
  const int64_t fit = groups > 0 ? cus / groups : 1, longest = keys / min_keys;
  int64_t splits = fit < longest ? fit : longest;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  const int64_t at_least = (keys + kMaxKeysPerSplit - 1) / kMaxKeysPerSplit;
  if (splits < at_least) splits = at_least;
  int64_t kps = (keys + splits - 1) / splits;
  kps = (kps + kTK - 1) / kTK * kTK;
  splits = (keys + kps - 1) / kps;
  p.splits = (int)splits;
  p.keys_per_split = (int)kps;
  // bf16 partial outputs, then fp32 (max, sum) pairs
  p.workspace = splits > 1 ? (size_t)splits * rows * heads * (kDV * 2 + 2 * sizeof(float)) : 0;
  return p;
}

AttnPlan plan_attn_bf16(int32_t num_rows, int32_t num_heads, int32_t topk, int32_t max_cus) {
  // (64-bit arithmetic: the callers bound the sizes, this keeps any int32 input defined)
  const int64_t rows = num_rows, heads = num_heads, keys = topk;
  const AttnPlan whole = plan_for(rows, heads, keys, kNumCUs, keys);
  if (max_cus >= kNumCUs) return whole;
  // Fewer CUs: never more key splits than the whole-GPU plan (the workspace is splits x
  // rows x heads partials for every kernel), so its workspace (hs_attn_workspace_bytes)
  // serves every call.
  return plan_for(rows, heads, keys, max_cus > 0 ? max_cus : 1, whole.splits);
}

template <bool kPaged>
static hipError_t launch_attn32(const __bf16 *qb, const uint8_t *kvb, int64_t kv_rows,
                                const int32_t *indices, int32_t num_rows, int32_t num_heads,
                                int32_t topk, float scale_log2, __bf16 *ob, float *lse,
                                void *workspace, const AttnPlan &plan, const PagedMap &pg,
                                const AltSource &alt, hipStream_t stream) {
  const int units = num_rows * plan.splits * (num_heads / kHG);
  const int grid = (units + 7) / 8 * 8;
  if (plan.splits == 1) {
    hipLaunchKernelGGL((attn_bf16_kernel<false, kPaged>), dim3(grid), dim3(kThreads8), 0, stream,
                       qb, kvb, kv_rows, indices, num_rows, num_heads, topk, plan.keys_per_split,
                       1, scale_log2, ob, lse, nullptr, nullptr, pg, alt);
    return hipGetLastError();
  }
  __bf16 *ws_o = static_cast<__bf16 *>(workspace);
  float *ws_ml = reinterpret_cast<float *>(ws_o + (size_t)plan.splits * num_rows * num_heads * kDV);
  hipLaunchKernelGGL((attn_bf16_kernel<true, kPaged>), dim3(grid), dim3(kThreads8), 0, stream, qb,
                     kvb, kv_rows, indices, num_rows, num_heads, topk, plan.keys_per_split,
                     plan.splits, scale_log2, ob, lse, ws_o, ws_ml, pg, alt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_attn_combine(ws_o, ws_ml, plan.splits, num_rows, num_heads, ob, lse, stream);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const void *q, const void *kv, int64_t kv_rows, const int32_t *indices,
                            int32_t num_rows, int32_t num_heads, int32_t topk, float scale,
                            void *out, float *lse, void *workspace, const AttnPlan &plan,
                            const PagedMap *paged, const AltSource *alt, hipStream_t stream) {
  if (plan.heads_per_wg == 128)
    return launch_attn128(q, kv, kv_rows, indices, num_rows, num_heads, topk, scale, out, lse,
                          workspace, plan, paged, alt, stream);
  if (plan.heads_per_wg == 64)
    return launch_attn64(q, kv, kv_rows, indices, num_rows, num_heads, topk, scale, out, lse,
                         workspace, plan, paged, alt, stream);
  const float scale_log2 = scale * 1.44269504088896340736f;
  const __bf16 *qb = static_cast<const __bf16 *>(q);
  const uint8_t *kvb = static_cast<const uint8_t *>(kv);
  __bf16 *ob = static_cast<__bf16 *>(out);
  if (paged != nullptr)
    return launch_attn32<true>(qb, kvb, kv_rows, indices, num_rows, num_heads, topk, scale_log2, ob,
                               lse, workspace, plan, *paged, AltSource{}, stream);
  return launch_attn32<false>(qb, kvb, kv_rows, indices, num_rows, num_heads, topk, scale_log2, ob,
                              lse, workspace, plan, PagedMap{},
                              alt ? *alt : AltSource{}, stream);
}

hipError_t launch_attn_f32(const float *q, const float *kv, int64_t kv_rows, const int32_t *indices,
                           int32_t num_rows, int32_t num_heads, int32_t d_qk, int32_t d_v,
                           int32_t topk, float scale, float *out, float *lse, hipStream_t stream) {
  hipLaunchKernelGGL(attn_f32_kernel, dim3(num_rows * num_heads), dim3(64), 0, stream, q, kv,
                     kv_rows, indices, num_heads, d_qk, d_v, topk, scale, out, lse);
  return hipGetLastError();
}

int attn_f32_max_topk() { return kF32MaxTopk; }
int attn_f32_max_d() { return kF32MaxD; }

}  // namespace hs
