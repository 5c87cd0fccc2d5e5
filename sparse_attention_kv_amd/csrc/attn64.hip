// sparse_decode_attn, 64 heads per workgroup (gfx950).
//
// P1 "hiSparse-MTP", "1. 启动阶段": the DSA attention backend reads KV through HiSparse.
// P3 "vllm 分析（十二）——Hisparse下篇", resolve_topk listing: attention gets the cache and
// per-row indices (-1 padded) and reads only those rows.
//
// Workgroup = (query row, group of 64 heads, key split); 4 waves, each owning 16 heads end
// to end, so a gathered KV tile serves 64 heads and every wave's softmax is its own:
//   * tiles of 64 selected rows are gathered direct-to-LDS and double buffered; the 18
//     slot issues for the next tile are spread one per k-step over QK^T, so the texture
//     path works while the matrix cores do.  Tile layout (below) puts the 16 keys a wave
//     gathers in its own 18 KiB region, so a lane needs two row indices per tile;
//   * S^T (64 keys x the wave's 16 heads) = K Q^T with v_mfma_f32_16x16x32_bf16, four
//     16-key blocks per k-step, Q resident in registers (72 VGPRs);
//   * a lane holds 16 scores of one head (4 lanes per head): the head maximum takes two
//     cross-lane steps; the reference maximum moves lazily (see tile::kRescaleSlack);
//   * O^T (512 dims x 16 heads) += V^T P^T with v_mfma_f32_16x16x32_bf16: the k-slots of
//     the P^T operand are the keys a lane already holds, V^T is read with two transposed
//     8-byte LDS reads per MFMA; O stays in 128 accumulation registers;
//   * one workgroup barrier per tile (buffer reuse); the epilogue stages O through LDS so
//     each store instruction writes whole 1 KiB head rows.

#include "attn_tile.h"

namespace hs {
namespace {

using namespace tile;

constexpr int kHW = 16;                 // heads per wave
constexpr int kH64 = kHW * kWaves;      // heads per workgroup
constexpr int kKSteps = kD / 32;        // 18 k-steps of 32 over the latent row
constexpr int kNB = kDV / 16;           // 32 value-dim blocks of 16
constexpr int kVDepth = 6;              // V operand ring: value blocks in flight
constexpr int kOStride = kDV * 2 + 16;  // epilogue staging row stride in bytes
static_assert(kKSteps == kLoadsPerThread, "one gather slot per k-step");
static_assert(kWaves * kHW * kOStride <= kTileBytes, "O staging fits one tile buffer");

// Part (0..3) of a 32-dim k-step that lane group G of an MFMA operand holds.  Any order
// works as long as K and Q agree; this one keeps the K reads free of bank conflicts.
__device__ __forceinline__ int kPartOf(int g) { return ((g & 1) << 1) | (g >> 1); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Tile layout: the 16-byte part p (0..71) of tile key k (0..63) sits at byte
//   18432 (k >> 4) + 9216 h + 1024 (p >> 3) + 16 ((k & 7) + 8 ((p & 7) ^ h)),  h = (k >> 3) & 1.
// Wave w gathers keys 16w .. 16w+15 as 18 one-KiB slots (h, p >> 3): lane l of a slot
// brings part 8 (p >> 3) + ((l >> 3) ^ h) of key 16w + 8h + (l & 7), i.e. 8 rows x 128 B
// per instruction.  A 16-byte LDS read serves the lane octets in the pairs (0,3), (1,2),
// (4,7), (5,6); a pair is conflict free when it covers 256 distinct bytes mod 256.  The
// QK^T operand reads let lane group G take part 4 ks + kPartOf(G) (Q uses the same order),
// which gives every octet pair both 128-byte halves; the transposed PV reads of a half
// wave cover 256 distinct bytes.  So no LDS bank conflicts, and every access of a k-step
// or value block is base + immediate.
constexpr int kRegionBytes = 16 * kRowBytes;  // 18432: one wave's 16 keys
constexpr int kHalfBytes = 8 * kRowBytes;     // 9216: 8 keys

__device__ __forceinline__ void gather64(const uint8_t *__restrict__ kv, const int32_t *sidx,
                                         int n_valid, int t, uint8_t *dst, int w, int l) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kk = t * kTK + 16 * w + 8 * h + (l & 7);
    const int row = sidx[kk < n_valid - 1 ? kk : n_valid - 1];
    const uint8_t *src = kv + (int64_t)row * kRowBytes + 16 * ((l >> 3) ^ h);
#pragma unroll
    for (int pg = 0; pg < 9; ++pg)
      dma16(src + 128 * pg, dst + w * kRegionBytes + h * kHalfBytes + 1024 * pg);
  }
}

template <bool kSplit, bool kPaged>
__global__ __launch_bounds__(kThreads, 1) void attn64_kernel(
    const __bf16 *__restrict__ q, const uint8_t *__restrict__ kv, int64_t kv_rows,
    const int32_t *__restrict__ indices, int32_t num_rows, int32_t num_heads, int32_t topk,
    int32_t keys_per_split, int32_t splits, int32_t units, float scale_log2,
    __bf16 *__restrict__ out, float *__restrict__ lse, __bf16 *__restrict__ ws_o,
    float *__restrict__ ws_ml, PagedMap pg, AltSource alt) {
  __shared__ __attribute__((aligned(16))) uint8_t s_kv0[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_kv1[kTileBytes];
  __shared__ __attribute__((aligned(16))) int32_t s_sidx[kMaxKeysPerSplit];
  __shared__ int s_scan[kWaves];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  // Dispatch i runs on XCD i % 8; XCD x takes units [x * per, (x + 1) * per).  Units are
  // ordered (row, split, head group), so the head groups and splits of a row share one
  // L2 for its KV rows and its Q.
  const int per = (units + 7) / 8;
  const int u = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (u >= units) return;
  const int n_hg = num_heads / kH64;
  const int hg = u % n_hg;
  const int split = (u / n_hg) % splits;
  const int row = u / (n_hg * splits);
  if (alt.row_sel != nullptr && alt.row_sel[row] != 0) {  // this row reads the second source
    kv = alt.kv;
    kv_rows = alt.kv_rows;
    indices = alt.indices;
  }
  const int hw = hg * kH64 + kHW * w;  // first head of this wave
  const int kbeg = split * keys_per_split;
  const int kcnt = max(0, min(keys_per_split, topk - kbeg));

  // ---- indices (or token positions) of this split: they gate the first gather ----
  const int32_t *irow = indices + (int64_t)row * topk + kbeg;
  const int pk = (kcnt + kThreads - 1) / kThreads;  // <= 8
  int vals[kMaxKeysPerSplit / kThreads];
  load_split_indices<kPaged>(irow, pk, kcnt, tid, pg, row, vals);
  // ---- Q of the wave's 16 heads: B operand of S^T = K Q^T (head l&15, dims 32ks +
  // 8 kPartOf(l>>4) ..) ----
  bf16x8 qreg[kKSteps];
  {
    const __bf16 *qh = q + ((int64_t)row * num_heads + hw + (l & 15)) * kD + 8 * kPartOf(l >> 4);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qreg[ks] = *reinterpret_cast<const bf16x8 *>(qh + 32 * ks);
  }
  // ---- compact the valid indices into LDS (order preserved) ----
  int n_valid;
  {
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kMaxKeysPerSplit / kThreads; ++k) {
      const bool ok = vals[k] >= 0 && vals[k] < kv_rows;
      vals[k] = ok ? vals[k] : -1;
      cnt += ok;
    }
    int wave_total;
    static_assert(kMaxKeysPerSplit / kThreads <= kSmallScanMax, "per-lane key count fits the scan");
    const int ex = wave_exclusive_scan_small(cnt, wave_total);
    if (l == 0) s_scan[w] = wave_total;
    lds_barrier();
    int base = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const int c = s_scan[i];
      base += i < w ? c : 0;
      total += c;
    }
    int pos = base + ex;
#pragma unroll
    for (int k = 0; k < kMaxKeysPerSplit / kThreads; ++k)
      if (vals[k] >= 0) s_sidx[pos++] = vals[k];
    n_valid = total;
    lds_barrier();
  }
  const int ntiles = (n_valid + kTK - 1) / kTK;
  if (ntiles > 0) gather64(kv, s_sidx, n_valid, 0, s_kv0, w, l);

  f32x4 oacc[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[nb][i] = 0.f;
  float m_ref = -INFINITY;  // reference maximum of head (l & 15), log2 domain
  float l_run = 0.f;        // this lane's share of that head's softmax sum
  const int G = l >> 4;

  // K operand (A of S^T): lane l reads key 16kb + (l&15), part 4ks + kPartOf(G), which the
  // tile layout puts at kb region + 9216 h + 16 ((l & 7) + 8 (kPartOf(G) ^ h)) + 512 ks.
  const int hl = (l >> 3) & 1;
  const int k_off = hl * kHalfBytes + 16 * ((l & 7) + 8 * (kPartOf(G) ^ hl));

  // O^T += V^T P^T for one tile.  p[4kb + r] is the probability of key 16kb + 4G + r.
  // PV step st covers keys 32st .. 32st + 31; its k-slots for lane group G are keys
  // 32st + 4G + {0..3} (p[8st + 0..3]) then 32st + 16 + 4G + {0..3} (p[8st + 4..7]).
  // V^T for dims 16nb + j (j = l & 15, r = j >> 2, c = j & 3): a transposed read at key
  // row key_base + r, bytes 32nb + 8c .. +7 (part 2nb + (c >> 1)) gives lane j the 4 keys
  // at dim 16nb + j.  In the tile layout that is base(key row) + 256 nb with
  // base = region + 9216 h + 16 (key & 7) + 128 ((c >> 1) ^ h) + 8 (c & 1).
  auto pv_tile = [&](const uint8_t *cur, const float (&p)[16]) {
    const int j = l & 15, r = j >> 2, c = j & 3;
    const int h = G >> 1;                   // key & 15 = 4G + r
    const int v_off = h * kHalfBytes + 16 * (4 * (G & 1) + r) + 128 * ((c >> 1) ^ h) + 8 * (c & 1);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      bf16x8 pa;
#pragma unroll
      for (int e = 0; e < 8; ++e) pa[e] = (__bf16)p[8 * st + e];
      const uint8_t *blo = cur + (2 * st) * kRegionBytes + v_off;      // keys 32st + 4G + r
      const uint8_t *bhi = cur + (2 * st + 1) * kRegionBytes + v_off;  // keys 32st + 16 + 4G + r
      // Ring of kVDepth value fragments: the reads for block nb + kVDepth go out right after
      // block nb's MFMA (one wave per SIMD: nothing else covers LDS latency); the scheduling
      // barriers keep that order.
      s16x4 vlo[kVDepth], vhi[kVDepth];
      auto load_v = [&](int nb, int bb) {
        vlo[bb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HS_LDS s16x4 *)(blo + 256 * nb));
        vhi[bb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HS_LDS s16x4 *)(bhi + 256 * nb));
      };
#pragma unroll
      for (int i = 0; i < kVDepth; ++i) load_v(i, i);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const int bb = nb % kVDepth;
        const s16x8 vv = {vlo[bb][0], vlo[bb][1], vlo[bb][2], vlo[bb][3],
                          vhi[bb][0], vhi[bb][1], vhi[bb][2], vhi[bb][3]};
        __builtin_amdgcn_sched_barrier(0);
        oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pa,
                                                           oacc[nb], 0, 0, 0);
        if (nb + kVDepth < kNB) load_v(nb + kVDepth, bb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // The inner loop touches O only through MFMA; a tile that needs a new reference (always
  // the first) leaves it, O is rescaled once outside, and the loop resumes.
  int t = 0;
  while (t < ntiles) {
    bool renorm = false;
    float p[16];
    float alpha = 1.f;
    for (; t < ntiles; ++t) {
      const uint8_t *cur = (t & 1) ? s_kv1 : s_kv0;
      uint8_t *nxt = (t & 1) ? s_kv0 : s_kv1;
      wait_vmem();
      lds_barrier();
      const bool more = t + 1 < ntiles;
      // next tile's two source rows of this lane (8-key halves h = 0, 1 of the wave's keys)
      const uint8_t *gsrc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kk = (t + 1) * kTK + 16 * w + 8 * h + (l & 7);
        const int row = more ? s_sidx[kk < n_valid - 1 ? kk : n_valid - 1] : 0;
        gsrc[h] = kv + (int64_t)row * kRowBytes + 16 * ((l >> 3) ^ h);
      }
      uint8_t *gdst = nxt + w * kRegionBytes;

      // ---- S^T: 4 blocks of 16 keys x 16 heads, k-steps of 32 dims ----
      f32x4 sacc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[kb][i] = 0.f;
      {
        const uint8_t *kbase = cur + k_off;
        bf16x8 kf[3][4];
        auto load_k = [&](int ks, int buf) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            kf[buf][kb] = *reinterpret_cast<const bf16x8 *>(kbase + kb * kRegionBytes + 512 * ks);
        };
        load_k(0, 0);
        load_k(1, 1);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
          if (ks + 2 < kKSteps) load_k(ks + 2, (ks + 2) % 3);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks % 3][kb], qreg[ks], sacc[kb], 0, 0, 0);
          // slot ks: half ks / 9, parts 8 (ks % 9) ..
          if (more) dma16(gsrc[ks / 9] + 128 * (ks % 9), gdst + (ks / 9) * kHalfBytes + 1024 * (ks % 9));
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- scores of head (l & 15): lane holds keys 16kb + 4G + r of the tile ----
      float s[16];
      const int kq = t * kTK + 4 * G;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = (kq + 16 * kb + r < n_valid) ? sacc[kb][r] * scale_log2 : -INFINITY;
          s[4 * kb + r] = v;
          mx = vmax(mx, v);
        }
      mx = xor32_max(xor16_max(mx));
      const bool over = mx > m_ref + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(over) != 0) {
        // new reference for the heads whose maximum moved up (rare after the first tile)
        alpha = over ? __builtin_amdgcn_exp2f(m_ref - mx) : 1.f;
        m_ref = over ? mx : m_ref;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[i] = __builtin_amdgcn_exp2f(s[i] - m_ref);
          l_run += p[i];
        }
        renorm = true;
        break;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s[i] - m_ref);
        l_run += p[i];
      }
      pv_tile(cur, p);
    }
    if (!renorm) break;
    // ---- rare path: rescale O by this lane's head factor, then this tile's PV ----
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[nb][i] *= alpha;
    pv_tile((t & 1) ? s_kv1 : s_kv0, p);
    ++t;
  }

  // ---- epilogue: head sums, normalise, stage O^T -> LDS rows, whole-row stores ----
  float lt = l_run;
  lt = xor32_sum(xor16_sum(lt));
  const float inv = lt > 0.f ? __builtin_amdgcn_rcpf(lt) : 0.f;
  lds_barrier();  // every wave is done with the tile buffers
  uint8_t *stg = s_kv0 + w * kHW * kOStride;
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (__bf16)(oacc[nb][i] * inv);
    *reinterpret_cast<bf16x4 *>(stg + (l & 15) * kOStride + (16 * nb + 4 * G) * 2) = v;
  }
  __bf16 *dst = kSplit ? ws_o + (int64_t)split * num_rows * num_heads * kDV : out;
  dst += ((int64_t)row * num_heads + hw) * kDV + 8 * l;
#pragma unroll
  for (int hh = 0; hh < kHW; ++hh)
    *reinterpret_cast<i32x4 *>(dst + hh * kDV) =
        *reinterpret_cast<const i32x4 *>(stg + hh * kOStride + 16 * l);
  if (l < kHW) {
    const int64_t hi = (int64_t)row * num_heads + hw + l;
    if constexpr (kSplit) {
      ws_ml[((int64_t)split * num_rows * num_heads + hi) * 2 + 0] = m_ref;
      ws_ml[((int64_t)split * num_rows * num_heads + hi) * 2 + 1] = lt;
    } else if (lse != nullptr) {
      lse[hi] = lt > 0.f ? (m_ref + __log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

template <bool kPaged>
static hipError_t launch64(const __bf16 *qb, const uint8_t *kvb, int64_t kv_rows,
                           const int32_t *indices, int32_t num_rows, int32_t num_heads, int32_t topk,
                           float scale_log2, __bf16 *ob, float *lse, void *workspace,
                           const AttnPlan &plan, const PagedMap &pg,
                            const AltSource &alt, hipStream_t stream) {
  const int units = num_rows * (num_heads / kH64) * plan.splits;
  const int grid = (units + 7) / 8 * 8;
  if (plan.splits == 1) {
    hipLaunchKernelGGL((attn64_kernel<false, kPaged>), dim3(grid), dim3(kThreads), 0, stream, qb,
                       kvb, kv_rows, indices, num_rows, num_heads, topk, plan.keys_per_split, 1,
                       units, scale_log2, ob, lse, nullptr, nullptr, pg, alt);
    return hipGetLastError();
  }
  __bf16 *ws_o = static_cast<__bf16 *>(workspace);
  float *ws_ml = reinterpret_cast<float *>(ws_o + (size_t)plan.splits * num_rows * num_heads * kDV);
  hipLaunchKernelGGL((attn64_kernel<true, kPaged>), dim3(grid), dim3(kThreads), 0, stream, qb, kvb,
                     kv_rows, indices, num_rows, num_heads, topk, plan.keys_per_split, plan.splits,
                     units, scale_log2, ob, lse, ws_o, ws_ml, pg, alt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_attn_combine(ws_o, ws_ml, plan.splits, num_rows, num_heads, ob, lse, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn64(const void *q, const void *kv, int64_t kv_rows, const int32_t *indices,
                         int32_t num_rows, int32_t num_heads, int32_t topk, float scale, void *out,
                         float *lse, void *workspace, const AttnPlan &plan, const PagedMap *paged,
                          const AltSource *alt, hipStream_t stream) {
  const float scale_log2 = scale * 1.44269504088896340736f;
  const __bf16 *qb = static_cast<const __bf16 *>(q);
  const uint8_t *kvb = static_cast<const uint8_t *>(kv);
  __bf16 *ob = static_cast<__bf16 *>(out);
  if (paged != nullptr)
    return launch64<true>(qb, kvb, kv_rows, indices, num_rows, num_heads, topk, scale_log2, ob, lse,
                          workspace, plan, *paged, AltSource{}, stream);
  return launch64<false>(qb, kvb, kv_rows, indices, num_rows, num_heads, topk, scale_log2, ob, lse,
                         workspace, plan, PagedMap{},
                          alt ? *alt : AltSource{}, stream);
}

}  // namespace hs
