// sparse_decode_attn, 128 heads per workgroup (gfx950): the large-batch kernel.
//
// P1 "hiSparse-MTP", "1. 启动阶段": the DSA attention backend reads KV through HiSparse.
// P3 "vllm 分析（十二）——Hisparse下篇", resolve_topk listing: attention gets the cache and
// per-row indices (-1 padded) and reads only those rows.
//
// Workgroup = (query row, 128 heads, key split); 4 waves, each owning 32 heads end to end,
// so every gathered KV tile serves all 128 heads of its row once:
//   * tiles of 64 selected rows are gathered direct-to-LDS and double buffered; a wave's
//     18 slot issues for the next tile are spread over the S^T phases of its two 32-key
//     blocks, one every other k-step pair;
//   * per 32-key block: S^T (32 keys x the wave's 32 heads) = K Q^T with
//     v_mfma_f32_32x32x16_bf16, Q resident in 144 VGPRs, two accumulator chains;
//   * a lane holds 16 scores of one head: the head maximum takes one cross-half step; the
//     reference maximum moves lazily (tile::kRescaleSlack);
//   * O^T (512 dims x 32 heads) += V^T P^T with v_mfma_f32_32x32x16_bf16: the k-slots of
//     the P^T operand are the keys the lane already holds, V^T comes from two transposed
//     8-byte LDS reads per MFMA; O lives in the 256 accumulation registers;
//   * one workgroup barrier per tile (buffer reuse); the epilogue stages O through LDS so
//     each store instruction writes a whole 1 KiB head row.
// The compiler gives every MFMA result of a kernel one register class; O must be in the
// accumulation registers, so the S^T MFMAs are written as inline asm on VGPRs, with the
// wait states the matrix pipeline requires around them (mfma_s / mfma_s_drain).

#include "attn_tile.h"

namespace hs {
namespace {

using namespace tile;

constexpr int kHW = 32;                  // heads per wave
constexpr int kH128 = kHW * kWaves;      // heads per workgroup
constexpr int kKS = kD / 16;             // 36 k-steps of 16 over the latent row
constexpr int kNB = kDV / 32;            // 16 value-dim blocks of 32
constexpr int kKDepth = 3;               // K operand ring: k-step pairs in flight + 1
constexpr int kVDepth = 4;               // V operand ring: value blocks in flight
constexpr int kOStride = kDV * 2 + 16;   // epilogue staging row stride in bytes
static_assert(kWaves * kHW * kOStride <= 2 * kTileBytes, "O staging fits the two tile buffers");

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Tile layout.  The 16-byte part p (0..71) of tile key k (0..63) sits at byte
//   18432 (k >> 4) + 9216 h + 1024 (p >> 3) + 16 (((k & 7) ^ 4 b) + 8 ((p & 7) ^ h)),
// with h = (k >> 3) & 1 and b = (p >> 1) & 1.  Wave w gathers keys 16w .. 16w+15 as 18
// one-KiB slots (h, p >> 3); lane l of a slot brings part 8 (p >> 3) + ((l >> 3) ^ h) of key
// 16w + 8h + ((l & 7) ^ 4 b).  S^T operand reads (32 keys x one part) and the transposed PV
// reads both cover 256 distinct bytes per half wave: no bank conflicts, and each k-step or
// value block is base + immediate.
constexpr int kRegionBytes = 16 * kRowBytes;  // 18432: 16 keys
constexpr int kHalfBytes = 8 * kRowBytes;     // 9216: 8 keys

__device__ __forceinline__ void gather128_half(const uint8_t *__restrict__ kv, const int32_t *sidx,
                                               int n_valid, int t, uint8_t *dst, int w, int l,
                                               int h, const uint8_t *&src) {
  const int pp = (l >> 3) ^ h;  // part & 7 this lane brings
  const int k7 = (l & 7) ^ (4 * ((pp >> 1) & 1));
  const int kk = t * kTK + 16 * w + 8 * h + k7;
  const int row = sidx[kk < n_valid - 1 ? kk : n_valid - 1];
  src = kv + (int64_t)row * kRowBytes + 16 * pp;
  (void)dst;
}

// S^T accumulation on VGPRs.  Wait states (gfx950 matrix pipeline): the leading s_nop covers
// a vector-ALU write of an operand just before the asm (copies the compiler may insert); the
// trailing one covers a later overwrite of the A/B operands; mfma_s_drain covers the
// result -> vector-ALU read latency of the last MFMA of a chain.
__device__ __forceinline__ void mfma_s0(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0\n\ts_nop 4"
               : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 4"
               : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_drain(f32x16 &a, f32x16 &b) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b));
}

template <bool kSplit, bool kPaged>
__global__ __launch_bounds__(kThreads, 1) void attn128_kernel(
    const __bf16 *__restrict__ q, const uint8_t *__restrict__ kv, int64_t kv_rows,
    const int32_t *__restrict__ indices, int32_t num_rows, int32_t num_heads, int32_t topk,
    int32_t keys_per_split, int32_t splits, int32_t units, float scale_log2,
    __bf16 *__restrict__ out, float *__restrict__ lse, __bf16 *__restrict__ ws_o,
    float *__restrict__ ws_ml, PagedMap pg, AltSource alt) {
  __shared__ __attribute__((aligned(16))) uint8_t s_kv[2 * kTileBytes];
  __shared__ __attribute__((aligned(16))) int32_t s_sidx[kMaxKeysPerSplit];
  __shared__ int s_scan[kWaves];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  // Dispatch i runs on XCD i % 8; XCD x takes units [x * per, (x + 1) * per); units are
  // ordered (row, split, head group).
  const int per = (units + 7) / 8;
  const int u = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (u >= units) return;
  const int n_hg = num_heads / kH128;
  const int hg = u % n_hg;
  const int split = (u / n_hg) % splits;
  const int row = u / (n_hg * splits);
  if (alt.row_sel != nullptr && alt.row_sel[row] != 0) {  // this row reads the second source
    kv = alt.kv;
    kv_rows = alt.kv_rows;
    indices = alt.indices;
  }
  const int hw = hg * kH128 + kHW * w;  // first head of this wave
  const int kbeg = split * keys_per_split;
  const int kcnt = max(0, min(keys_per_split, topk - kbeg));

  // ---- indices (or token positions) of this split: they gate the first gather ----
  const int32_t *irow = indices + (int64_t)row * topk + kbeg;
  const int pk = (kcnt + kThreads - 1) / kThreads;  // <= 8
  int vals[kMaxKeysPerSplit / kThreads];
  load_split_indices<kPaged>(irow, pk, kcnt, tid, pg, row, vals);
  // ---- Q of the wave's 32 heads: B operand of S^T (head l&31, dims 16ks + 8(l>>5) ..) ----
  bf16x8 qreg[kKS];
  const __bf16 *qh = q + ((int64_t)row * num_heads + hw + (l & 31)) * kD + 8 * (l >> 5);
  auto load_q = [&]() {
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qreg[ks] = *reinterpret_cast<const bf16x8 *>(qh + 16 * ks);
  };
  load_q();
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
  if (ntiles > 0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint8_t *src;
      gather128_half(kv, s_sidx, n_valid, 0, s_kv, w, l, h, src);
#pragma unroll
      for (int pg = 0; pg < 9; ++pg)
        dma16(src + 128 * pg, s_kv + w * kRegionBytes + h * kHalfBytes + 1024 * pg);
    }
  }

  f32x16 oacc[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[nb][i] = 0.f;
    asm volatile("" : "+a"(oacc[nb]));  // O lives in the accumulation registers
  }
  float m_ref = -INFINITY;  // reference maximum of head (l & 31), log2 domain
  float l_run = 0.f;        // this lane's share of that head's softmax sum
  const int g = l >> 5;     // lane half
  const int G = l >> 4;     // 16-lane group

  // S^T A operand: lane l reads key 32kb + (l & 31), part 2ks + g.  In the tile layout that
  // is kbase[ks & 1] + 256 ks (two base pointers per block: the key XOR depends on ks & 1).
  const int hk = (l >> 3) & 1;
  const int k_off = 18432 * ((l >> 4) & 1) + 9216 * hk + 128 * (g ^ hk);
  // V^T for dims 32nb + 16(G&1) + j (j = l & 15, r = j >> 2, c = j & 3): a transposed read
  // at key row 16st + 4(G>>1) + r (+8 for the second read) gives lane j the 4 keys at its
  // dim; in the tile layout that is vbase[st][hi] + 512 nb.
  const int vr = (l & 15) >> 2, vc = l & 3;
  const int v_off = 64 * ((G >> 1) ^ (G & 1)) + 16 * vr + 256 * (G & 1) + 8 * (vc & 1);

  // O^T += V^T P^T for one 32-key block kb of tile buffer `cur`; p[i] is the probability
  // of key 8(i>>2) + 4g + (i&3) of the block for head (l & 31).
  auto pv_block = [&](const uint8_t *cur, int kb, const float (&p)[16]) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      bf16x8 pa;
#pragma unroll
      for (int e = 0; e < 8; ++e) pa[e] = (__bf16)p[8 * st + e];
      // keys 32kb + 16st + ..: region 2kb + st; hi read is the h = 1 half (keys +8)
      const uint8_t *blo = cur + (2 * kb + st) * kRegionBytes + v_off + 128 * ((vc >> 1) ^ 0);
      const uint8_t *bhi = cur + (2 * kb + st) * kRegionBytes + kHalfBytes + v_off + 128 * ((vc >> 1) ^ 1);
      // A ring of kVDepth value fragments: the reads for block nb + kVDepth go out right after
      // block nb's MFMA, so each read has kVDepth - 1 MFMAs to land (one wave per SIMD has
      // no other wave to cover LDS latency).  The scheduling barriers keep that order.
      s16x4 vlo[kVDepth], vhi[kVDepth];
      auto load_v = [&](int nb, int bb) {
        vlo[bb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HS_LDS s16x4 *)(blo + 512 * nb));
        vhi[bb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HS_LDS s16x4 *)(bhi + 512 * nb));
      };
#pragma unroll
      for (int i = 0; i < kVDepth; ++i) load_v(i, i);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const int bb = nb % kVDepth;
        const s16x8 vv = {vlo[bb][0], vlo[bb][1], vlo[bb][2], vlo[bb][3],
                          vhi[bb][0], vhi[bb][1], vhi[bb][2], vhi[bb][3]};
        __builtin_amdgcn_sched_barrier(0);
        oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pa,
                                                           oacc[nb], 0, 0, 0);
        asm volatile("" : "+a"(oacc[nb]));
        if (nb + kVDepth < kNB) load_v(nb + kVDepth, bb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // The inner loop touches O only through MFMA.  The first block sets the reference (O is
  // still zero); a later block that needs a new one jumps out of the loop, O is rescaled
  // outside, and the loop resumes.  That rare path re-reads Q afterwards, so Q's registers
  // are free while it runs.  No load may still be in flight where control enters the loop
  // head (prologue, rare path): the compiler would then wait for it inside the loop, and
  // that wait also counts the tile DMAs it cannot see, stalling each block on the gather
  // it has just issued.  Hence the explicit waits before the loop and at the rare path's
  // end, and the rescale one block of 16 at a time (all 256 at once spills, and the reloads
  // would be such loads).
  const int nblocks = 2 * ntiles;
  // Q and tile 0 have landed before the loop (its first block would wait here anyway), so
  // no load of the prologue is still counted at the loop head.
  wait_vmem();
  int b = 0;
  float s[16];
  float alpha = 1.f;
  for (;;) {
    for (; b < nblocks; ++b) {
      const int t = b >> 1, kb = b & 1;
      const uint8_t *cur = s_kv + (t & 1) * kTileBytes;
      uint8_t *nxt = s_kv + ((t + 1) & 1) * kTileBytes;
      const bool more = t + 1 < ntiles;
      if (kb == 0) {
        wait_vmem();
        lds_barrier();
      }
      // this wave's 9 gather slots of the next tile for half h = kb (issued with the S MFMAs)
      const uint8_t *gsrc = nullptr;
      if (more) gather128_half(kv, s_sidx, n_valid, t + 1, nxt, w, l, kb, gsrc);
      uint8_t *gdst = nxt + w * kRegionBytes + kb * kHalfBytes;

      // ---- S^T: 32 keys x 32 heads, two chains over the 36 k-steps ----
      f32x16 sa, sb;
      {
        const uint8_t *kbe = cur + (2 * kb) * kRegionBytes + k_off + 16 * ((l & 7) ^ 0);
        const uint8_t *kbo = cur + (2 * kb) * kRegionBytes + k_off + 16 * ((l & 7) ^ 4);
        // Ring of kKDepth k-step pairs: pair kp + kKDepth - 1 is read into the slot that pair
        // kp - 1 used (its MFMAs have issued), before pair kp's MFMAs.
        bf16x8 kf[kKDepth][2];
        auto load_k = [&](int ks, int buf) {
          kf[buf][ks & 1] = *reinterpret_cast<const bf16x8 *>(((ks & 1) ? kbo : kbe) + 256 * ks);
        };
#pragma unroll
        for (int i = 0; i + 1 < kKDepth; ++i) {
          load_k(2 * i, i);
          load_k(2 * i + 1, i);
        }
#pragma unroll
        for (int kp = 0; kp < kKS / 2; ++kp) {  // pairs of k-steps
          const int bb = kp % kKDepth;
          __builtin_amdgcn_sched_barrier(0);
          if (kp + kKDepth - 1 < kKS / 2) {
            load_k(2 * (kp + kKDepth - 1), (kp + kKDepth - 1) % kKDepth);
            load_k(2 * (kp + kKDepth - 1) + 1, (kp + kKDepth - 1) % kKDepth);
          }
          if (kp == 0) {
            mfma_s0(sa, kf[bb][0], qreg[0]);
            mfma_s0(sb, kf[bb][1], qreg[1]);
          } else {
            mfma_s(sa, kf[bb][0], qreg[2 * kp]);
            mfma_s(sb, kf[bb][1], qreg[2 * kp + 1]);
          }
          // one slot every other k-step pair: a wave that waits to issue a DMA stalls its
          // MFMAs too, so the issues are spread over the whole S^T phase
          if (more && (kp & 1) == 0) dma16(gsrc + 128 * (kp >> 1), gdst + 1024 * (kp >> 1));
          __builtin_amdgcn_sched_barrier(0);
        }
        mfma_s_drain(sa, sb);
      }

      // ---- scores of head (l & 31): keys 32kb + 8(i>>2) + 4g + (i&3) of the tile ----
      const int kq = t * kTK + 32 * kb + 4 * g;
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float v = (kq + 8 * (i >> 2) + (i & 3) < n_valid) ? (sa[i] + sb[i]) * scale_log2 : -INFINITY;
        s[i] = v;
        mx = vmax(mx, v);
      }
      mx = xor32_max(mx);
      const bool over = mx > m_ref + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(over) != 0) {
        alpha = over ? __builtin_amdgcn_exp2f(m_ref - mx) : 1.f;
        m_ref = over ? mx : m_ref;
        l_run *= alpha;
        if (b > 0) goto rare;
      }
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s[i] - m_ref);
        l_run += p[i];
      }
      pv_block(cur, kb, p);
    }
    break;  // every block done
  rare:
    // ---- rare path: rescale O by this lane's head factor, then this block's P V ----
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      f32x16 tmp = oacc[nb];
      asm volatile("" : "+v"(tmp));
#pragma unroll
      for (int i = 0; i < 16; ++i) tmp[i] *= alpha;
      asm volatile("" : "+v"(tmp));
      oacc[nb] = tmp;
      asm volatile("" : "+a"(oacc[nb]));
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s[i] - m_ref);
        l_run += p[i];
      }
      pv_block(s_kv + ((b >> 1) & 1) * kTileBytes, b & 1, p);
    }
    load_q();
    wait_vmem();
    ++b;
  }

  // ---- epilogue: head sums, normalise, stage O^T -> LDS rows, whole-row stores ----
  const float lt = xor32_sum(l_run);
  const float inv = lt > 0.f ? __builtin_amdgcn_rcpf(lt) : 0.f;
  lds_barrier();  // every wave is done with the tile buffers
  uint8_t *stg = s_kv + w * kHW * kOStride;
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    asm volatile("" : "+a"(oacc[nb]));
    const f32x16 ob = oacc[nb];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(ob[4 * qd + e] * inv);
      *reinterpret_cast<bf16x4 *>(stg + (l & 31) * kOStride + 2 * (32 * nb + 8 * qd + 4 * g)) = v;
    }
  }
  __bf16 *dst = kSplit ? ws_o + (int64_t)split * num_rows * num_heads * kDV : out;
  dst += ((int64_t)row * num_heads + hw) * kDV + 8 * l;
#pragma unroll 4
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
static hipError_t launch128(const __bf16 *qb, const uint8_t *kvb, int64_t kv_rows,
                            const int32_t *indices, int32_t num_rows, int32_t num_heads,
                            int32_t topk, float scale_log2, __bf16 *ob, float *lse, void *workspace,
                            const AttnPlan &plan, const PagedMap &pg,
                            const AltSource &alt, hipStream_t stream) {
  const int units = num_rows * (num_heads / kH128) * plan.splits;
  const int grid = (units + 7) / 8 * 8;
  if (plan.splits == 1) {
    hipLaunchKernelGGL((attn128_kernel<false, kPaged>), dim3(grid), dim3(kThreads), 0, stream, qb,
                       kvb, kv_rows, indices, num_rows, num_heads, topk, plan.keys_per_split, 1,
                       units, scale_log2, ob, lse, nullptr, nullptr, pg, alt);
    return hipGetLastError();
  }
  __bf16 *ws_o = static_cast<__bf16 *>(workspace);
  float *ws_ml = reinterpret_cast<float *>(ws_o + (size_t)plan.splits * num_rows * num_heads * kDV);
  hipLaunchKernelGGL((attn128_kernel<true, kPaged>), dim3(grid), dim3(kThreads), 0, stream, qb,
                     kvb, kv_rows, indices, num_rows, num_heads, topk, plan.keys_per_split,
                     plan.splits, units, scale_log2, ob, lse, ws_o, ws_ml, pg, alt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_attn_combine(ws_o, ws_ml, plan.splits, num_rows, num_heads, ob, lse, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn128(const void *q, const void *kv, int64_t kv_rows, const int32_t *indices,
                          int32_t num_rows, int32_t num_heads, int32_t topk, float scale, void *out,
                          float *lse, void *workspace, const AttnPlan &plan, const PagedMap *paged,
                          const AltSource *alt, hipStream_t stream) {
  const float scale_log2 = scale * 1.44269504088896340736f;
  const __bf16 *qb = static_cast<const __bf16 *>(q);
  const uint8_t *kvb = static_cast<const uint8_t *>(kv);
  __bf16 *ob = static_cast<__bf16 *>(out);
  if (paged != nullptr)
    return launch128<true>(qb, kvb, kv_rows, indices, num_rows, num_heads, topk, scale_log2, ob,
                           lse, workspace, plan, *paged, AltSource{}, stream);
  return launch128<false>(qb, kvb, kv_rows, indices, num_rows, num_heads, topk, scale_log2, ob,
                          lse, workspace, plan, PagedMap{},
                          alt ? *alt : AltSource{}, stream);
}

}  // namespace hs
