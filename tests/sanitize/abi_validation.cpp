// Host-side exercise of the C ABI's argument validation, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (device code is built as usual) and run on a
// machine without a GPU: every call below must return its status before any kernel launch.
// Also sweeps the attention planner (hs_attn_workspace_bytes, hs_attn_plan_info) over
// extreme but type-valid sizes, where size arithmetic could overflow.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "hisparse.h"

static int failures = 0;

static void expect(const char *what, int got, int want) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  // fake device addresses: validation never dereferences them
  int32_t *p = reinterpret_cast<int32_t *>(uintptr_t(4096));
  void *v = reinterpret_cast<void *>(uintptr_t(8192));
  void *mis = reinterpret_cast<void *>(uintptr_t(8200));  // not 16-byte aligned
  const int E = HS_ERR_INVALID_ARG, U = HS_ERR_UNSUPPORTED;

  // resolve
  expect("resolve zero rows", hs_resolve_topk(nullptr, 0, 16, nullptr, nullptr, 1, nullptr, 4, 16, 16, nullptr, nullptr, nullptr), HS_OK);
  expect("resolve negative rows", hs_resolve_topk(p, -1, 16, p, p, 1, p, 4, 16, 16, p, nullptr, nullptr), E);
  expect("resolve zero topk", hs_resolve_topk(p, 2, 0, p, p, 1, p, 4, 16, 16, p, nullptr, nullptr), E);
  expect("resolve zero block", hs_resolve_topk(p, 2, 16, p, p, 1, p, 4, 0, 16, p, nullptr, nullptr), E);
  expect("resolve null out", hs_resolve_topk(p, 2, 16, p, p, 1, p, 4, 16, 16, nullptr, nullptr, nullptr), E);
  expect("resolve null table", hs_resolve_topk(p, 2, 16, p, p, 1, nullptr, 4, 16, 16, p, nullptr, nullptr), E);

  // hot state
  hs_hot_state st{2, 24, p, p, p, 256, 64, HS_F32, v, v};
  expect("swap capacity", hs_swap_in(&st, p, 25, 1, p, p, nullptr, nullptr), HS_ERR_CAPACITY);
  expect("swap null state", hs_swap_in(nullptr, p, 16, 1, p, p, nullptr, nullptr), E);
  expect("swap null rows", hs_swap_in(&st, nullptr, 16, 1, p, p, nullptr, nullptr), E);
  expect("swap zero topk", hs_swap_in(&st, p, 0, 1, p, p, nullptr, nullptr), E);
  hs_hot_state bad = st; bad.row_elems = 6;
  expect("swap row bytes", hs_swap_in(&bad, p, 16, 1, p, p, nullptr, nullptr), E);
  bad = st; bad.hot_kv = mis;
  expect("swap misaligned", hs_swap_in(&bad, p, 16, 1, p, p, nullptr, nullptr), E);
  bad = st; bad.dtype = 7;
  expect("swap dtype", hs_swap_in(&bad, p, 16, 1, p, p, nullptr, nullptr), E);
  bad = st; bad.host_rows = (int64_t(1) << 31);
  expect("swap host rows", hs_swap_in(&bad, p, 16, 1, p, p, nullptr, nullptr), E);
  bad = st; bad.num_reqs = 1 << 20; bad.capacity = 1 << 14;
  expect("swap slot count", hs_swap_in(&bad, p, 16, 1, p, p, nullptr, nullptr), E);
  bad = st; bad.num_reqs = 0x7fffffff; bad.capacity = 0x7fffffff;
  expect("swap huge sizes", hs_swap_in(&bad, p, 16, 1, p, p, nullptr, nullptr), E);
  bad = st; bad.row_elems = 0x7fffffff;
  expect("swap huge row", hs_swap_in(&bad, p, 16, 1, p, p, nullptr, nullptr), E);
  bad = st; bad.capacity = 20000;
  expect("swap capacity limit", hs_swap_in(&bad, p, 16, 1, p, p, nullptr, nullptr), U);

  // finalize
  expect("finalize vocab", hs_finalize_accepted(&st, v, 0, p, v, 3, p, p, 8, 16, 1, p, p, p, nullptr), E);
  expect("finalize rows", hs_finalize_accepted(&st, v, 100, p, v, 0, p, p, 8, 16, 1, p, p, p, nullptr), E);
  expect("finalize rows > cap", hs_finalize_accepted(&st, v, 100, p, v, 25, p, p, 8, 16, 1, p, p, p, nullptr), E);
  expect("finalize null", hs_finalize_accepted(&st, nullptr, 100, p, v, 3, p, p, 8, 16, 1, p, p, p, nullptr), E);
  expect("finalize misaligned", hs_finalize_accepted(&st, v, 100, p, mis, 3, p, p, 8, 16, 1, p, p, p, nullptr), E);

  expect("argmax zero rows", hs_greedy_argmax(nullptr, 0, 10, nullptr, nullptr), HS_OK);
  expect("argmax vocab", hs_greedy_argmax(v, 4, 0, p, nullptr), E);
  expect("argmax misaligned", hs_greedy_argmax(mis, 4, 10, p, nullptr), E);
  expect("argmax null out", hs_greedy_argmax(v, 4, 10, nullptr, nullptr), E);
  expect("finalize from argmax, misaligned rows", hs_finalize_accepted(&st, nullptr, 0, p, mis, 3, p, p, 8, 16, 1, p, p, p, nullptr), E);

  // attention
  expect("attn zero rows", hs_sparse_decode_attn(v, v, 10, p, 0, 128, 576, 512, 2048, 0.1f, HS_BF16, v, nullptr, nullptr, 0, nullptr), HS_OK);
  expect("attn dtype", hs_sparse_decode_attn(v, v, 10, p, 2, 128, 576, 512, 2048, 0.1f, 9, v, nullptr, nullptr, 0, nullptr), E);
  expect("attn shape", hs_sparse_decode_attn(v, v, 10, p, 2, 128, 512, 512, 2048, 0.1f, HS_BF16, v, nullptr, nullptr, 0, nullptr), U);
  expect("attn heads", hs_sparse_decode_attn(v, v, 10, p, 2, 100, 576, 512, 2048, 0.1f, HS_BF16, v, nullptr, nullptr, 0, nullptr), U);
  expect("attn no workspace", hs_sparse_decode_attn(v, v, 10, p, 2, 128, 576, 512, 2048, 0.1f, HS_BF16, v, nullptr, nullptr, 0, nullptr), E);
  expect("attn misaligned", hs_sparse_decode_attn(mis, v, 10, p, 2, 128, 576, 512, 2048, 0.1f, HS_BF16, v, nullptr, v, 1 << 30, nullptr), E);
  expect("attn kv rows", hs_sparse_decode_attn(v, v, int64_t(1) << 31, p, 2, 128, 576, 512, 2048, 0.1f, HS_BF16, v, nullptr, v, 1 << 30, nullptr), E);
  expect("attn huge batch", hs_sparse_decode_attn(v, v, 10, p, 0x7fffffff, 0x7fffffe0, 576, 512, 2048, 0.1f, HS_BF16, v, nullptr, v, 1 << 30, nullptr), U);
  expect("attn huge topk", hs_sparse_decode_attn(v, v, 10, p, 4, 128, 576, 512, 0x7fffffff, 0.1f, HS_BF16, v, nullptr, v, 1 << 30, nullptr), U);
  expect("attn f32 d", hs_sparse_decode_attn(v, v, 10, p, 2, 4, 2048, 48, 16, 0.1f, HS_F32, v, nullptr, nullptr, 0, nullptr), U);
  expect("cus zero", hs_sparse_decode_attn_cus(v, v, 10, p, 2, 128, 576, 512, 2048, 0.1f, HS_BF16, v, nullptr, v, 1 << 30, 0, nullptr), E);
  expect("cus no workspace", hs_sparse_decode_attn_cus(v, v, 10, p, 2, 128, 576, 512, 2048, 0.1f, HS_BF16, v, nullptr, nullptr, 0, 128, nullptr), E);
  expect("noalloc scratch", hs_sparse_decode_attn_noalloc(v, v, 10, p, 256, 256, 576, 512, 4096, 0.1f, HS_BF16, v, nullptr, nullptr), HS_ERR_SCRATCH);
  expect("paged null table", hs_sparse_decode_attn_paged(v, v, 10, p, p, p, 1, nullptr, 4, 16, 16, 2, 128, 576, 512, 2048, 0.1f, HS_BF16, v, nullptr, v, 1 << 30, nullptr), E);
  expect("mixed cus zero", hs_sparse_decode_attn_mixed_cus(v, v, 10, p, v, 10, p, p, 2, 128, 576, 512, 2048, 0.1f, HS_BF16, v, nullptr, v, 1 << 30, 0, nullptr), E);
  expect("mixed f32", hs_sparse_decode_attn_mixed(v, v, 10, p, v, 10, p, p, 2, 128, 576, 512, 2048, 0.1f, HS_F32, v, nullptr, v, 1 << 30, nullptr), U);

  // plan arithmetic over extreme sizes (no launch): workspace and plan must stay defined
  const int32_t rows[] = {1, 2, 7, 8, 31, 32, 255, 256, 4096, 1 << 20, 0x7fffffff};
  const int32_t heads[] = {32, 64, 96, 128, 256, 4096, 1 << 20, 0x7fffffe0};
  const int32_t topks[] = {1, 63, 64, 2047, 2048, 2049, 4096, 1 << 20, 0x7fffffff};
  for (int32_t r : rows)
    for (int32_t h : heads)
      for (int32_t k : topks) {
        int32_t hpw = -1, spl = -1;
        const int st_ = hs_attn_plan_info(r, h, 576, 512, k, HS_BF16, &hpw, &spl);
        const size_t ws = hs_attn_workspace_bytes(r, h, 576, 512, k, HS_BF16);
        if (st_ == HS_OK) {
          if (!(hpw == 32 || hpw == 64 || hpw == 128) || spl < 1) {
            std::printf("FAIL plan %d %d %d: heads/wg %d splits %d\n", r, h, k, hpw, spl);
            ++failures;
          }
          if ((spl > 1) != (ws > 0)) {
            std::printf("FAIL plan %d %d %d: splits %d workspace %zu\n", r, h, k, spl, ws);
            ++failures;
          }
        } else if (ws != 0) {
          std::printf("FAIL plan %d %d %d: rejected (%d) but workspace %zu\n", r, h, k, st_, ws);
          ++failures;
        }
        // the plan for part of the GPU: accepted exactly when the whole-GPU one is, never
        // more key splits (so the same workspace serves)
        for (int32_t c : {1, 64, 128, 255, 256, 0x7fffffff}) {
          int32_t hc = -1, sc = -1;
          const int stc = hs_attn_plan_info_cus(r, h, 576, 512, k, HS_BF16, c, &hc, &sc);
          if (stc != st_ || (stc == HS_OK && (!(hc == 32 || hc == 64 || hc == 128) || sc < 1 || sc > spl))) {
            std::printf("FAIL plan cus %d %d %d %d: status %d heads/wg %d splits %d (whole %d)\n",
                        r, h, k, c, stc, hc, sc, spl);
            ++failures;
          }
        }
      }

  // other calls
  expect("backup rows", hs_backup_rows(v, 10, v, 10, 1, 24, p, 0, p, 5, 1, 1, nullptr), E);
  expect("backup zero", hs_backup_rows(nullptr, 10, nullptr, 10, 1, 32, nullptr, 0, nullptr, 0, 1, 1, nullptr), HS_OK);
  expect("plan reuse rows", hs_apply_plan(v, v, int64_t(1) << 31, 1, 2, 24, 1152, p, 16, p, p, p, nullptr), E);
  expect("append row bytes", hs_append_accepted(v, 10, 24, p, 4, 16, 16, p, v, p, 2, 3, nullptr), E);
  expect("host read size", hs_host_read(v, v, 24, nullptr), E);
  expect("host read zero", hs_host_read(nullptr, nullptr, 0, nullptr), HS_OK);
  for (int s = -6; s <= 1; ++s)
    if (hs_status_string(s) == nullptr) { std::printf("FAIL status string %d\n", s); ++failures; }
  if (hs_version() == nullptr) ++failures;

  if (failures) return 1;
  std::printf("abi validation ok\n");
  return 0;
}
