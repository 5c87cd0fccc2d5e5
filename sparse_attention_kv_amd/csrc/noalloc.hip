// hs_sparse_decode_attn_noalloc: attention whose key-split workspace is a fixed scratch
// array in device memory, for callers that cannot allocate.
//
// The array below is a file-scope device variable: each GPU the library runs on holds its
// own copy at its own address for the life of the process.  In host code its name only
// stands for the symbol; the device address is looked up once per device with
// hipGetSymbolAddress (that device current) and kept, and only that address is passed to
// kernels.

#include <mutex>

#include "ops.h"

namespace {

constexpr size_t kScratchBytes = HS_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_lock;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the current device, looked up on the first call there.
hs_status scratch_on_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return HS_ERR_HIP;
  }
  std::lock_guard<std::mutex> guard(g_lock);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return HS_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return HS_OK;
}

}  // namespace

extern "C" hs_status hs_sparse_decode_attn_noalloc(const void *q, const void *kv, int64_t kv_rows,
                                                   const int32_t *indices, int32_t num_rows,
                                                   int32_t num_heads, int32_t d_qk, int32_t d_v,
                                                   int32_t topk, float scale, int32_t dtype,
                                                   void *out, float *lse, void *stream) {
  if (dtype == HS_BF16 && num_rows > 0 && num_heads > 0 && topk > 0 &&
      hs_attn_workspace_bytes(num_rows, num_heads, d_qk, d_v, topk, dtype) > kScratchBytes)
    return HS_ERR_SCRATCH;
  void *ws = nullptr;
  const hs_status s = scratch_on_current_device(&ws);
  if (s != HS_OK) return s;
  return hs::sparse_decode_attn_checked(q, kv, kv_rows, indices, num_rows, num_heads, d_qk, d_v,
                                        topk, scale, dtype, out, lse, ws, kScratchBytes, stream, hs::kNumCUs);
}
