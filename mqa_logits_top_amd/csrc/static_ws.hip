// The fused indexer without a caller workspace, for callers that cannot allocate
// (code under stream capture, tight serving loops, harnesses that forbid
// hipMalloc): its workspace is a file-scope device array of IDX_STATIC_WS_BYTES.
//
// Each GPU the library runs on holds its own copy of the array from the moment the
// library's code is loaded there until the process ends.  The host-side name of the
// array is not a device address; the address is looked up once per device with
// hipGetSymbolAddress (while that device is current) and kept, and only that
// address is handed to kernels.  The fused path needs no zeroed workspace (every
// word it reads it has written earlier in the same call), so nothing is cleared.
// Every call on one GPU shares the array: calls that overlap in time on one GPU (two
// streams, two host threads) race and give undefined results.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/idx.h"
#include "api_internal.h"

static __device__ __align__(256) uint8_t scratch[IDX_STATIC_WS_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::atomic<void *> scratch_on_device[MAX_DEVICES];   // device address of `scratch`, per device

// This device's copy of the array (looked up on the first call on the device).  Host threads
// that race here only repeat the lookup, which returns the same address.
hipError_t scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  void *p = scratch_on_device[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_on_device[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" idx_status idx_logits_topk_fused_static(const idx_problem *p, int32_t K, int32_t block_k,
                                                   int32_t row_chunk, const uint8_t *mask, int64_t ld_mask,
                                                   int32_t *out_idx, float *out_val, void *stream) {
  return idx::fused_impl(p, K, block_k, row_chunk, mask, ld_mask, nullptr, 0, 0, 1, nullptr, out_idx, out_val, nullptr,
                         nullptr, (size_t)IDX_STATIC_WS_BYTES, stream, scratch_address);
}
