// Device-side precondition check, run before an entry point's kernels when the
// environment variable IDX_DEBUG is set to a value other than "0".
//
// The host cannot see preconditions that live in device memory (window bounds,
// scale signs, finite inputs) without a synchronisation.  In debug mode every entry
// point first launches these checks on its stream, waits for them, and returns
// IDX_E_DEVICE_CHECK without enqueueing any other kernel when one fails.  The
// result word is a file-scope device array (one per GPU, its address looked up once
// per device); calls that overlap on one GPU in debug mode share it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "../../include/idx.h"
#include "api_internal.h"

static __device__ uint32_t debug_word[1];

namespace {

constexpr int MAX_DEVICES = 64;
std::atomic<uint32_t *> word_on_device[MAX_DEVICES];

hipError_t word_address(uint32_t **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  uint32_t *p = word_on_device[dev].load(std::memory_order_acquire);
  if (!p) {
    void *v = nullptr;
    e = hipGetSymbolAddress(&v, HIP_SYMBOL(debug_word));
    if (e != hipSuccess) return e;
    if (!v) return hipErrorInvalidSymbol;
    p = (uint32_t *)v;
    word_on_device[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

__global__ void clear_kernel(uint32_t *word) { *word = 0u; }

__device__ bool finite_f32(float x) { return (__float_as_uint(x) & 0x7F800000u) != 0x7F800000u; }

// Rows: 0 <= ks <= ke <= L, ke - ks <= W (W >= 0), and, with scores, q_scale >= 0 and
// finite, w finite.  H = 0 skips the per-head checks.
__global__ void check_rows_kernel(const int32_t *ks, const int32_t *ke, int32_t T, int32_t L, int64_t W,
                                  const float *q_scale, const float *w, int32_t H, uint32_t *word) {
  uint32_t bad = 0;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < (int64_t)T * (H > 0 ? H : 1);
       i += (int64_t)gridDim.x * blockDim.x) {
    if (H > 0) {
      const float qs = q_scale[i], wv = w[i];
      if (!finite_f32(qs) || !(qs >= 0.f)) bad |= 4u;
      if (!finite_f32(wv)) bad |= 8u;
    }
    if (H <= 0 || i % H == 0) {
      const int64_t t = H > 0 ? i / H : i;
      const int32_t a = ks[t], b = ke[t];
      if (a < 0 || a > b || b > L) bad |= 1u;
      if (W >= 0 && (int64_t)b - a > W) bad |= 2u;
    }
  }
  if (bad) atomicOr(word, bad);
}

// Keys: fp8 scales >= 0 and finite; MXFP4 scale codes other than the E8M0 NaN (0xFF).
__global__ void check_keys_kernel(const uint8_t *k_scale, int32_t k_fmt, int32_t L, uint32_t *word) {
  uint32_t bad = 0;
  const int64_t n = k_fmt == 0 ? (int64_t)L : (int64_t)L * 4;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    if (k_fmt == 0) {
      const float s = ((const float *)k_scale)[i];
      if (!finite_f32(s) || !(s >= 0.f)) bad |= 16u;
    } else if (k_scale[i] == 0xFFu) {
      bad |= 16u;
    }
  }
  if (bad) atomicOr(word, bad);
}

}  // namespace

namespace idx {

bool debug_enabled() {
  const char *v = std::getenv("IDX_DEBUG");
  return v && *v && std::strcmp(v, "0") != 0;
}

bool exact_enabled() {
  const char *v = std::getenv("IDX_EXACT");
  return v && *v && std::strcmp(v, "0") != 0;
}

idx_status debug_check(const int32_t *ks, const int32_t *ke, int32_t T, int32_t L, int64_t W, const idx_problem *p,
                       void *stream) {
  if (!debug_enabled()) return IDX_OK;
  hipStream_t s = (hipStream_t)stream;
  uint32_t *word = nullptr;
  if (word_address(&word) != hipSuccess) return IDX_E_LAUNCH;
  hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(1), 0, s, word);
  if (T > 0) {
    const int32_t H = p ? p->H : 0;
    const int64_t n = (int64_t)T * (H > 0 ? H : 1);
    const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(check_rows_kernel, dim3(blocks), dim3(256), 0, s, ks, ke, T, L, W, p ? p->q_scale : nullptr,
                       p ? p->w : nullptr, H, word);
  }
  if (p && p->L > 0) {
    const int64_t n = p->k_fmt == 0 ? (int64_t)p->L : (int64_t)p->L * 4;
    const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(check_keys_kernel, dim3(blocks), dim3(256), 0, s, (const uint8_t *)p->k_scale, p->k_fmt,
                       p->L, word);
  }
  if (hipGetLastError() != hipSuccess) return IDX_E_LAUNCH;
  uint32_t host = 0;
  if (hipMemcpyAsync(&host, word, sizeof(host), hipMemcpyDeviceToHost, s) != hipSuccess) return IDX_E_LAUNCH;
  if (hipStreamSynchronize(s) != hipSuccess) return IDX_E_LAUNCH;
  return host ? IDX_E_DEVICE_CHECK : IDX_OK;
}

}  // namespace idx
