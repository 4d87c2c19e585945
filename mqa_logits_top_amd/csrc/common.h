// Small device helpers shared by the selection kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace idx {

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1, so that
// register arrays are only ever indexed by constants (no scratch spills).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Order-preserving map fp32 -> uint32 (larger key <=> larger value; -0 ranks as +0).
// Key 0 is never produced by a real number below NaN patterns and serves as "empty".
__device__ __forceinline__ uint32_t fkey(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float kval(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return lane ? (~0ull >> (64 - lane)) : 0ull; }

}  // namespace idx
