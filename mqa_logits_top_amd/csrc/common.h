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
  const uint32_t u = __float_as_uint(v + 0.0f);   // -0 + 0 = +0 (round to nearest): one key for both zeros
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float kval(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave-wide reductions and scans on DPP / permlane moves (no LDS traffic, no
// lane-address registers): quad swaps, half-row and row mirrors pair the lanes
// of a 16-lane row, then permlane16/32 swaps pair rows.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x, Op op) {
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false));  // row half mirror
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false));  // row mirror
  const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(r16[0], r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(r32[0], r32[1]);
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  return wave_reduce(x, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  return wave_reduce(x, [](uint32_t a, uint32_t b) { return min(a, b); });
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  return wave_reduce(x, [](uint32_t a, uint32_t b) { return max(a, b); });
}
// Inclusive prefix sum over the wave's lanes: shifts by 1, 2, 4, 8 inside each
// 16-lane row, then the last lane of row 0 / 2 into rows 1 / 3 and of row 1 into
// rows 2 and 3 (lanes without a source add 0).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}
// The same reduction for floats (any associative op; the order of combination is fixed).
template <class Op>
__device__ __forceinline__ float wave_reduce_f32(float x, Op op) {
  return __uint_as_float(wave_reduce(__float_as_uint(x), [&](uint32_t a, uint32_t b) {
    return __float_as_uint(op(__uint_as_float(a), __uint_as_float(b)));
  }));
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return lane ? (~0ull >> (64 - lane)) : 0ull; }

}  // namespace idx
