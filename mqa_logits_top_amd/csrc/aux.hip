// Memory-bound helper kernels of the indexer path.
//  - fill_tail:   dense logits are [T, W] with W the longest window (P1 section 1:
//                 [T, max_seqlen_k]); columns past a row's own window hold -inf.
//  - pool_dense:  the candidate source's 8-key block pooling over dense logits
//                 (P1 section 1, select_candidate_blocks "pads and pools"): block b
//                 of row t is the max over columns [pool b, pool b + pool) inside
//                 the window, so a partial last block takes its in-window max.
//  - expand_mask: the published candidate mask, one byte per (row, column),
//                 written in place into the caller's [rows, lc] buffer (P2
//                 Modifications), from the kept block ids.
//  - ragged:      per-row windows of a varlen batch, built once per batch on the
//                 device (P3: one ragged plan per batch, no per-request syncs), over
//                 plain or compressed keys (P1 section 1: the ratio-1/2 source layers).
//  - tail rows:   the last n rows of every request, for outputs restricted to each
//                 request's tail rows (P2 Modifications: tail-only candidate masks).
//  - gather rows: a row subset of a problem (q, q_scale, w, ks, ke) copied into a
//                 compact problem, so that any entry point serves just those rows.
#include "kernels.h"

namespace idx {
namespace {

__global__ __launch_bounds__(256) void fill_tail_kernel(float *logits, int64_t ld, int32_t W, const int32_t *ks,
                                                        const int32_t *ke, int32_t row0) {
  const int r = blockIdx.y;
  const int t = row0 + r;
  const int win = min(max(ke[t] - max(ks[t], 0), 0), W);
  float *row = logits + (int64_t)r * ld;
  for (int j = win + blockIdx.x * 256 + threadIdx.x; j < W; j += gridDim.x * 256) row[j] = -__builtin_inff();
}

__global__ __launch_bounds__(256) void pool_dense_kernel(const float *logits, int64_t ld, int32_t W,
                                                         const int32_t *ks, const int32_t *ke, int32_t row0,
                                                         int32_t pool, float *out, int64_t ld_out, int32_t ncols_out) {
  const int r = blockIdx.y;
  const int t = row0 + r;
  const int win = min(max(ke[t] - max(ks[t], 0), 0), W);
  const int nb = min((win + pool - 1) / pool, ncols_out);
  const float *row = logits + (int64_t)r * ld;
  for (int b = blockIdx.x * 256 + threadIdx.x; b < nb; b += gridDim.x * 256) {
    const int j0 = b * pool, j1 = min(j0 + pool, win);
    float m = row[j0];
    for (int j = j0 + 1; j < j1; ++j) m = __builtin_fmaxf(m, row[j]);
    out[(int64_t)r * ld_out + b] = m;
  }
}

// One workgroup per row: kept blocks -> LDS bitmap -> bytes over [0, W).
__global__ __launch_bounds__(256) void expand_mask_kernel(const int32_t *blocks, int32_t n_blocks, const int32_t *ks,
                                                          const int32_t *ke, int32_t row0, int32_t pool, int32_t W,
                                                          uint8_t *mask, int64_t ld_mask) {
  extern __shared__ uint32_t bits[];
  const int r = blockIdx.x;
  const int t = row0 + r;
  const int win = min(max(ke[t] - max(ks[t], 0), 0), W);
  const int nbk = (W + pool - 1) / pool;
  const int nwords = (nbk + 31) / 32;
  for (int i = threadIdx.x; i < nwords; i += 256) bits[i] = 0;
  __syncthreads();
  const int32_t *brow = blocks + (int64_t)r * n_blocks;
  for (int i = threadIdx.x; i < n_blocks; i += 256) {
    const int b = brow[i];
    if (b >= 0 && b < nbk) atomicOr(&bits[b >> 5], 1u << (b & 31));
  }
  __syncthreads();
  uint8_t *mrow = mask + (int64_t)t * ld_mask;
  const bool vec = ((uintptr_t)mrow & 15) == 0;
  if (pool == 8 && vec) {
    // 16 aligned bytes are blocks 2c and 2c + 1 of 8 keys: two bits of one bitmap word
    for (int j0 = threadIdx.x * 16; j0 < W; j0 += 256 * 16) {
      const uint32_t wd = bits[j0 >> 8] >> ((j0 >> 3) & 31);
      const uint32_t lo = (wd & 1u) ? 0x01010101u : 0u, hi = (wd & 2u) ? 0x01010101u : 0u;
      uint4 v = make_uint4(lo, lo, hi, hi);
      if (j0 + 16 > win) {   // the window ends inside these bytes (or before them)
        uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (j0 + e >= win) w4[e >> 2] &= ~(0xFFu << (8 * (e & 3)));
        v = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
      if (j0 + 16 <= W) {
        *(uint4 *)(mrow + j0) = v;
      } else {
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        for (int e = 0; e < 16 && j0 + e < W; ++e) mrow[j0 + e] = (uint8_t)(w4[e >> 2] >> (8 * (e & 3)));
      }
    }
    return;
  }
  for (int j0 = threadIdx.x * 16; j0 < W; j0 += 256 * 16) {
    uint32_t w4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t v = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 4 * q + e;
        const int b = j / pool;
        const bool on = j < win && ((bits[b >> 5] >> (b & 31)) & 1u);
        v |= (on ? 1u : 0u) << (8 * e);
      }
      w4[q] = v;
    }
    if (vec && j0 + 16 <= W) {
      *(uint4 *)(mrow + j0) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    } else {
      for (int e = 0; e < 16 && j0 + e < W; ++e) mrow[j0 + e] = (uint8_t)(w4[e >> 2] >> (8 * (e & 3)));
    }
  }
}

__global__ __launch_bounds__(256) void ragged_kernel(const int32_t *cu_q, const int32_t *cu_k, const int32_t *cu_c,
                                                     int32_t ratio, int32_t B, int32_t T, int32_t *ks, int32_t *ke) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  if (B <= 0 || t >= cu_q[B] || t < cu_q[0]) {
    ks[t] = 0;
    ke[t] = 0;
    return;
  }
  int lo = 0, hi = B - 1;  // largest i with cu_q[i] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int lq = cu_q[lo + 1] - cu_q[lo];
  const int lk = cu_k[lo + 1] - cu_k[lo];
  const int lc = cu_c[lo + 1] - cu_c[lo];
  const int j = t - cu_q[lo];
  // new row j is token (lk - lq) + j of its request and sees the keys of the complete
  // groups of `ratio` tokens up to and including it (floor division)
  const int seen = (lk - lq) + j + 1;
  const int groups = seen >= 0 ? seen / ratio : -((-seen + ratio - 1) / ratio);
  ks[t] = cu_c[lo];
  ke[t] = cu_c[lo] + min(groups, lc);
}

// rows[i * n + m] = row cu_q[i+1] - n + m of request i, or -1 where the request is
// shorter than n.
__global__ __launch_bounds__(256) void tail_rows_kernel(const int32_t *cu_q, int32_t B, int32_t n, int32_t *rows) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= (int64_t)B * n) return;
  const int i = (int)(x / n), m = (int)(x % n);
  const int t = cu_q[i + 1] - n + m;
  rows[x] = t >= cu_q[i] ? t : -1;
}

// One workgroup per output row: its q bytes (H * D), q_scale and w (H floats each),
// and its window.  Row -1 gets zeros and the empty window [0, 0).
__global__ __launch_bounds__(256) void gather_rows_kernel(const int32_t *rows, int32_t T, const uint8_t *q,
                                                          const float *q_scale, const float *w, const int32_t *ks,
                                                          const int32_t *ke, int32_t H, int32_t D, uint8_t *oq,
                                                          float *oqs, float *ow, int32_t *oks, int32_t *oke) {
  const int r = blockIdx.x;
  const int t = rows[r];
  const bool ok = t >= 0 && t < T;
  const int64_t nq = (int64_t)H * D / 16;   // 16-byte words of one q row
  const uint4 *src = (const uint4 *)(q + (ok ? (int64_t)t * H * D : 0));
  uint4 *dst = (uint4 *)(oq + (int64_t)r * H * D);
  for (int64_t i = threadIdx.x; i < nq; i += 256) dst[i] = ok ? src[i] : make_uint4(0u, 0u, 0u, 0u);
  for (int h = threadIdx.x; h < H; h += 256) {
    oqs[(int64_t)r * H + h] = ok ? q_scale[(int64_t)t * H + h] : 0.f;
    ow[(int64_t)r * H + h] = ok ? w[(int64_t)t * H + h] : 0.f;
  }
  if (threadIdx.x == 0) {
    oks[r] = ok ? ks[t] : 0;
    oke[r] = ok ? ke[t] : 0;
  }
}

}  // namespace

hipError_t launch_tail_rows(const int32_t *cu_q, int32_t B, int32_t n, int32_t *rows, hipStream_t s) {
  const int64_t total = (int64_t)B * n;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(tail_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, cu_q, B, n, rows);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const int32_t *rows, int32_t R, int32_t T, const uint8_t *q, const float *q_scale,
                              const float *w, const int32_t *ks, const int32_t *ke, int32_t H, int32_t D, uint8_t *oq,
                              float *oqs, float *ow, int32_t *oks, int32_t *oke, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)R), dim3(256), 0, s, rows, T, q, q_scale, w, ks, ke, H, D, oq,
                     oqs, ow, oks, oke);
  return hipGetLastError();
}

hipError_t launch_fill_tail(float *logits, int64_t ld, int32_t W, const int32_t *ks, const int32_t *ke, int32_t row0,
                            int32_t nrows, hipStream_t s) {
  if (nrows <= 0 || W <= 0) return hipSuccess;
  const int gx = min((W + 255) / 256, 64);
  hipLaunchKernelGGL(fill_tail_kernel, dim3(gx, nrows), dim3(256), 0, s, logits, ld, W, ks, ke, row0);
  return hipGetLastError();
}

hipError_t launch_pool_dense(const float *logits, int64_t ld, int32_t W, const int32_t *ks, const int32_t *ke,
                             int32_t row0, int32_t nrows, int32_t pool, float *out, int64_t ld_out, int32_t ncols_out,
                             hipStream_t s) {
  if (nrows <= 0 || ncols_out <= 0) return hipSuccess;
  const int gx = min((ncols_out + 255) / 256, 64);
  hipLaunchKernelGGL(pool_dense_kernel, dim3(gx, nrows), dim3(256), 0, s, logits, ld, W, ks, ke, row0, pool, out,
                     ld_out, ncols_out);
  return hipGetLastError();
}

hipError_t launch_expand_mask(const int32_t *blocks, int32_t n_blocks, const int32_t *ks, const int32_t *ke,
                              int32_t row0, int32_t nrows, int32_t pool, int32_t W, uint8_t *mask, int64_t ld_mask,
                              hipStream_t s) {
  if (nrows <= 0 || W <= 0) return hipSuccess;
  const int nbk = (W + pool - 1) / pool;
  const size_t lds = (size_t)((nbk + 31) / 32) * 4;
  hipLaunchKernelGGL(expand_mask_kernel, dim3(nrows), dim3(256), lds, s, blocks, n_blocks, ks, ke, row0, pool, W,
                     mask, ld_mask);
  return hipGetLastError();
}

hipError_t launch_ragged(const int32_t *cu_q, const int32_t *cu_k, const int32_t *cu_c, int32_t ratio, int32_t B,
                         int32_t T, int32_t *ks, int32_t *ke, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(ragged_kernel, dim3((T + 255) / 256), dim3(256), 0, s, cu_q, cu_k, cu_c, ratio, B, T, ks, ke);
  return hipGetLastError();
}

}  // namespace idx
