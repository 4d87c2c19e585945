// Exact per-row top-K with a running merge (P1 section 2.3: topk(union) ==
// topk(union of per-block topk), so a row's candidates can arrive block by
// block; P2 Modifications: the top-k of each chunk goes into one shared
// selected buffer).
//
// One workgroup (512 threads) owns one row.  The running top-K (ids ascending,
// fp32 values) lives in LDS while the row's columns are consumed in passes of
// up to 8192 values held in registers.  Thread `tid` owns the contiguous
// columns P + 16 tid .. P + 16 tid + 15 of a pass starting at column P and the
// contiguous running slots 5 tid .. 5 tid + 4, so id order is thread-major and
// every ordered compaction is one per-thread count plus one block-wide
// exclusive scan (all register indices are compile-time constants).  A pass:
//   1. map fp32 values to order-preserving uint32 keys (0 is reserved for
//      "not a candidate": excluded by window, mask, padding, or -- once the
//      running list is full -- by not beating its smallest entry, which wins
//      every tie because running ids precede the pass's ids);
//   2. find the key of the K-th largest candidate (running + pass), counting
//      multiplicity.  The candidate key interval [lo, hi] is narrowed by
//      histogram levels: bins are (key - lo) >> s with the smallest s that
//      gives < 2048 bins, so each level consumes >= 11 bits of the interval and
//      at most three levels are needed; once <= 512 candidates remain they are
//      ranked directly in LDS;
//   3. keep keys above the threshold and, among keys equal to it, the ones
//      with the lowest ids (total order: value desc, id asc), written in id
//      order.  Running ids precede the pass's ids, so the list stays ascending.
// All steps are integer/comparison work on exact keys, so the result is the
// unique top-K under the total order, independent of how rows or columns are
// split into launches and passes.
#include "common.h"
#include "kernels.h"

namespace idx {
namespace {

constexpr int NTH = 512;
constexpr int NWV = NTH / 64;
constexpr int VPT = 16;           // pass values per thread (contiguous columns); small code, fits the I-cache
constexpr int SPAN = NTH * VPT;   // columns one pass can hold
constexpr int RS = 5;             // running slots per thread (K <= 2560)
constexpr int KMAX = RS * NTH;
constexpr int NB = 2048;          // histogram bins
constexpr int CAP = 512;          // direct ranking threshold

struct Smem {
  int run_id[2][KMAX];
  float run_val[2][KMAX];
  uint32_t hist[NB];
  uint32_t cand[CAP];
  uint32_t red[3][NWV];
  uint32_t wsum[2][NWV];
  uint32_t bcast[4];
};

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  for (int o = 32; o > 0; o >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, o));
  return x;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  for (int o = 32; o > 0; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o));
  return x;
}

// Block-wide sum / min / max of one value per thread (all threads must call).
__device__ __forceinline__ uint32_t block_sum(Smem &sm, uint32_t x, int lane, int wave) {
  x = wave_sum(x);
  __syncthreads();
  if (lane == 0) sm.red[0][wave] = x;
  __syncthreads();
  uint32_t s = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) s += sm.red[0][w];
  return s;
}
__device__ __forceinline__ void block_minmax(Smem &sm, uint32_t &lo, uint32_t &hi, int lane, int wave) {
  lo = wave_min(lo);
  hi = wave_max(hi);
  __syncthreads();
  if (lane == 0) { sm.red[1][wave] = lo; sm.red[2][wave] = hi; }
  __syncthreads();
  lo = 0xFFFFFFFFu;
  hi = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) { lo = min(lo, sm.red[1][w]); hi = max(hi, sm.red[2][w]); }
}

// Two simultaneous block-wide exclusive scans in thread order, with their totals.
__device__ __forceinline__ void block_scan2(Smem &sm, uint32_t a, uint32_t b, uint32_t &ea, uint32_t &eb,
                                            uint32_t &ta, uint32_t &tb, int lane, int wave) {
  uint32_t ia = a, ib = b;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t ya = __shfl_up(ia, o), yb = __shfl_up(ib, o);
    if (lane >= o) { ia += ya; ib += yb; }
  }
  __syncthreads();
  if (lane == 63) { sm.wsum[0][wave] = ia; sm.wsum[1][wave] = ib; }
  __syncthreads();
  uint32_t pa = 0, pb = 0;
  ta = 0;
  tb = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    const uint32_t sa = sm.wsum[0][w], sb = sm.wsum[1][w];
    if (w < wave) { pa += sa; pb += sb; }
    ta += sa;
    tb += sb;
  }
  ea = pa + ia - a;
  eb = pb + ib - b;
}

__global__ __launch_bounds__(NTH) void topk_kernel(TopkArgs a) {
  __shared__ Smem sm;
  const int r = blockIdx.x;
  const int t = a.row0 + r;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.K;

  const int ks = max(a.ks[t], 0);
  const int ke = max(a.ke[t], ks);
  int off, id_lo, id_hi;
  switch (a.mode) {
    case TOPK_DENSE: off = ks; id_lo = ks; id_hi = ke; break;
    case TOPK_BLOCK: off = a.key0; id_lo = ks; id_hi = ke; break;
    case TOPK_POOL_DENSE: off = 0; id_lo = 0; id_hi = (ke - ks + a.pool - 1) / a.pool; break;
    default: off = (a.key0 - ks) / a.pool; id_lo = 0; id_hi = (ke - ks + a.pool - 1) / a.pool; break;
  }
  const int c_lo = max(id_lo - off, 0);
  const int c_hi = min(id_hi - off, a.ncols);
  int32_t *oidx = a.out_idx + (int64_t)r * K;
  float *oval = a.out_val ? a.out_val + (int64_t)r * K : nullptr;
  if (!a.first && c_lo >= c_hi) return;  // nothing new for this row: running state stays as is

  // ---- running state
  int cur = 0;
  int run_n = 0;
  if (!a.first) {
    uint32_t cnt = 0;
    for (int p = tid; p < K; p += NTH) {
      const int id = oidx[p];
      sm.run_id[0][p] = id;
      sm.run_val[0][p] = oval[p];
      cnt += id >= 0;
    }
    run_n = (int)block_sum(sm, cnt, lane, wave);
  }

  const float *vrow = a.vals + (int64_t)r * a.ld;
  const uint8_t *mrow = a.mask ? a.mask + (int64_t)t * a.ld_mask : nullptr;
  const int mshift = (a.mode == TOPK_DENSE || a.mode == TOPK_BLOCK) ? off - ks : 0;  // mask byte = c + mshift
  // 16-byte loads when every row and every thread's first column are 16-byte aligned
  const bool vec = ((a.ld & 3) == 0) && (((uintptr_t)a.vals & 15) == 0);
  const int span = min(a.block, SPAN) & ~3;   // a.block is a multiple of 4 or >= SPAN
  const int pbase = vec ? (c_lo & ~3) : c_lo;

  for (int P = pbase; P < c_hi; P += span) {
    const int c0 = max(P, c_lo), c1 = min(P + span, c_hi);  // valid columns of this pass
    // running slots of this thread: RS consecutive entries
    uint32_t rkey[RS];
    uint32_t rmin = 0xFFFFFFFFu, rmax = 0;
    static_for<RS>([&](auto j) __attribute__((always_inline)) {
      const int p = tid * RS + j;
      const bool ok = p < run_n;
      rkey[j] = ok ? fkey(sm.run_val[cur][p]) : 0u;
      if (ok) { rmin = min(rmin, rkey[j]); rmax = max(rmax, rkey[j]); }
    });
    // once the list is full, a pass value must beat its smallest entry (which wins ties by id)
    uint32_t floor_key = 0;
    if (run_n == K) {
      block_minmax(sm, rmin, rmax, lane, wave);
      floor_key = rmin;
    }
    // pass columns of this thread: cb .. cb + VPT - 1
    const int cb = P + tid * VPT;
    uint32_t key[VPT];
    if (vec && cb >= c0 && cb + VPT <= c1) {
      static_for<VPT / 4>([&](auto q) __attribute__((always_inline)) {
        const float4 v = *(const float4 *)(vrow + cb + 4 * q);
        key[4 * q + 0] = fkey(v.x);
        key[4 * q + 1] = fkey(v.y);
        key[4 * q + 2] = fkey(v.z);
        key[4 * q + 3] = fkey(v.w);
      });
    } else {
      static_for<VPT>([&](auto j) __attribute__((always_inline)) {
        const int c = cb + j;
        key[j] = (c >= c0 && c < c1) ? fkey(vrow[c]) : 0u;
      });
    }
    static_for<VPT>([&](auto j) __attribute__((always_inline)) {
      uint32_t k = key[j];
      if (mrow) {
        const int c = cb + j;
        const int64_t mj = (int64_t)c + mshift;
        if (!(c >= c0 && c < c1 && mj < a.mask_w && mrow[mj])) k = 0;
      }
      key[j] = k > floor_key ? k : 0u;
    });

    uint32_t nloc = 0;
    static_for<RS>([&](auto j) __attribute__((always_inline)) { nloc += rkey[j] != 0; });
    static_for<VPT>([&](auto j) __attribute__((always_inline)) { nloc += key[j] != 0; });
    const int total = (int)block_sum(sm, nloc, lane, wave);

    uint32_t thk = 0;   // threshold key (0: take every candidate)
    int need_eq = 0;    // how many keys equal to thk to take, lowest ids first
    if (total > K) {
      uint32_t clo = 1, chi = 0xFFFFFFFFu;  // current candidate key interval
      int need = K, cnt = total;
      bool done = false;
      for (int level = 0; level < 4 && !done; ++level) {
        uint32_t lo = 0xFFFFFFFFu, hi = 0;
        auto mm = [&](uint32_t k) __attribute__((always_inline)) {
          if (k >= clo && k <= chi) { lo = min(lo, k); hi = max(hi, k); }
        };
        static_for<RS>([&](auto j) __attribute__((always_inline)) { mm(rkey[j]); });
        static_for<VPT>([&](auto j) __attribute__((always_inline)) { mm(key[j]); });
        block_minmax(sm, lo, hi, lane, wave);
        if (lo == hi) { thk = lo; done = true; break; }
        if (cnt <= CAP) {
          // rank the remaining candidates directly
          __syncthreads();
          if (tid == 0) sm.bcast[0] = 0;
          __syncthreads();
          auto put = [&](uint32_t k) __attribute__((always_inline)) {
            if (k >= lo && k <= hi) {
              const uint32_t slot = atomicAdd(&sm.bcast[0], 1u);
              if (slot < CAP) sm.cand[slot] = k;
            }
          };
          static_for<RS>([&](auto j) __attribute__((always_inline)) { put(rkey[j]); });
          static_for<VPT>([&](auto j) __attribute__((always_inline)) { put(key[j]); });
          __syncthreads();
          if (tid < cnt) {
            const uint32_t mine = sm.cand[tid];
            int gt = 0, ge = 0;
            for (int j = 0; j < cnt; ++j) {
              const uint32_t o = sm.cand[j];
              gt += o > mine;
              ge += o >= mine;
            }
            if (gt < need && need <= ge) sm.bcast[1] = mine;
          }
          __syncthreads();
          thk = sm.bcast[1];
          done = true;
          break;
        }
        int sh = 0;
        while (((hi - lo) >> sh) >= (uint32_t)NB) ++sh;
        __syncthreads();
        for (int i = tid; i < NB; i += NTH) sm.hist[i] = 0;
        __syncthreads();
        auto bin = [&](uint32_t k) __attribute__((always_inline)) {
          if (k >= lo && k <= hi) atomicAdd(&sm.hist[(k - lo) >> sh], 1u);
        };
        static_for<RS>([&](auto j) __attribute__((always_inline)) { bin(rkey[j]); });
        static_for<VPT>([&](auto j) __attribute__((always_inline)) { bin(key[j]); });
        __syncthreads();
        // bin b* with (count above b*) < need <= (count at or above b*); thread i owns bins 4i..4i+3
        {
          constexpr int BPT = NB / NTH;
          uint32_t h[BPT];
          uint32_t tot = 0;
#pragma unroll
          for (int i = 0; i < BPT; ++i) { h[i] = sm.hist[tid * BPT + i]; tot += h[i]; }
          uint32_t incl = tot;  // inclusive suffix within the wave (lanes >= this one)
          for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_down(incl, o);
            if (lane + o < 64) incl += y;
          }
          __syncthreads();
          if (lane == 0) sm.red[0][wave] = incl;  // wave total
          __syncthreads();
          uint32_t above = incl - tot;
          for (int w = wave + 1; w < NWV; ++w) above += sm.red[0][w];
#pragma unroll
          for (int i = BPT - 1; i >= 0; --i) {
            if (above < (uint32_t)need && (uint32_t)need <= above + h[i]) {
              sm.bcast[0] = tid * BPT + i;
              sm.bcast[1] = above;
              sm.bcast[2] = h[i];
            }
            above += h[i];
          }
        }
        __syncthreads();
        const uint32_t bstar = sm.bcast[0];
        need -= (int)sm.bcast[1];
        cnt = (int)sm.bcast[2];
        clo = lo + (bstar << sh);
        const uint64_t top = (uint64_t)lo + ((uint64_t)(bstar + 1) << sh) - 1;
        chi = (uint32_t)min<uint64_t>(top, (uint64_t)hi);
      }
      if (!done) thk = clo;  // unreachable: each level narrows the interval by >= 11 of 32 bits
      uint32_t gt = 0;
      static_for<RS>([&](auto j) __attribute__((always_inline)) { gt += rkey[j] > thk; });
      static_for<VPT>([&](auto j) __attribute__((always_inline)) { gt += key[j] > thk; });
      need_eq = K - (int)block_sum(sm, gt, lane, wave);
    }

    // ---- selection in id order: keys above thk, then the first need_eq keys equal to it.
    // Running slots (ids below every pass id) come first, each group in thread order.
    uint32_t eq_r = 0, eq_p = 0;
    if (need_eq > 0) {
      static_for<RS>([&](auto j) __attribute__((always_inline)) { eq_r += rkey[j] == thk; });
      static_for<VPT>([&](auto j) __attribute__((always_inline)) { eq_p += key[j] == thk; });
    }
    uint32_t eo_r, eo_p, et_r, et_p;
    block_scan2(sm, eq_r, eq_p, eo_r, eo_p, et_r, et_p, lane, wave);
    // equal keys are taken in id order: running ones first (ranks 0 .. et_r - 1), then the pass's
    const uint32_t eqrank_r = eo_r, eqrank_p = et_r + eo_p;
    auto taken = [&](uint32_t k, uint32_t &eqrank) __attribute__((always_inline)) -> bool {
      if (k == 0) return false;
      if (k > thk) return true;
      if (k == thk && need_eq > 0) return eqrank++ < (uint32_t)need_eq;
      return false;
    };
    uint32_t tk_r = 0, tk_p = 0;
    {
      uint32_t e1 = eqrank_r, e2 = eqrank_p;
      static_for<RS>([&](auto j) __attribute__((always_inline)) { tk_r += taken(rkey[j], e1); });
      static_for<VPT>([&](auto j) __attribute__((always_inline)) { tk_p += taken(key[j], e2); });
    }
    uint32_t po_r, po_p, pt_r, pt_p;
    block_scan2(sm, tk_r, tk_p, po_r, po_p, pt_r, pt_p, lane, wave);
    const int nxt = cur ^ 1;
    {
      uint32_t e1 = eqrank_r, e2 = eqrank_p;
      uint32_t pr = po_r, pp = pt_r + po_p;
      static_for<RS>([&](auto j) __attribute__((always_inline)) {
        if (taken(rkey[j], e1)) {
          if (pr < (uint32_t)KMAX) {
            sm.run_id[nxt][pr] = sm.run_id[cur][tid * RS + j];
            sm.run_val[nxt][pr] = kval(rkey[j]);
          }
          ++pr;
        }
      });
      static_for<VPT>([&](auto j) __attribute__((always_inline)) {
        if (taken(key[j], e2)) {
          if (pp < (uint32_t)KMAX) {
            sm.run_id[nxt][pp] = off + cb + j;
            sm.run_val[nxt][pp] = kval(key[j]);
          }
          ++pp;
        }
      });
    }
    run_n = min((int)(pt_r + pt_p), K);
    cur = nxt;
    __syncthreads();
  }

  // ---- write the running list
  __syncthreads();
  for (int p = tid; p < K; p += NTH) {
    const bool ok = p < run_n;
    oidx[p] = ok ? sm.run_id[cur][p] : -1;
    if (oval) oval[p] = ok ? sm.run_val[cur][p] : -__builtin_inff();
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
  if (a.nrows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.nrows), dim3(NTH), 0, s, a);
  return hipGetLastError();
}

}  // namespace idx
