// Exact per-row top-K with a running merge (P1 section 2.3: topk(union) ==
// topk(union of per-block topk), so a row's candidates can arrive block by
// block; P2 Modifications: the top-k of each chunk goes into one shared
// selected buffer).
//
// One workgroup (512 threads) owns one row.  The running top-K (ids ascending,
// fp32 values) lives in LDS while the row's columns are consumed in passes of
// up to 32768 values held in registers (64 per thread).  Each pass:
//   1. map fp32 values to order-preserving uint32 keys (0 is reserved for
//      "not a candidate": excluded by window, mask or padding);
//   2. find the key of the K-th largest candidate (running + pass), counting
//      multiplicity.  The candidate key interval [lo, hi] is narrowed by
//      histogram levels: bins are (key - lo) >> s with the smallest s that
//      gives < 2048 bins, so each level consumes >= 11 bits of the interval and
//      at most three levels are needed; once <= 512 candidates remain they are
//      ranked directly in LDS;
//   3. select keys above the threshold and, among keys equal to it, the ones
//      with the lowest ids (total order: value desc, id asc), writing them in
//      id order with ordered ballot scans.  Running ids precede the pass's ids,
//      so the merged list stays ascending.
// All steps are integer/comparison work on exact keys, so the result is the
// unique top-K under the total order, independent of how rows or columns are
// split into launches and passes.
#include "kernels.h"

namespace idx {
namespace {

constexpr int NTH = 512;
constexpr int NWV = NTH / 64;
constexpr int VPT = 64;           // pass values per thread
constexpr int RS = 4;             // running slots per thread (K <= 2048)
constexpr int KMAX = RS * NTH;
constexpr int NB = 2048;          // histogram bins
constexpr int CAP = 512;          // direct ranking threshold
constexpr int NSEG = (RS + VPT) * NWV;

__device__ __forceinline__ uint32_t fkey(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0;  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float kval(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

struct Smem {
  int run_id[2][KMAX];
  float run_val[2][KMAX];
  uint32_t hist[NB];
  uint32_t cand[CAP];
  int seg[NSEG + 1];
  uint32_t red[3][NWV];
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
__device__ uint32_t block_sum(Smem &sm, uint32_t x, int lane, int wave) {
  x = wave_sum(x);
  __syncthreads();
  if (lane == 0) sm.red[0][wave] = x;
  __syncthreads();
  uint32_t s = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) s += sm.red[0][w];
  return s;
}
__device__ void block_minmax(Smem &sm, uint32_t &lo, uint32_t &hi, int lane, int wave) {
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

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return lane ? (~0ull >> (64 - lane)) : 0ull; }

// Exclusive ordered scan of per-element flags.  Element order: running stripe
// j (slot j*NTH + tid), j < RS, then pass stripe j (column c0 + j*NTH + tid).
// flag(s) gives this thread's flag for stripe s; emit(s, pos) is called for
// flagged elements with their rank.  Returns the total count.
template <class Flag, class Emit>
__device__ int ordered_scan(Smem &sm, int lane, int wave, Flag flag, Emit emit) {
  __syncthreads();
#pragma unroll
  for (int s = 0; s < RS + VPT; ++s) {
    const uint64_t b = __ballot(flag(s));
    if (lane == 0) sm.seg[s * NWV + wave] = __popcll(b);
  }
  __syncthreads();
  if (wave == 0) {
    constexpr int PER = (NSEG + 63) / 64;
    int local[PER];
    int tot = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane * PER + i;
      local[i] = e < NSEG ? sm.seg[e] : 0;
      tot += local[i];
    }
    int incl = tot;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    int run = incl - tot;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane * PER + i;
      if (e < NSEG) sm.seg[e] = run;
      run += local[i];
    }
    if (lane == 63) sm.seg[NSEG] = incl;
  }
  __syncthreads();
  const uint64_t lt = lanemask_lt(lane);
#pragma unroll
  for (int s = 0; s < RS + VPT; ++s) {
    const bool f = flag(s);
    const uint64_t b = __ballot(f);
    if (f) emit(s, sm.seg[s * NWV + wave] + (int)__popcll(b & lt));
  }
  return sm.seg[NSEG];
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

  for (int c0 = c_lo; c0 < c_hi; c0 += a.block) {
    const int c1 = min(c0 + a.block, c_hi);
    uint32_t key[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int c = c0 + j * NTH + tid;
      uint32_t k = 0;
      if (c < c1) {
        const int64_t mj = (int64_t)c + mshift;
        const bool allowed = !mrow || (mj < a.mask_w && mrow[mj]);
        if (allowed) k = fkey(vrow[c]);
      }
      key[j] = k;
    }
    uint32_t rkey[RS];
    int rid[RS];
#pragma unroll
    for (int j = 0; j < RS; ++j) {
      const int p = j * NTH + tid;
      const bool ok = p < run_n;
      rkey[j] = ok ? fkey(sm.run_val[cur][p]) : 0u;
      rid[j] = ok ? sm.run_id[cur][p] : -1;
    }
    auto keyof = [&](int s) -> uint32_t { return s < RS ? rkey[s] : key[s - RS]; };

    uint32_t nloc = 0;
#pragma unroll
    for (int s = 0; s < RS + VPT; ++s) nloc += keyof(s) != 0;
    const int total = (int)block_sum(sm, nloc, lane, wave);

    uint32_t thk = 0;   // threshold key (0: take every candidate)
    int need_eq = 0;    // how many keys equal to thk to take, lowest ids first
    if (total > K) {
      uint32_t clo = 1, chi = 0xFFFFFFFFu;  // current candidate key interval
      int need = K, cnt = total;
      bool done = false;
      for (int level = 0; level < 4 && !done; ++level) {
        uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
        for (int s = 0; s < RS + VPT; ++s) {
          const uint32_t k = keyof(s);
          if (k >= clo && k <= chi) { lo = min(lo, k); hi = max(hi, k); }
        }
        block_minmax(sm, lo, hi, lane, wave);
        if (lo == hi) { thk = lo; done = true; break; }
        if (cnt <= CAP) {
          // rank the remaining candidates directly
          __syncthreads();
          if (tid == 0) sm.bcast[0] = 0;
          __syncthreads();
#pragma unroll
          for (int s = 0; s < RS + VPT; ++s) {
            const uint32_t k = keyof(s);
            if (k >= lo && k <= hi) {
              const uint32_t slot = atomicAdd(&sm.bcast[0], 1u);
              if (slot < CAP) sm.cand[slot] = k;
            }
          }
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
#pragma unroll
        for (int s = 0; s < RS + VPT; ++s) {
          const uint32_t k = keyof(s);
          if (k >= lo && k <= hi) atomicAdd(&sm.hist[(k - lo) >> sh], 1u);
        }
        __syncthreads();
        // bin b* with (count above b*) < need <= (count at or above b*); thread i owns bins 4i..4i+3
        {
          constexpr int BPT = NB / NTH;
          uint32_t h[BPT];
          uint32_t tot = 0;
#pragma unroll
          for (int i = 0; i < BPT; ++i) { h[i] = sm.hist[tid * BPT + i]; tot += h[i]; }
          // suffix sum over threads: exclusive sum of totals of higher threads
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
          // walk my bins from high to low
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
      if (!done) {
        // unreachable: each level narrows the interval by >= 11 bits of 32
        thk = clo;
      }
      uint32_t gt = 0;
#pragma unroll
      for (int s = 0; s < RS + VPT; ++s) gt += keyof(s) > thk;
      need_eq = K - (int)block_sum(sm, gt, lane, wave);
    }

    // ---- selection in id order: keys above thk, then the first need_eq keys equal to it
    uint64_t eqp = 0;   // pass stripes whose equal-to-threshold key is taken
    uint32_t eqr = 0;   // running stripes whose equal-to-threshold key is taken
    if (need_eq > 0) {
      ordered_scan(sm, lane, wave, [&](int s) { return keyof(s) == thk; },
                   [&](int s, int pos) {
                     if (pos < need_eq) {
                       if (s < RS) eqr |= 1u << s;
                       else eqp |= 1ull << (s - RS);
                     }
                   });
    }
    auto take = [&](int s) -> bool {
      const uint32_t k = keyof(s);
      if (k == 0) return false;
      if (k > thk) return true;
      if (k != thk || need_eq <= 0) return false;
      return s < RS ? ((eqr >> s) & 1u) : ((eqp >> (s - RS)) & 1ull);
    };
    const int nxt = cur ^ 1;
    run_n = ordered_scan(sm, lane, wave, take, [&](int s, int pos) {
      if (pos >= KMAX) return;
      if (s < RS) {
        sm.run_id[nxt][pos] = rid[s];
        sm.run_val[nxt][pos] = kval(rkey[s]);
      } else {
        sm.run_id[nxt][pos] = off + c0 + (s - RS) * NTH + tid;
        sm.run_val[nxt][pos] = kval(key[s - RS]);
      }
    });
    run_n = min(run_n, K);
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
