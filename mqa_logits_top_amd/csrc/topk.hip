// Exact per-row top-K with a running merge (P1 section 2.3: topk(union) ==
// topk(union of per-block topk), so a row's candidates can arrive block by
// block; P2 Modifications: the top-k of each chunk goes into one shared
// selected buffer).
//
// One workgroup (512 threads) owns one row.  The running top-K (ids ascending,
// fp32 values) lives in LDS; the row's columns are consumed in segments of up to
// 32768 columns, each merged into the running list.  A segment is read from
// memory once, into registers: thread `tid` holds columns 8192 c + 16 tid + j
// (c < 4, j < 16) as order-preserving uint32 keys (0 is reserved for "not a
// candidate": excluded by window, mask or -- once the running list is full -- by
// not beating its smallest entry, which wins every tie because running ids
// precede the segment's ids).  Register sweeps then
//   1. count the union of running and segment candidates and find its key range;
//   2. histogram the union into 2048 bins anchored at the largest key (the first
//      level covers 2^26 keys -- eight binades -- below it in bins of 2^15 keys,
//      plus a catch-all bin under them), find the bin b* holding the K-th
//      largest key, and narrow to that bin while the segment's candidates at or
//      above it would not fit the LDS list;
//   3. collect the segment's keys at or above the bin, in column order, into LDS.
// The exact K-th key and the number of keys equal to it that are taken (lowest
// ids first) are then found among the LDS-resident candidates of bin b*, and the
// taken running and segment entries are written, in id order, as the new list.
// All decisions are integer comparisons of exact keys, so the result is the
// unique top-K under (value desc, id asc), whatever the segment boundaries.
#include "common.h"
#include "kernels.h"

namespace idx {
namespace {

constexpr int NTH = 512;
constexpr int NWV = NTH / 64;
constexpr int VPT = 16;             // columns per thread per chunk (contiguous)
constexpr int SPAN = NTH * VPT;     // columns per chunk
constexpr int NCH = 4;              // chunks per segment
constexpr int SEG = NCH * SPAN;     // columns per segment (segment offsets fit 16 bits)
constexpr int KMAX = 2560;          // longest running list
constexpr int NB = 2048;            // histogram bins
constexpr int CAPK = 4608;          // segment candidates held in LDS
constexpr int CAP = 512;            // direct ranking threshold
constexpr int CAPS_MAX = 512;       // largest candidate slab the merge path gathers
constexpr int TOP_LOG2 = 26;        // level 0 resolves the 2^26 keys below the largest
constexpr int TOP_SH = TOP_LOG2 - 11;

constexpr int NI = KMAX + CAPK;     // items: the running list, then a segment's collected keys

struct Smem {
  // Items in id order: the running list [0, run_n), then the candidates collected
  // from a segment, then one spare slot per lane for writes that are dropped.  A merge
  // compacts them in place.
  alignas(16) uint32_t ikey[NI + 64];
  alignas(16) int32_t iid[NI + 64];
  // histogram bins (+ one spare slot per lane); the first CAP words double as the
  // ranking list
  alignas(16) uint32_t hist[NB + 64];
  uint32_t bmap[BMAP_BITS / 32];  // the row's allowed blocks over the launch's columns (block consumer)
  uint32_t red[3][NWV];
  uint32_t wsum[2][NWV];
  uint32_t bcast[4];
};

// Block-wide sum, min and max of one value per thread (all threads must call; S has red[3][waves]).
template <class S>
__device__ __forceinline__ void block_sum_minmax(S &sm, uint32_t &s, uint32_t &lo, uint32_t &hi, int lane,
                                                 int wave) {
  s = wave_sum(s);
  lo = wave_min(lo);
  hi = wave_max(hi);
  __syncthreads();
  if (lane == 0) { sm.red[0][wave] = s; sm.red[1][wave] = lo; sm.red[2][wave] = hi; }
  __syncthreads();
  s = 0;
  lo = 0xFFFFFFFFu;
  hi = 0;
#pragma unroll
  for (int w = 0; w < (int)(sizeof(sm.red[0]) / 4); ++w) {
    s += sm.red[0][w];
    lo = min(lo, sm.red[1][w]);
    hi = max(hi, sm.red[2][w]);
  }
}

// Two simultaneous block-wide exclusive scans in thread order, with their totals (S has wsum[2][waves]).
template <class S>
__device__ __forceinline__ void block_scan2(S &sm, uint32_t a, uint32_t b, uint32_t &ea, uint32_t &eb,
                                            uint32_t &ta, uint32_t &tb, int lane, int wave) {
  const uint32_t ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  __syncthreads();
  if (lane == 63) { sm.wsum[0][wave] = ia; sm.wsum[1][wave] = ib; }
  __syncthreads();
  uint32_t pa = 0, pb = 0;
  ta = 0;
  tb = 0;
#pragma unroll
  for (int w = 0; w < (int)(sizeof(sm.wsum[0]) / 4); ++w) {
    const uint32_t sa = sm.wsum[0][w], sb = sm.wsum[1][w];
    if (w < wave) { pa += sa; pb += sb; }
    ta += sa;
    tb += sb;
  }
  ea = pa + ia - a;
  eb = pb + ib - b;
}

// Bin of key k in a histogram anchored at chi: (chi - k) >> sh, the last bin
// catching everything further down.
__device__ __forceinline__ uint32_t bin_of(uint32_t k, uint32_t chi, int sh) {
  return min((chi - k) >> sh, (uint32_t)(NB - 1));
}

// The exact K-th key among the items ikey[0, N).  Entries in [clo, chi] number icnt;
// `need` picks remain inside that interval.  Gives thk and need_eq, the number of
// entries equal to thk that are taken.
__device__ __forceinline__ void lds_select(Smem &sm, int N, uint32_t clo, uint32_t chi, int need, uint32_t icnt,
                                           uint32_t &thk, int &need_eq, int tid, int lane, int wave) {
  auto item_key = [&](int i) __attribute__((always_inline)) -> uint32_t { return sm.ikey[i]; };
  for (;;) {
    if (clo == chi) { thk = clo; need_eq = need; break; }
    if (icnt <= (uint32_t)CAP) {
      // rank the interval's entries directly
      __syncthreads();
      if (tid == 0) sm.bcast[0] = 0;
      __syncthreads();
      for (int i = tid; i < N; i += NTH) {
        const uint32_t k = item_key(i);
        if (k >= clo && k <= chi) {
          const uint32_t slot = atomicAdd(&sm.bcast[0], 1u);
          if (slot < (uint32_t)CAP) sm.hist[slot] = k;
        }
      }
      __syncthreads();
      const int n = (int)min(sm.bcast[0], (uint32_t)CAP);
      // pad the list to whole 16-byte words with zero keys (below any key of the interval
      // but key 0, whose count is corrected)
      const int n4 = (n + 3) >> 2;
      if (tid < 4 * n4 - n) sm.hist[n + tid] = 0u;
      __syncthreads();
      if (tid < n) {
        const uint32_t mine = sm.hist[tid];
        int gt = 0, ge = mine == 0u ? n - 4 * n4 : 0;
        const uint4 *h4 = reinterpret_cast<const uint4 *>(sm.hist);
#pragma unroll 4
        for (int j = 0; j < n4; ++j) {
          const uint4 o = h4[j];
          gt += (o.x > mine) + (o.y > mine) + (o.z > mine) + (o.w > mine);
          ge += (o.x >= mine) + (o.y >= mine) + (o.z >= mine) + (o.w >= mine);
        }
        if (gt < need && need <= ge) { sm.bcast[1] = mine; sm.bcast[2] = (uint32_t)(need - gt); }
      }
      __syncthreads();
      thk = sm.bcast[1];
      need_eq = (int)sm.bcast[2];
      break;
    }
    const uint32_t span = chi - clo;
    int sh = 0;
    while ((span >> sh) >= (uint32_t)NB) ++sh;
    __syncthreads();
    for (int i = tid; i < NB; i += NTH) sm.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < N; i += NTH) {
      const uint32_t k = item_key(i);
      if (k >= clo && k <= chi) atomicAdd(&sm.hist[bin_of(k, chi, sh)], 1u);
    }
    __syncthreads();
    {
      constexpr int BPT = NB / NTH;
      uint32_t h[BPT], tot = 0;
#pragma unroll
      for (int i = 0; i < BPT; ++i) { h[i] = sm.hist[tid * BPT + i]; tot += h[i]; }
      uint32_t before, d0, t0, t1;
      block_scan2(sm, tot, 0u, before, d0, t0, t1, lane, wave);
#pragma unroll
      for (int i = 0; i < BPT; ++i) {
        if (before < (uint32_t)need && (uint32_t)need <= before + h[i]) {
          sm.bcast[0] = tid * BPT + i;
          sm.bcast[1] = before;
          sm.bcast[2] = h[i];
        }
        before += h[i];
      }
    }
    __syncthreads();
    const uint32_t bstar = sm.bcast[0];
    need -= (int)sm.bcast[1];
    icnt = sm.bcast[2];
    const uint32_t nhi = chi - (bstar << sh);
    clo = max(clo, nhi - min(nhi - clo, (1u << sh) - 1u));
    chi = nhi;
  }
}

// New running list: the taken items of ikey / iid [0, N) -- keys above thk, then
// need_eq keys equal to thk in item order -- compacted in place, in item (= id)
// order.  Items from run_n on carry ids relative to id0.  Thread tid reads items
// 16 tid .. 16 tid + 15 into registers; one scan of (equal, above) counts places them.
// Returns the new list length.
__device__ __forceinline__ int merge_items(Smem &sm, int N, int run_n, int id0, uint32_t thk, int need_eq, int K,
                                           int tid, int lane, int wave) {
  constexpr int IPT = 16;
  static_assert(IPT * NTH >= NI, "items per thread");
  const int i0 = tid * IPT;
  uint32_t kk[IPT];
  int kid[IPT];
  if (i0 < N) {  // i0 + IPT <= NI + 64
    static_for<IPT / 4>([&](auto q) __attribute__((always_inline)) {
      const uint4 k4 = *(const uint4 *)&sm.ikey[i0 + 4 * q];
      const int4 d4 = *(const int4 *)&sm.iid[i0 + 4 * q];
      kk[4 * q] = k4.x; kk[4 * q + 1] = k4.y; kk[4 * q + 2] = k4.z; kk[4 * q + 3] = k4.w;
      kid[4 * q] = d4.x; kid[4 * q + 1] = d4.y; kid[4 * q + 2] = d4.z; kid[4 * q + 3] = d4.w;
    });
  } else {
    static_for<IPT>([&](auto u) __attribute__((always_inline)) { kk[u] = 0u; kid[u] = -1; });
  }
  uint32_t m1 = 0, m2 = 0;  // items above thk / equal to it (taken by rank)
  static_for<IPT>([&](auto u) __attribute__((always_inline)) {
    const uint32_t k = i0 + u < N ? kk[u] : 0u;
    m1 |= (uint32_t)(k != 0u && k > thk) << u;
    m2 |= (uint32_t)(k != 0u && k == thk && need_eq > 0) << u;
  });
  // (the scan's barriers also order every read above before the writes below)
  uint32_t eo, ao, etot, atot;
  block_scan2(sm, __builtin_popcount(m2), __builtin_popcount(m1), eo, ao, etot, atot, lane, wave);
  const uint32_t ne = (uint32_t)need_eq;
  uint32_t e = eo, pos = ao + min(eo, ne);
  static_for<IPT>([&](auto u) __attribute__((always_inline)) {
    const bool tk = ((m1 >> u) & 1u) || (((m2 >> u) & 1u) && e < ne);
    e += (m2 >> u) & 1u;
    const int slot = tk && pos < (uint32_t)KMAX ? (int)pos : NI + lane;
    sm.ikey[slot] = kk[u];
    sm.iid[slot] = kid[u] + (i0 + u >= run_n ? id0 : 0);
    pos += tk;
  });
  __syncthreads();
  return min((int)(atot + min(etot, ne)), K);
}

template <bool BLOCKS>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(4, 4))) void topk_kernel(TopkArgs a) {
  __shared__ Smem sm;
  // newest rows first: the scoring launch before this one wrote them last, so they are the
  // ones still held in the memory-side cache
  const int r = a.nrows - 1 - (int)blockIdx.x;
  if (a.only_rows && a.only_rows[r] == 0u) return;   // uniform
  if (!a.first && a.launch_flag && (*a.launch_flag & 2u) != 0u) return;   // an empty launch (uniform)
  if (a.kshift) a.key0 += *a.kshift;                  // (as the scoring launch's key range)
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
    // column c holds the block whose first key lies in octet key0 / pool + c; the row's block b
    // starts in octet ks / pool + b (blocks start at ks)
    default: off = a.key0 / a.pool - ks / a.pool; id_lo = 0; id_hi = (ke - ks + a.pool - 1) / a.pool; break;
  }
  const int c_lo = max(id_lo - off, 0);
  const int c_hi = min(id_hi - off, a.ncols);
  const int c_rd = min(c_hi, a.vcols > 0 ? a.vcols : a.ncols);   // columns present in vals
  int32_t *oidx = a.out_idx + (int64_t)r * K;
  float *oval = a.out_val ? a.out_val + (int64_t)r * K : nullptr;
  if (!a.first && c_lo >= c_hi) return;  // nothing new for this row: running state stays as is

  // ---- running state
  int run_n = 0;
  if (!a.first) {
    uint32_t cnt = 0, d0 = 0, d1 = 0;
    constexpr int LPT = KMAX / NTH;  // entries per thread, all loads in flight at once
    int idv[LPT];
    float vv[LPT];
    static_for<LPT>([&](auto u) __attribute__((always_inline)) {
      const int p = tid + u * NTH;
      idv[u] = p < K ? oidx[p] : -1;
      vv[u] = p < K ? oval[p] : 0.f;
    });
    static_for<LPT>([&](auto u) __attribute__((always_inline)) {
      const int p = tid + u * NTH;
      if (p < K) {
        sm.iid[p] = idv[u];
        sm.ikey[p] = idv[u] >= 0 ? fkey(vv[u]) : 0u;
        cnt += idv[u] >= 0;
      }
    });
    block_sum_minmax(sm, cnt, d0, d1, lane, wave);
    run_n = (int)cnt;
  }

  const float *vrow = a.vals + (int64_t)r * a.ld;
  const uint8_t *mrow = a.mask ? a.mask + (int64_t)t * a.ld_mask : nullptr;
  const int mshift = (a.mode == TOPK_DENSE || a.mode == TOPK_BLOCK) ? off - ks : 0;  // mask byte = c + mshift
  // block consumer: bit b of bmap <=> row-relative block b_lo + b is allowed
  int b_lo = 0;
  if (BLOCKS) {
    const int j0 = max(c_lo + mshift, 0);
    b_lo = j0 >> a.bpool_sh;
    const int nb = c_hi > c_lo ? ((c_hi - 1 + mshift) >> a.bpool_sh) - b_lo + 1 : 0;
    for (int i = tid; i < BMAP_BITS / 32; i += NTH) sm.bmap[i] = 0;
    __syncthreads();
    const int32_t *brow = a.blocks + (int64_t)t * a.ld_blocks;
    for (int i = tid; i < a.n_blocks; i += NTH) {
      const int b = brow[i];
      if (b >= 0 && b - b_lo >= 0 && b - b_lo < min(nb, BMAP_BITS)) atomicOr(&sm.bmap[(b - b_lo) >> 5], 1u << ((b - b_lo) & 31));
    }
    __syncthreads();
  }
  auto block_ok = [&](int64_t j) __attribute__((always_inline)) -> bool {  // row-relative position j
    const int64_t b = (j >> a.bpool_sh) - b_lo;
    return b >= 0 && b < BMAP_BITS && ((sm.bmap[b >> 5] >> (b & 31)) & 1u);
  };
  // 16-byte loads when every row and every thread's first column are 16-byte aligned
  const bool vec = ((a.ld & 3) == 0) && (((uintptr_t)a.vals & 15) == 0);
  const int seg = max(min(a.block, SEG) & ~3, 4);
  const int sbase = vec ? (c_lo & ~3) : c_lo;

  uint32_t list_min = 0;  // smallest key of the list after the last merge (once it is full)

  if (a.col_rows && tid == 0) a.col_rows[r] = 1u;   // this row reads the launch's columns
  for (int S = sbase; S < c_rd; S += seg) {
    const int s0 = max(S, c_lo), s1 = min(S + seg, c_rd);  // valid columns of this segment

    auto run_key = [&](int p) __attribute__((always_inline)) -> uint32_t { return sm.ikey[p]; };
    uint32_t floor_key = 0;
    if (run_n == K) {  // a full list: segment keys must beat its smallest entry
      uint32_t rlo = 0xFFFFFFFFu, rhi = 0, rn = 0;
      for (int p = tid; p < run_n; p += NTH) rlo = min(rlo, run_key(p));
      block_sum_minmax(sm, rn, rlo, rhi, lane, wave);
      floor_key = rlo;
    }

    // ---- the segment's keys, in registers: key[c][j] is column S + 8192 c + 16 tid + j;
    // their count and range are taken as each chunk converts, while later chunks still load
    uint32_t key[NCH][VPT];
    uint32_t seg_n = 0, seg_lo = 0xFFFFFFFFu, seg_hi = 0;
    uint32_t live = 0;   // bit c: this thread's chunk c holds a nonzero key
    {
      float raw[NCH][VPT];
      static_for<NCH>([&](auto c) __attribute__((always_inline)) {
        const int cb = S + c * SPAN + tid * VPT;
        if (vec && cb >= s0 && cb + VPT <= s1) {
          static_for<VPT / 4>([&](auto q) __attribute__((always_inline)) {
            const float4 v = *(const float4 *)(vrow + cb + 4 * q);
            raw[c][4 * q + 0] = v.x;
            raw[c][4 * q + 1] = v.y;
            raw[c][4 * q + 2] = v.z;
            raw[c][4 * q + 3] = v.w;
          });
        } else if (cb >= s1 || cb + VPT <= s0) {
          static_for<VPT>([&](auto j) __attribute__((always_inline)) { raw[c][j] = 0.f; });   // outside the window
        } else {
          static_for<VPT>([&](auto j) __attribute__((always_inline)) {
            const int col = cb + j;
            raw[c][j] = (col >= s0 && col < s1) ? vrow[col] : 0.f;
          });
        }
      });
      uint32_t seg_lm1 = 0xFFFFFFFFu;   // smallest nonzero key minus 1 (a zero key wraps to the top)
      auto keep = [&](uint32_t &slot, uint32_t k) __attribute__((always_inline)) {
        k = k > floor_key ? k : 0u;
        slot = k;
        seg_n += k != 0u;
        seg_lm1 = min(seg_lm1, k - 1u);
        seg_hi = max(seg_hi, k);
      };
      static_for<NCH>([&](auto c) __attribute__((always_inline)) {
        const int cb = S + c * SPAN + tid * VPT;
        const uint32_t n0 = seg_n;
        if (cb >= s0 && cb + VPT <= s1 && !mrow && !BLOCKS) {
          // the whole chunk lies in the window and no consumer filter applies: no per-column tests
          static_for<VPT>([&](auto j) __attribute__((always_inline)) { keep(key[c][j], fkey(raw[c][j])); });
        } else if (cb >= s1 || cb + VPT <= s0) {
          // the whole chunk lies outside the window: no keys (short rows of ragged batches)
          static_for<VPT>([&](auto j) __attribute__((always_inline)) { key[c][j] = 0u; });
        } else {
          static_for<VPT>([&](auto j) __attribute__((always_inline)) {
            const int col = cb + j;
            const bool inside = col >= s0 && col < s1;
            uint32_t k = inside ? fkey(raw[c][j]) : 0u;
            if (mrow) {
              const int64_t mj = (int64_t)col + mshift;
              if (!(inside && mj < a.mask_w && mrow[mj])) k = 0;
            }
            if (BLOCKS && !(inside && block_ok((int64_t)col + mshift))) k = 0;
            keep(key[c][j], k);
          });
        }
        live |= (uint32_t)(seg_n != n0) << c;
      });
      seg_lo = seg_lm1 == 0xFFFFFFFFu ? 0xFFFFFFFFu : seg_lm1 + 1u;
    }

    // ---- size and key range of the union: the segment's part from the load, the running list's here
    uint32_t total = 0, umin = 0xFFFFFFFFu, umax = 0;
    {
      uint32_t n = seg_n;
      umin = seg_lo;
      umax = seg_hi;
      for (int p = tid; p < run_n; p += NTH) {
        const uint32_t k = run_key(p);
        ++n;
        umin = min(umin, k);
        umax = max(umax, k);
      }
      total = n;
      block_sum_minmax(sm, total, umin, umax, lane, wave);
    }

    // ---- passes 2..: the bin holding the K-th largest key
    uint32_t clo = umin, chi = umax;  // candidate interval
    int need = K;                     // picks still to make inside [clo, chi]
    uint32_t sel = 0;                 // union entries above the interval (all taken)
    uint32_t icnt = total;            // union entries inside the interval
    uint32_t theta = 1;               // collect segment keys >= theta
    uint32_t thk = 0;                 // final: keys > thk taken, then need_eq keys == thk by id
    int need_eq = 0;
    bool decided = false;             // thk / need_eq known before the LDS stage
    if ((int)total <= K) {
      decided = true;                 // everything is taken
    } else {
      for (int level = 0;; ++level) {
        if (clo == chi) { thk = clo; need_eq = need; decided = true; break; }
        // segment entries at or above clo: union entries there minus running ones
        uint32_t rge = (uint32_t)run_n;
        if (level > 0) {
          uint32_t d0 = 0, d1 = 0;
          rge = 0;
          for (int p = tid; p < run_n; p += NTH) rge += run_key(p) >= clo;
          block_sum_minmax(sm, rge, d0, d1, lane, wave);
        }
        if (sel + icnt - rge <= (uint32_t)CAPK) { theta = clo; break; }
        const uint32_t span = chi - clo;
        int sh = 0;
        if (level == 0 && (span >> TOP_LOG2) != 0) sh = TOP_SH;
        else while ((span >> sh) >= (uint32_t)NB) ++sh;
        __syncthreads();
        for (int i = tid; i < NB; i += NTH) sm.hist[i] = 0;
        __syncthreads();
        for (int p = tid; p < run_n; p += NTH) {
          const uint32_t k = run_key(p);
          if (k >= clo && k <= chi) atomicAdd(&sm.hist[bin_of(k, chi, sh)], 1u);
        }
        static_for<NCH>([&](auto c) __attribute__((always_inline)) {
          // chunks without keys are skipped (whole waves of them in short windows)
          if ((live >> c) & 1u) static_for<VPT>([&](auto j) __attribute__((always_inline)) {
            const uint32_t k = key[c][j];
            if (k >= clo && k <= chi) atomicAdd(&sm.hist[bin_of(k, chi, sh)], 1u);
          });
          __builtin_amdgcn_sched_barrier(0);  // one chunk at a time: bounded live ranges
        });
        __syncthreads();
        // b*: (entries in bins before b*) < need <= (entries in bins up to b*); thread i owns bins 4i..4i+3
        {
          constexpr int BPT = NB / NTH;
          uint32_t h[BPT], tot = 0;
#pragma unroll
          for (int i = 0; i < BPT; ++i) { h[i] = sm.hist[tid * BPT + i]; tot += h[i]; }
          uint32_t before, d0, t0, t1;
          block_scan2(sm, tot, 0u, before, d0, t0, t1, lane, wave);
#pragma unroll
          for (int i = 0; i < BPT; ++i) {
            if (before < (uint32_t)need && (uint32_t)need <= before + h[i]) {
              sm.bcast[0] = tid * BPT + i;
              sm.bcast[1] = before;
              sm.bcast[2] = h[i];
            }
            before += h[i];
          }
        }
        __syncthreads();
        const uint32_t bstar = sm.bcast[0];
        const uint32_t above = sm.bcast[1];
        icnt = sm.bcast[2];
        need -= (int)above;
        sel += above;
        const int64_t hi64 = (int64_t)chi - ((int64_t)bstar << sh);
        const int64_t lo64 = bstar == NB - 1 ? (int64_t)clo : (int64_t)chi - ((int64_t)(bstar + 1) << sh) + 1;
        clo = (uint32_t)max(lo64, (int64_t)clo);
        chi = (uint32_t)hi64;
      }
    }

    // ---- pass: collect the segment's keys at or above theta (or, with thk decided,
    // those that are taken), in column order.  Entries equal to thk are taken
    // running ones first, then the segment's in column order.
    uint32_t eq_run = 0;  // running entries equal to thk (taken first among equals)
    if (decided && need_eq > 0) {
      uint32_t e = 0, d0 = 0, d1 = 0;
      for (int p = tid; p < run_n; p += NTH) e += run_key(p) == thk;
      block_sum_minmax(sm, e, d0, d1, lane, wave);
      eq_run = e;
    }
    const uint32_t eq_budget = need_eq > (int)eq_run ? (uint32_t)need_eq - eq_run : 0u;
    const bool ties = decided && eq_budget > 0;   // block-uniform
    auto kind_of = [&](uint32_t k) __attribute__((always_inline)) -> int {  // 1: taken, 2: equal to thk
      if (!decided) return k >= theta ? 1 : 0;
      if (k > thk) return 1;
      return (k == thk && k != 0) ? 2 : 0;
    };
    // Ordered compaction in column order (chunk, thread, j): per-chunk counts of
    // each thread, packed two 16-bit fields to a word, go through one block scan.
    auto scan4 = [&](const uint32_t (&cnt)[NCH], uint32_t (&base)[NCH]) __attribute__((always_inline)) -> uint32_t {
      uint32_t e0, e1, t0, t1;
      block_scan2(sm, cnt[0] | (cnt[1] << 16), cnt[2] | (cnt[3] << 16), e0, e1, t0, t1, lane, wave);
      const uint32_t tot[NCH] = {t0 & 0xFFFFu, t0 >> 16, t1 & 0xFFFFu, t1 >> 16};
      const uint32_t ex[NCH] = {e0 & 0xFFFFu, e0 >> 16, e1 & 0xFFFFu, e1 >> 16};
      uint32_t acc = 0;
      static_for<NCH>([&](auto c) __attribute__((always_inline)) {
        base[c] = acc + ex[c];
        acc += tot[c];
      });
      return acc;
    };
    uint32_t eqb[NCH] = {0u, 0u, 0u, 0u};   // equal keys before this thread's chunk-c entries
    if (ties) {
      uint32_t ne[NCH];
      static_for<NCH>([&](auto c) __attribute__((always_inline)) {
        ne[c] = 0;
        static_for<VPT>([&](auto j) __attribute__((always_inline)) { ne[c] += kind_of(key[c][j]) == 2; });
      });
      scan4(ne, eqb);
    }
    // taken entries of chunk c as a 16-bit mask (bit j: column 8192 c + 16 tid + j)
    uint32_t tb[NCH], nt[NCH], posb[NCH];
    if (!ties) {
      // keys >= X: theta while the K-th key is still open, thk + 1 once it is known
      const bool none = decided && thk == 0xFFFFFFFFu;
      const uint32_t X = decided ? thk + 1u : theta;
      static_for<NCH>([&](auto c) __attribute__((always_inline)) {
        tb[c] = 0;
        if ((live >> c) & 1u) static_for<VPT>([&](auto j) __attribute__((always_inline)) {
          tb[c] |= (uint32_t)(key[c][j] >= X && !none) << j;
        });
        nt[c] = __builtin_popcount(tb[c]);
      });
    } else {
      static_for<NCH>([&](auto c) __attribute__((always_inline)) {
        uint32_t e = eqb[c];
        tb[c] = 0;
        static_for<VPT>([&](auto j) __attribute__((always_inline)) {
          const int kd = kind_of(key[c][j]);
          const bool tk = kd == 1 || (kd == 2 && e++ < eq_budget);
          tb[c] |= (uint32_t)tk << j;
        });
        nt[c] = __builtin_popcount(tb[c]);
      });
    }
    const int M_all = (int)scan4(nt, posb);
    // every entry is written: taken ones to their slot, the rest to this lane's spare slot
    static_for<NCH>([&](auto c) __attribute__((always_inline)) {
      uint32_t pos = posb[c];
      if (tb[c] != 0u) static_for<VPT>([&](auto j) __attribute__((always_inline)) {
        const bool tk = (tb[c] >> j) & 1u;
        if (tk && pos < (uint32_t)CAPK) {
          sm.ikey[run_n + pos] = key[c][j];
          sm.iid[run_n + pos] = c * SPAN + tid * VPT + j;   // made absolute by the merge
        }
        pos += tk;
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    int M = M_all;
    M = min(M, CAPK);
    __syncthreads();

    // ---- exact K-th key among the LDS-resident entries of [clo, chi]
    const int N = run_n + M;
    if (!decided) {
      lds_select(sm, N, clo, chi, need, icnt, thk, need_eq, tid, lane, wave);
    } else if ((int)total <= K) {
      thk = 0;       // take every entry
      need_eq = 0;
    }

    // ---- new running list: taken entries of (running ++ collected), id order
    run_n = merge_items(sm, N, run_n, off + S, thk, need_eq, K, tid, lane, wave);
    list_min = (int)total > K ? thk : umin;
  }

  // ---- write the running list (and, for a following scoring launch, its threshold)
  __syncthreads();
  for (int p = tid; p < K; p += NTH) {
    const bool ok = p < run_n;
    oidx[p] = ok ? sm.iid[p] : -1;
    if (oval) oval[p] = ok ? kval(sm.ikey[p]) : -__builtin_inff();
  }
  // a full list's smallest entry is the K-th key of the last merge (or, when that merge
  // took its whole union, the union's smallest key)
  if (a.thr_out && tid == 0) a.thr_out[r] = run_n == K ? kval(list_min) : __builtin_nanf("");
}

// ---- Slab merge (P1 section 2.3: the top-K of a union is the top-K of the union of its parts'
// top-Ks).  After a candidate-slab scoring launch, a row's new running list is the top Kc of
// its running list and the candidates its slabs hold (every one above the list's smallest
// entry), under (value desc, id asc), in id order.  One workgroup per row keeps the items in
// registers: thread t holds items MIPT t .. MIPT t + MIPT - 1 of the running list followed by
// the slab shares, which is id order (the list holds keys of earlier launches, and the shares
// hold consecutive key ranges, each in key order).  A histogram select over the register keys
// finds the Kc-th key; a block scan then writes the taken items to the list in item order.  The
// LDS holds only the histogram and the share table, so several rows share a CU.
// Rows of a row block flagged by the slab check (scored again into the scratch) and rows that
// do not meet the merge's conditions get col_rows = 1 and are left to topk_kernel.
constexpr int MNT = 512;               // threads
constexpr int MNW = MNT / 64;
constexpr int MIPT = 16;               // items per thread
constexpr int CPT = NTH / MNT;         // count words per thread (a launch has at most NTH shares)
static_assert(MNT * MIPT >= KMAX + CAPK && NB % MNT == 0 && NTH % MNT == 0, "merge layout");

struct MergeSmem {
  uint32_t hist[NB + 64];              // histogram bins; the first CAP words double as the ranking list
  uint32_t soff[NTH];                  // share e: first item (after the running list)
  uint32_t sbeg[NTH];                  // share e: slab entry of its first candidate
  uint32_t red[3][MNW];
  uint32_t wsum[2][MNW];
  uint32_t bcast[4];
};

// (6 waves per SIMD: three rows per CU; 256 threads with 32 items each measured slower)
__global__ __launch_bounds__(MNT) __attribute__((amdgpu_waves_per_eu(6))) void merge_kernel(TopkArgs a) {
  __shared__ MergeSmem sm;
  const int r = a.nrows - 1 - (int)blockIdx.x;        // newest rows first (as topk_kernel)
  if (a.launch_flag && (*a.launch_flag & 2u) != 0u) return;   // an empty launch: no slab was written
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.K;
  int32_t *oidx = a.out_idx + (int64_t)r * K;
  float *oval = a.out_val + (int64_t)r * K;
  auto leave = [&](uint32_t cols) __attribute__((always_inline)) {
    if (tid == 0) a.col_rows[r] = cols;
  };
  if (a.slab_flags[r / a.slab_rpw] != 0u) { leave(1u); return; }   // uniform

  // ---- share table: count words CPT t .. CPT t + CPT - 1 -> item offsets
  const int ne = a.nslab * CAND_PARTS;
  uint32_t cw[CPT], cs[CPT], my_c = 0, my_o = 0;
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int e = CPT * tid + q;
    cw[q] = e < ne ? a.ccnt[(int64_t)r * ne + e] : 0u;
    cs[q] = cw[q] & 0xFFFFu;
    if (cs[q] == CAND_OVER) { cs[q] = 0; ++my_o; }
    my_c += cs[q];
  }
  uint32_t ex, d1, tot_c, osum;
  block_scan2(sm, my_c, my_o, ex, d1, tot_c, osum, lane, wave);
  if (osum != 0 || tot_c > (uint32_t)CAPK || a.caps > CAPS_MAX || ne > NTH || K > KMAX) { leave(1u); return; }
  if (tot_c == 0) { leave(0u); return; }   // nothing above the list: list and threshold stay
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int e = CPT * tid + q;
    if (e < ne) { sm.soff[e] = ex; sm.sbeg[e] = cw[q] >> 16; }
    ex += cs[q];
  }
  __syncthreads();

  // ---- items into registers: one round of loads (running list entries, slab candidates).
  // The new list overwrites the old one in place: every load is consumed before the block
  // reduction below, and the writes come after two more block barriers.
  const int N = K + (int)tot_c;
  const int i0 = tid * MIPT;
  uint32_t key[MIPT];
  int32_t id[MIPT];
  {
    // the share of this thread's first candidate: the last e with soff[e] <= j
    int e = 0;
    const int j0 = max(i0 - K, 0);
    if (i0 + MIPT > K && i0 < N) {
      int lo = 0, hi = ne - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int)sm.soff[mid] <= j0) lo = mid;
        else hi = mid - 1;
      }
      e = lo;
    }
    // value bits into key[], ids into id[]; then the values become order-preserving keys
    const uint2 *slabs = (const uint2 *)a.cand + (int64_t)r * a.cand_ld;
    static_for<MIPT>([&](auto u) __attribute__((always_inline)) {
      const int i = i0 + u;
      id[u] = -1;
      key[u] = 0u;
      if (i < K) {
        id[u] = oidx[i];
        key[u] = __float_as_uint(oval[i]);
      } else if (i < N) {
        const int j = i - K;
        while (e + 1 < ne && (int)sm.soff[e + 1] <= j) ++e;
        const uint2 c = slabs[(e / CAND_PARTS) * a.caps + sm.sbeg[e] + (j - (int)sm.soff[e])];
        key[u] = c.x;
        id[u] = (int32_t)c.y;
      }
    });
    static_for<MIPT>([&](auto u) __attribute__((always_inline)) {
      key[u] = i0 + (int)u < N && id[u] >= 0 ? fkey(__uint_as_float(key[u])) : 0u;
    });
  }
  // size (nonzero keys, low half) and full running list entries (high half), key range
  uint32_t cnt = 0, umin = 0xFFFFFFFFu, umax = 0;
  static_for<MIPT>([&](auto u) __attribute__((always_inline)) {
    const uint32_t k = key[u];
    cnt += (k != 0u) + ((uint32_t)(i0 + (int)u < K && id[u] >= 0) << 16);
    umin = min(umin, k != 0u ? k : 0xFFFFFFFFu);
    umax = max(umax, k);
  });
  block_sum_minmax(sm, cnt, umin, umax, lane, wave);
  const uint32_t total = cnt & 0xFFFFu;
  if ((int)(cnt >> 16) != K) { leave(1u); return; }   // (not reached: a row with a partial list has
                                                      // a NaN threshold, which the slab check flags)

  // ---- the K-th largest key thk and the number need_eq of keys equal to it that are taken
  uint32_t thk = 0;
  int need_eq = 0;
  if ((int)total > K) {
    uint32_t clo = umin, chi = umax, icnt = total;
    int need = K;
    for (;;) {
      if (clo == chi) { thk = clo; need_eq = need; break; }
      if (icnt <= (uint32_t)CAP) {
        // rank the interval's keys directly
        __syncthreads();
        if (tid == 0) sm.bcast[0] = 0;
        __syncthreads();
        static_for<MIPT>([&](auto u) __attribute__((always_inline)) {
          const uint32_t k = key[u];
          if (k >= clo && k <= chi) {
            const uint32_t slot = atomicAdd(&sm.bcast[0], 1u);
            if (slot < (uint32_t)CAP) sm.hist[slot] = k;
          }
        });
        __syncthreads();
        const int n = (int)min(sm.bcast[0], (uint32_t)CAP);
        const int n4 = (n + 3) >> 2;
        if (tid < 4 * n4 - n) sm.hist[n + tid] = 0u;   // pad with key 0, below the interval
        __syncthreads();
        const uint4 *h4 = reinterpret_cast<const uint4 *>(sm.hist);
        for (int q = tid; q < n; q += MNT) {
          const uint32_t mine = sm.hist[q];
          int gt = 0, ge = 0;
#pragma unroll 4
          for (int j = 0; j < n4; ++j) {
            const uint4 o = h4[j];
            gt += (o.x > mine) + (o.y > mine) + (o.z > mine) + (o.w > mine);
            ge += (o.x >= mine) + (o.y >= mine) + (o.z >= mine) + (o.w >= mine);
          }
          if (gt < need && need <= ge) { sm.bcast[1] = mine; sm.bcast[2] = (uint32_t)(need - gt); }
        }
        __syncthreads();
        thk = sm.bcast[1];
        need_eq = (int)sm.bcast[2];
        break;
      }
      const uint32_t span = chi - clo;
      int sh = 0;
      while ((span >> sh) >= (uint32_t)NB) ++sh;
      __syncthreads();
      for (int i = tid; i < NB; i += MNT) sm.hist[i] = 0;
      __syncthreads();
      static_for<MIPT>([&](auto u) __attribute__((always_inline)) {
        const uint32_t k = key[u];
        if (k >= clo && k <= chi) atomicAdd(&sm.hist[bin_of(k, chi, sh)], 1u);
      });
      __syncthreads();
      {
        constexpr int BPT = NB / MNT;
        uint32_t h[BPT], tot = 0;
#pragma unroll
        for (int i = 0; i < BPT; ++i) { h[i] = sm.hist[tid * BPT + i]; tot += h[i]; }
        uint32_t before, d0, t0, t1;
        block_scan2(sm, tot, 0u, before, d0, t0, t1, lane, wave);
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
          if (before < (uint32_t)need && (uint32_t)need <= before + h[i]) {
            sm.bcast[0] = tid * BPT + i;
            sm.bcast[1] = before;
            sm.bcast[2] = h[i];
          }
          before += h[i];
        }
      }
      __syncthreads();
      const uint32_t bstar = sm.bcast[0];
      need -= (int)sm.bcast[1];
      icnt = sm.bcast[2];
      const uint32_t nhi = chi - (bstar << sh);
      clo = max(clo, nhi - min(nhi - clo, (1u << sh) - 1u));
      chi = nhi;
    }
  }

  // ---- the new list: keys above thk, then need_eq keys equal to it in item order
  uint32_t n1 = 0, n2 = 0;
  static_for<MIPT>([&](auto u) __attribute__((always_inline)) {
    const uint32_t k = key[u];
    n1 += k != 0u && k > thk;
    n2 += k != 0u && k == thk && need_eq > 0;
  });
  uint32_t eo, ao, etot, atot;
  block_scan2(sm, n2, n1, eo, ao, etot, atot, lane, wave);
  const uint32_t neq = (uint32_t)need_eq;
  uint32_t e = eo, pos = ao + min(eo, neq);
  static_for<MIPT>([&](auto u) __attribute__((always_inline)) {
    const uint32_t k = key[u];
    const bool eq = k != 0u && k == thk && need_eq > 0;
    const bool tk = (k != 0u && k > thk) || (eq && e < neq);
    e += eq;
    if (tk && pos < (uint32_t)K) {
      oidx[pos] = id[u];
      oval[pos] = kval(k);
    }
    pos += tk;
  });
  const uint32_t taken = atot + min(etot, neq);
  // (taken == K when total > K; otherwise every item is taken and the list is the union)
  if ((int)taken < K)
    for (int p = (int)taken + tid; p < K; p += MNT) {
      oidx[p] = -1;
      oval[p] = -__builtin_inff();
    }
  if (tid == 0) {
    a.col_rows[r] = 0u;
    if (a.thr_out) a.thr_out[r] = (int)taken == K ? kval((int)total > K ? thk : umin) : __builtin_nanf("");
  }
}

// One wave per row block: does any of its rows need the block's scores?  The conditions
// are those under which merge_kernel leaves a row to topk_kernel's column pass.
// Lanes take the row's count words (nshares <= NTH); the wave sums them.
__global__ __launch_bounds__(64) void slab_check_kernel(const uint32_t *ccnt, int32_t nshares, const float *thr,
                                                        int32_t nrows, int32_t rpw, uint32_t *flags,
                                                        const uint32_t *launch_flag) {
  const int b = blockIdx.x, lane = threadIdx.x;
  if (launch_flag && (*launch_flag & 2u) != 0u) {   // the launch scored nothing: no row needs the scores
    if (lane == 0) flags[b] = 0u;
    return;
  }
  bool need = nshares > NTH;
  for (int r = b * rpw; r < min((b + 1) * rpw, nrows); ++r) {
    uint32_t tot = 0, over = 0;
    for (int e = lane; e < nshares; e += 64) {
      const uint32_t c = ccnt[(int64_t)r * nshares + e] & 0xFFFFu;
      over |= c == CAND_OVER;
      tot += c == CAND_OVER ? 0u : c;
    }
    tot = wave_sum(tot);
    over = wave_max(over);
    need |= over != 0u || tot > (uint32_t)CAPK || !(thr[r] == thr[r]);   // NaN: the row's list is not full
  }
  if (lane == 0) flags[b] = need ? 1u : 0u;
}

}  // namespace

hipError_t launch_slab_check(const uint32_t *ccnt, int32_t nshares, const float *thr, int32_t nrows, int32_t rpw,
                             uint32_t *flags, const uint32_t *launch_flag, hipStream_t s) {
  const int nb = (nrows + rpw - 1) / rpw;
  if (nb <= 0) return hipSuccess;
  hipLaunchKernelGGL(slab_check_kernel, dim3(nb), dim3(64), 0, s, ccnt, nshares, thr, nrows, rpw, flags,
                     launch_flag);
  return hipGetLastError();
}

hipError_t launch_merge(const TopkArgs &a, hipStream_t s) {
  if (a.nrows <= 0) return hipSuccess;
  if (!a.cand || !a.ccnt || !a.slab_flags || !a.col_rows || !a.out_val || a.mask || a.blocks) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)a.nrows), dim3(MNT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
  if (a.nrows <= 0) return hipSuccess;
  if (a.cand) return hipErrorInvalidValue;   // slab merges go to launch_merge
  if (a.blocks)
    hipLaunchKernelGGL(topk_kernel<true>, dim3((unsigned)a.nrows), dim3(NTH), 0, s, a);
  else
    hipLaunchKernelGGL(topk_kernel<false>, dim3((unsigned)a.nrows), dim3(NTH), 0, s, a);
  return hipGetLastError();
}

}  // namespace idx
